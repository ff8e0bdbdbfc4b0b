// Speculative decoding's accept / resample step for gfx950.
//
// Blog #54, interview question 3, and Part 8, "Thuật Toán Chấp Nhận & Từ
// Chối Phỏng Đoán": drafted token x_k is kept with probability
// min(1, p_k(x_k) / q_k(x_k)); at the first rejection the later drafts are
// dropped and a token is drawn from max(0, p_k - q_k) renormalised; when all
// K drafts are kept the target's pass also gives one more token, drawn from
// p_{K+1} (Blog #54, section 2.4 example).
//
// Decisions are taken exactly as stated in the header: float32 acceptance
// test u * q < p, and an inverse-CDF draw over integer weights
// floor(w * 2^32) whose sums are exact, so the token drawn does not depend on
// the order in which the kernel adds them.
//
// Each sequence's row is cut into chunks, one workgroup each, so that the
// whole batch's rows stream through the chip at once; the last chunk of a
// sequence to finish picks the chunk holding the target and scans it (16
// bytes per thread per load throughout).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "pa_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = kThreads;  // chunks per sequence (one summing thread each)
constexpr int kMaxBatchK = 8;         // acceptance tests whose loads are issued together
constexpr int kWaves = kThreads / 64;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// floor(w * 2^32) for a float32 weight in [0, 1]: the scaling by a power of
// two is exact and the conversion truncates.
__device__ __forceinline__ uint64_t fixed_weight(float w) {
  return static_cast<uint64_t>(w * 4294967296.0f);
}

// The weight of token x: the residual max(0, p - q) (p - q rounded once), or
// p itself.
__device__ __forceinline__ float weight(const float* p, const float* q, int64_t x) {
  return q ? fmaxf(p[x] - q[x], 0.f) : p[x];
}

// Sum over the workgroup (every thread receives it).
__device__ uint64_t block_sum(uint64_t v, uint64_t* red) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint64_t s = 0;
  for (int w = 0; w < kWaves; ++w) s += red[w];
  return s;
}

// Exclusive prefix over the workgroup in thread order; *total gets the sum.
__device__ uint64_t block_exclusive(uint64_t v, uint64_t* red, uint64_t* total) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  uint64_t incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  uint64_t before = 0, all = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) before += red[w];
    all += red[w];
  }
  *total = all;
  return before + incl - v;
}

// Total fixed-point weights of a row: the draw's (the residual when q is
// given, else p) into *sw and p's own into *sp, in one pass.
template <bool VEC>
__device__ void row_totals(const float* p, const float* q, int64_t V, uint64_t* red, uint64_t* sw,
                           uint64_t* sp) {
  uint64_t s = 0, t = 0;
  if constexpr (VEC) {
    const int64_t n4 = V / 4;
    constexpr int U = 8;  // 16-byte loads in flight per row and thread
    for (int64_t i0 = threadIdx.x; i0 < n4; i0 += int64_t(kThreads) * U) {
      f32x4 a[U], b[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int64_t i = i0 + int64_t(k) * kThreads;
        a[k] = i < n4 ? reinterpret_cast<const f32x4*>(p)[i] : (f32x4){0.f, 0.f, 0.f, 0.f};
        if (q) b[k] = i < n4 ? reinterpret_cast<const f32x4*>(q)[i] : (f32x4){0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int k = 0; k < U; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          t += fixed_weight(a[k][e]);
          if (q) s += fixed_weight(fmaxf(a[k][e] - b[k][e], 0.f));
        }
    }
  } else {
    for (int64_t x = threadIdx.x; x < V; x += kThreads) {
      t += fixed_weight(p[x]);
      if (q) s += fixed_weight(fmaxf(p[x] - q[x], 0.f));
    }
  }
  *sp = block_sum(t, red);
  *sw = q ? block_sum(s, red) : *sp;
}

// Smallest x whose running fixed-point weight exceeds T (T < the row total).
// A row of at most kFindSeg tokens per thread is scanned in one go: each
// thread loads its own run of consecutive tokens, one block scan orders the
// runs, and the thread whose run holds the target walks it. Longer rows go
// tile by tile.
constexpr int kFindSeg = 32;

template <bool VEC>
__device__ int32_t row_find_small(const float* p, const float* q, int64_t V, uint64_t T, uint64_t* red,
                                  int32_t* found) {
  constexpr int N4 = kFindSeg / 4;
  if (threadIdx.x == 0) *found = -1;
  const int64_t seg = ((V + kThreads - 1) / kThreads + 3) / 4 * 4;  // tokens per thread, <= kFindSeg
  const int64_t x0 = int64_t(threadIdx.x) * seg;
  f32x4 f[N4];
#pragma unroll
  for (int i = 0; i < N4; ++i) {
    const int64_t x = x0 + 4 * i;
    if (4 * i >= seg) {
      f[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    } else if (VEC && x + 4 <= V) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p + x);
      f[i] = a;
      if (q) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(q + x);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[i][e] = fmaxf(a[e] - b[e], 0.f);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[i][e] = x + e < V ? weight(p, q, x + e) : 0.f;
    }
  }
  uint64_t mine = 0;
#pragma unroll
  for (int i = 0; i < N4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) mine += fixed_weight(f[i][e]);
  uint64_t total = 0;
  const uint64_t before = block_exclusive(mine, red, &total);
  if (before <= T && T < before + mine) {  // exactly one thread holds the target
    uint64_t acc = before;
    int hit = -1;
#pragma unroll
    for (int i = 0; i < N4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += fixed_weight(f[i][e]);
        if (hit < 0 && acc > T) hit = 4 * i + e;
      }
    *found = int32_t(x0 + hit);
  }
  __syncthreads();
  return *found;
}

template <bool VEC>
__device__ int32_t row_find(const float* p, const float* q, int64_t V, uint64_t T, uint64_t* red,
                            int32_t* found) {
  if (V <= int64_t(kFindSeg) * kThreads) return row_find_small<VEC>(p, q, V, T, red, found);
  constexpr int PER = 4;  // consecutive tokens per thread in a tile
  uint64_t run = 0;       // weight of the tiles before this one
  if (threadIdx.x == 0) *found = -1;
  for (int64_t t0 = 0; t0 < V; t0 += int64_t(kThreads) * PER) {
    const int64_t x0 = t0 + int64_t(threadIdx.x) * PER;
    uint64_t w[PER];
    if (VEC && x0 + PER <= V) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p + x0);
      f32x4 f = a;
      if (q) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(q + x0);
#pragma unroll
        for (int e = 0; e < PER; ++e) f[e] = fmaxf(a[e] - b[e], 0.f);
      }
#pragma unroll
      for (int e = 0; e < PER; ++e) w[e] = fixed_weight(f[e]);
    } else {
#pragma unroll
      for (int e = 0; e < PER; ++e) w[e] = x0 + e < V ? fixed_weight(weight(p, q, x0 + e)) : 0;
    }
    const uint64_t mine = w[0] + w[1] + w[2] + w[3];
    uint64_t tile = 0;
    const uint64_t before = run + block_exclusive(mine, red, &tile);
    if (before <= T && T < before + mine) {  // exactly one thread holds the target
      uint64_t acc = before;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        acc += w[e];
        if (acc > T) {
          *found = int32_t(x0 + e);
          break;
        }
      }
    }
    run += tile;
    if (run > T) break;  // uniform: every thread has the same run
  }
  __syncthreads();
  return *found;
}

struct SpecArgs {
  const float* p;
  const float* q;
  const int32_t* draft;
  const float* u_accept;
  const uint32_t* u_draw;
  uint64_t* sums;      // [B][C][2]: the chunk's draw weight, and its p weight
  int32_t* counters;   // [B] arrival count, zero between calls
  int32_t* num_accepted;
  int32_t* tokens;
  int32_t K, C;
  int64_t V, chunk;    // chunk: tokens per chunk, a multiple of 4
};

// Workgroup (b, c) holds chunk c of sequence b's row. Every chunk workgroup
// takes the acceptance decisions (a few scalar reads), sums its chunk's
// fixed-point weights (the draw's, and p's for the fallback), publishes them
// at the device-coherent level and counts itself in; the workgroup that
// completes the count adds the C sums, finds the chunk holding the target and
// scans only that chunk.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void spec_accept_kernel(SpecArgs a) {
  __shared__ uint64_t red[kWaves];
  __shared__ int32_t found;
  __shared__ int arrived;
  __shared__ int64_t pick_chunk;
  __shared__ uint64_t pick_target;
  __shared__ int pick_use_p;
  const int b = blockIdx.x / a.C, c = blockIdx.x % a.C;
  const int K = a.K;
  const int64_t V = a.V;
  const float* pb = a.p + int64_t(b) * (K + 1) * V;
  const float* qb = a.q ? a.q + int64_t(b) * K * V : nullptr;
  // acceptance tests (every thread takes the same decisions): the drafts'
  // probabilities are loaded together, kMaxBatchK at a time, then decided
  int n = 0;
  bool valid = true, stop = false;
  for (int k0 = 0; k0 < K && !stop; k0 += kMaxBatchK) {
    const int kn = min(kMaxBatchK, K - k0);
    int32_t x[kMaxBatchK];
    float px[kMaxBatchK], qx[kMaxBatchK], u[kMaxBatchK];
#pragma unroll
    for (int i = 0; i < kMaxBatchK; ++i)
      if (i < kn) x[i] = a.draft[int64_t(b) * K + k0 + i];
#pragma unroll
    for (int i = 0; i < kMaxBatchK; ++i) {
      if (i < kn) {
        const int64_t xi = min<int64_t>(max(x[i], 0), V - 1);  // checked below
        px[i] = pb[int64_t(k0 + i) * V + xi];
        qx[i] = qb[int64_t(k0 + i) * V + xi];
        u[i] = a.u_accept[int64_t(b) * K + k0 + i];
      }
    }
    for (int i = 0; i < kn; ++i, ++n) {
      if (x[i] < 0 || x[i] >= V) {
        valid = false;
        stop = true;
        break;
      }
      if (!(px[i] >= qx[i] || u[i] * qx[i] < px[i])) {
        stop = true;
        break;
      }
    }
  }
  int32_t* out = a.tokens + int64_t(b) * (K + 1);
  if (!valid) {  // no chunk counts itself in: the counter stays zero
    if (c == 0) {
      for (int e = threadIdx.x; e <= K; e += kThreads) out[e] = -1;
      if (threadIdx.x == 0) a.num_accepted[b] = -1;
    }
    return;
  }
  // the row to draw from: the residual at the first rejection, else p_{K+1}
  const float* pr = pb + int64_t(n) * V;
  const float* qr = n < K ? qb + int64_t(n) * V : nullptr;
  const int64_t x0 = min(V, int64_t(c) * a.chunk), x1 = min(V, x0 + a.chunk);
  uint64_t s_w, s_p;
  row_totals<VEC>(pr + x0, qr ? qr + x0 : nullptr, x1 - x0, red, &s_w, &s_p);
  if (threadIdx.x == 0) {
    uint64_t* slot = a.sums + (int64_t(b) * a.C + c) * 2;
    __hip_atomic_store(slot, s_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slot + 1, s_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // the sums are complete before the chunk counts in
    arrived = __hip_atomic_fetch_add(&a.counters[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (arrived != a.C - 1) return;
  // last chunk in: the chunks' sums (one thread each, into LDS), then total
  // weight, target and the chunk that holds it
  __shared__ uint64_t chunk_sums[kMaxChunks][2];
  if (threadIdx.x < a.C) {
    const uint64_t* slot = a.sums + (int64_t(b) * a.C + threadIdx.x) * 2;
    chunk_sums[threadIdx.x][0] = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    chunk_sums[threadIdx.x][1] = __hip_atomic_load(slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t S = 0, Sp = 0;
    for (int cc = 0; cc < a.C; ++cc) {
      S += chunk_sums[cc][0];
      Sp += chunk_sums[cc][1];
    }
    int use_p = 0;
    if (S == 0 && qr) {  // residual zero to 2^-32 everywhere: draw from p
      use_p = 1;
      S = Sp;
    }
    int64_t chunk_hit = -1;
    uint64_t T = 0;
    if (S > 0) {
      const uint64_t U = a.u_draw[b];
      T = U * (S >> 32) + ((U * (S & 0xffffffffull)) >> 32);  // floor(U * S / 2^32)
      uint64_t run = 0;
      for (int cc = 0; cc < a.C; ++cc) {
        const uint64_t w = chunk_sums[cc][use_p];
        if (run + w > T) {
          chunk_hit = cc;
          break;
        }
        run += w;
      }
      T -= run;
    }
    pick_chunk = chunk_hit;
    pick_target = T;
    pick_use_p = use_p;
    __hip_atomic_store(&a.counters[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next call
  }
  __syncthreads();
  int32_t tok = -1;
  if (pick_chunk >= 0) {
    const int64_t y0 = pick_chunk * a.chunk, y1 = min(V, y0 + a.chunk);
    const float* qq = (qr && !pick_use_p) ? qr + y0 : nullptr;
    const int32_t local = row_find<VEC>(pr + y0, qq, y1 - y0, pick_target, red, &found);
    tok = local < 0 ? -1 : int32_t(y0 + local);
  }
  for (int e = threadIdx.x; e <= K; e += kThreads)
    out[e] = e < n ? a.draft[int64_t(b) * K + e] : (e == n ? tok : -1);
  if (threadIdx.x == 0) a.num_accepted[b] = n;
}

// Chunks per sequence: about 1024 workgroups in all (four per compute unit,
// all resident at once), each chunk at least 4096 tokens (a multiple of 4).
void spec_layout(int32_t num_seqs, int32_t vocab, int32_t* C, int64_t* chunk) {
  const int64_t want = (1024 + num_seqs - 1) / num_seqs;
  const int64_t most = std::max<int64_t>(1, std::min<int64_t>(kMaxChunks, int64_t(vocab) / 4096));
  const int64_t cc = std::max<int64_t>(1, std::min(want, most));
  const int64_t ch = ((int64_t(vocab) + cc - 1) / cc + 3) / 4 * 4;
  *C = int32_t((int64_t(vocab) + ch - 1) / ch);
  *chunk = ch;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

extern "C" size_t pa_spec_accept_workspace_size(int32_t num_seqs, int32_t vocab) {
  if (num_seqs < 1 || vocab < 1) return 0;
  int32_t C;
  int64_t chunk;
  spec_layout(num_seqs, vocab, &C, &chunk);
  return align256(size_t(num_seqs) * sizeof(int32_t)) + size_t(num_seqs) * C * 2 * sizeof(uint64_t);
}

extern "C" pa_status pa_spec_accept(const float* p, const float* q, const int32_t* draft,
                                    const float* u_accept, const uint32_t* u_draw, int32_t num_seqs,
                                    int32_t num_draft, int32_t vocab, int32_t* num_accepted,
                                    int32_t* tokens, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (num_seqs < 1 || num_draft < 0 || vocab < 1 || !p || !u_draw || !num_accepted || !tokens)
    return PA_ERR_INVALID_ARG;
  if (num_draft > 0 && (!q || !draft || !u_accept)) return PA_ERR_INVALID_ARG;
  const size_t need = pa_spec_accept_workspace_size(num_seqs, vocab);
  if (!workspace || workspace_bytes < need) return PA_ERR_INVALID_ARG;
  SpecArgs a;
  spec_layout(num_seqs, vocab, &a.C, &a.chunk);
  if (int64_t(num_seqs) * a.C > INT32_MAX) return PA_ERR_UNSUPPORTED;
  a.p = p;
  a.q = num_draft > 0 ? q : nullptr;
  a.draft = draft;
  a.u_accept = u_accept;
  a.u_draw = u_draw;
  a.counters = static_cast<int32_t*>(workspace);
  a.sums = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) +
                                       align256(size_t(num_seqs) * sizeof(int32_t)));
  a.num_accepted = num_accepted;
  a.tokens = tokens;
  a.K = num_draft;
  a.V = vocab;
  const bool vec = vocab % 4 == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.q) & 15) == 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(num_seqs) * unsigned(a.C));
  if (vec)
    hipLaunchKernelGGL(spec_accept_kernel<true>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(spec_accept_kernel<false>, grid, dim3(kThreads), 0, s, a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : pa::hip_failed(e);
}
