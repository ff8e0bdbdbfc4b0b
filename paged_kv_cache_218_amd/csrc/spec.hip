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
// One workgroup of 1024 threads per sequence: the acceptance tests are a few
// scalar reads; the draw reads the chosen row twice (the weight total, then
// a tiled prefix scan that stops at the tile holding the target), 16 bytes
// per thread per load.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_internal.h"

namespace {

constexpr int kThreads = 1024;
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

// Total fixed-point weight of a row (p - q residual when q is given).
template <bool VEC>
__device__ uint64_t row_total(const float* p, const float* q, int64_t V, uint64_t* red) {
  uint64_t s = 0;
  if constexpr (VEC) {
    const int64_t n4 = V / 4;
    for (int64_t i = threadIdx.x; i < n4; i += kThreads) {
      const f32x4 a = reinterpret_cast<const f32x4*>(p)[i];
      f32x4 w = a;
      if (q) {
        const f32x4 b = reinterpret_cast<const f32x4*>(q)[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = fmaxf(a[e] - b[e], 0.f);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) s += fixed_weight(w[e]);
    }
  } else {
    for (int64_t x = threadIdx.x; x < V; x += kThreads) s += fixed_weight(weight(p, q, x));
  }
  return block_sum(s, red);
}

// Smallest x whose running fixed-point weight exceeds T (T < the row total).
template <bool VEC>
__device__ int32_t row_find(const float* p, const float* q, int64_t V, uint64_t T, uint64_t* red,
                            int32_t* found) {
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

template <bool VEC>
__global__ __launch_bounds__(kThreads) void spec_accept_kernel(
    const float* __restrict__ p, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const float* __restrict__ u_accept, const uint32_t* __restrict__ u_draw, int32_t K, int64_t V,
    int32_t* __restrict__ num_accepted, int32_t* __restrict__ tokens) {
  __shared__ uint64_t red[kWaves];
  __shared__ int32_t found;
  const int b = blockIdx.x;
  const float* pb = p + int64_t(b) * (K + 1) * V;
  const float* qb = q ? q + int64_t(b) * K * V : nullptr;
  // acceptance tests (every thread takes the same decisions)
  int n = 0;
  bool valid = true;
  for (; n < K; ++n) {
    const int32_t x = draft[int64_t(b) * K + n];
    if (x < 0 || x >= V) {
      valid = false;
      break;
    }
    const float px = pb[int64_t(n) * V + x], qx = qb[int64_t(n) * V + x];
    const float u = u_accept[int64_t(b) * K + n];
    if (!(px >= qx || u * qx < px)) break;
  }
  int32_t* out = tokens + int64_t(b) * (K + 1);
  if (!valid) {
    for (int e = threadIdx.x; e <= K; e += kThreads) out[e] = -1;
    if (threadIdx.x == 0) num_accepted[b] = -1;
    return;
  }
  // the row to draw from: the residual at the first rejection, else p_{K+1}
  const float* pr = pb + int64_t(n) * V;
  const float* qr = n < K ? qb + int64_t(n) * V : nullptr;
  uint64_t S = row_total<VEC>(pr, qr, V, red);
  if (S == 0 && qr) {  // residual zero to 2^-32 everywhere: draw from p
    qr = nullptr;
    S = row_total<VEC>(pr, qr, V, red);
  }
  int32_t tok = -1;
  if (S > 0) {
    const uint64_t U = u_draw[b];
    const uint64_t T = U * (S >> 32) + ((U * (S & 0xffffffffull)) >> 32);  // floor(U * S / 2^32)
    tok = row_find<VEC>(pr, qr, V, T, red, &found);
  }
  for (int e = threadIdx.x; e <= K; e += kThreads)
    out[e] = e < n ? draft[int64_t(b) * K + e] : (e == n ? tok : -1);
  if (threadIdx.x == 0) num_accepted[b] = n;
}

}  // namespace

extern "C" pa_status pa_spec_accept(const float* p, const float* q, const int32_t* draft,
                                    const float* u_accept, const uint32_t* u_draw, int32_t num_seqs,
                                    int32_t num_draft, int32_t vocab, int32_t* num_accepted,
                                    int32_t* tokens, void* stream) {
  if (num_seqs < 1 || num_draft < 0 || vocab < 1 || !p || !u_draw || !num_accepted || !tokens)
    return PA_ERR_INVALID_ARG;
  if (num_draft > 0 && (!q || !draft || !u_accept)) return PA_ERR_INVALID_ARG;
  if (int64_t(num_seqs) > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
  const bool vec = vocab % 4 == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(q) & 15) == 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const float* qq = num_draft > 0 ? q : nullptr;
  if (vec)
    hipLaunchKernelGGL(spec_accept_kernel<true>, dim3(num_seqs), dim3(kThreads), 0, s, p, qq, draft,
                       u_accept, u_draw, num_draft, int64_t(vocab), num_accepted, tokens);
  else
    hipLaunchKernelGGL(spec_accept_kernel<false>, dim3(num_seqs), dim3(kThreads), 0, s, p, qq, draft,
                       u_accept, u_draw, num_draft, int64_t(vocab), num_accepted, tokens);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : pa::hip_failed(e);
}
