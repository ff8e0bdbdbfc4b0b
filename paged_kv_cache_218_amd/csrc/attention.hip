// Paged decode / verification attention for gfx950 (MI355X).
//
// What is computed (Part 8, "Thực Thi Kernel Toán Học Trong CUDA"): for query
// row q_i, softmax(q_i K^T / sqrt(d_k)) V over the sequence's context, where
// the keys and values live in physical blocks reached through the block
// table, processed block by block with an online softmax (running maximum,
// running sum of exponentials, rescaled accumulator).
//
// Work decomposition (one GPU):
//   * a workgroup owns one (sequence b, KV head g, partition p) and all
//     G*q_len query rows that read KV head g (GQA: query head h reads KV
//     head h / G), so each K/V byte is read from HBM once per sequence;
//   * a partition is a token range of partition_tokens; its wavefronts take
//     32- or 64-token steps round-robin, each keeping its own online-softmax
//     state, merged through LDS at the end;
//   * with one partition per sequence the workgroup writes the output; with
//     several, it writes (m, l, o) partials and the merge kernel combines them
//     with the log-sum-exp identity (sequence-parallel attention: local
//     attention per KV segment, then a reduction; "Mở rộng Quy mô và Triển
//     khai", "Song song hóa Chuỗi").
//
// Two main kernels:
//   mfma_attn  bf16. Per 32-token step, scores S^T[token][row] come from
//              v_mfma_f32_16x16x32_bf16 with the K rows as the A operand and
//              the query rows as B; the output accumulator O^T[d][row] from
//              the same instruction with the V^T slice as A and the bf16
//              probabilities as B. Each lane owns one query row (lane % 16),
//              so the softmax rescale is lane-local; only the per-step row
//              maximum crosses lanes.
//   valu_attn  f32 or bf16, any row count up to 16. One lane per token for
//              the scores (query rows broadcast from LDS), probabilities
//              through LDS, one lane per head-dim element for P.V.
// Scores are kept in the base-2 domain (scale * log2(e) folded into one
// multiplier) so every exponential is a single v_exp_f32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "pa_internal.h"

namespace {

constexpr int kCUs = 256;              // MI355X compute units
constexpr int kMaxPartitions = 4096;   // merge kernel keeps P weights in LDS
constexpr int kMfmaMaxRows = 32;       // two 16-row tiles
constexpr int kValuMaxRows = 16;
constexpr float kLog2e = 1.4426950408889634f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  void* out;
  float* part_ml;  // [rows_total][P][2]  (m in base-2 units, l)
  float* part_o;   // [rows_total][P][d]
  int32_t hq, hkv, group, mb, nb, q_len, max_ctx, parts, part_tokens;
  float scale_log2;  // scale * log2(e)
};

__device__ __forceinline__ float bf16_to_f(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

__device__ __forceinline__ uint16_t f_to_bf16(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// two floats -> packed bf16x2 (round to nearest even, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> __device__ __forceinline__ float load_f(const T* p);
template <> __device__ __forceinline__ float load_f<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p) { return bf16_to_f(*p); }

template <typename T> __device__ __forceinline__ void store_f(T* p, float v);
template <> __device__ __forceinline__ void store_f<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_f<uint16_t>(uint16_t* p, float v) { *p = f_to_bf16(v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Decode the workgroup id. Returns false when the partition is empty.
struct Tile {
  int b, g, part, L, t0, t1;
  bool bad;
};

__device__ __forceinline__ Tile decode_tile(const AttnArgs& a) {
  Tile t;
  t.part = blockIdx.x % a.parts;
  const int bg = blockIdx.x / a.parts;
  t.g = bg % a.hkv;
  t.b = bg / a.hkv;
  t.L = a.lens[t.b];
  t.bad = t.L < a.q_len || t.L > a.max_ctx;
  t.t0 = t.part * a.part_tokens;
  t.t1 = t.bad ? 0 : min(t.t0 + a.part_tokens, t.L);
  return t;
}

// Row r of a (b, g) group: draft position i = r / G, query head g*G + r % G.
// Flat output row index (matches out[B][q_len][H_q][d]).
__device__ __forceinline__ int out_row(const AttnArgs& a, int b, int g, int r) {
  const int i = r / a.group, hh = r % a.group;
  return (b * a.q_len + i) * a.hq + g * a.group + hh;
}

// Cross-wave merge of per-wave online-softmax states kept in LDS, then the
// final or partial write. m_s/l_s: [W][rows_pad]; o_s: [W][rows_pad][D].
template <typename T, int D>
__device__ void merge_and_store(const AttnArgs& a, const Tile& t, int R, int rows_pad, int W,
                                const float* m_s, const float* l_s, const float* o_s,
                                bool poisoned) {
  const int nthreads = blockDim.x;
  for (int e = threadIdx.x; e < R * D; e += nthreads) {
    const int r = e / D, c = e % D;
    float M = -INFINITY;
    for (int w = 0; w < W; ++w) M = fmaxf(M, m_s[w * rows_pad + r]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float l = 0.f, o = 0.f;
    for (int w = 0; w < W; ++w) {
      const float f = fast_exp2(m_s[w * rows_pad + r] - Mu);
      l += f * l_s[w * rows_pad + r];
      o += f * o_s[(w * rows_pad + r) * D + c];
    }
    const float val = poisoned ? NAN : (l > 0.f ? o / l : 0.f);
    const int row = out_row(a, t.b, t.g, r);
    if (a.parts == 1) {
      store_f<T>(static_cast<T*>(a.out) + int64_t(row) * D + c, val);
    } else {
      const int64_t pi = int64_t(row) * a.parts + t.part;
      a.part_o[pi * D + c] = val;
      if (c == 0) {
        a.part_ml[pi * 2 + 0] = poisoned ? NAN : M;
        a.part_ml[pi * 2 + 1] = poisoned ? NAN : l;
      }
    }
  }
}

// Sequence with an out-of-range length: every output row is NaN (written by
// partition 0 only, or by the merge kernel when there are partials).
template <typename T, int D>
__device__ void poison_rows(const AttnArgs& a, const Tile& t, int R) {
  if (t.part != 0 || a.parts != 1) return;
  for (int e = threadIdx.x; e < R * D; e += blockDim.x) {
    const int row = out_row(a, t.b, t.g, e / D);
    store_f<T>(static_cast<T*>(a.out) + int64_t(row) * D + e % D, NAN);
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel (bf16)
// ---------------------------------------------------------------------------
// Lane l: n = l % 16 (query row within a 16-row tile), j = l / 16.
// v_mfma_f32_16x16x32_bf16 operands: A lane l holds A[m = l%16][k = 8j..8j+7],
// B lane l holds B[k = 8j..8j+7][col = l%16], C lane l holds C[4j..4j+3][l%16].
// QK: two 16-token tiles per 32-token step; tile i's A row m is token
//   8*(m/4) + 4*i + m%4, so C of tile i gives lane l the scores of tokens
//   8j+4i .. 8j+4i+3 and, over both tiles, tokens 8j .. 8j+7 of the step.
// PV: O^T[d][row] += V^T[d][tok] P^T[tok][row]; the B operand is the lane's
//   own 8 probabilities (tokens 8j..8j+7 of row n), the A operand 8 adjacent
//   tokens of one head-dim row of the V^T slice: 16 contiguous bytes.
template <int D, int BS, int NT>
__global__ __launch_bounds__(256) void mfma_attn(AttnArgs a) {
  constexpr int KS = D / 32;  // k-steps over the head dim for QK
  constexpr int DT = D / 16;  // 16-row tiles of the head dim for PV
  extern __shared__ float smem[];
  const int W = blockDim.x / 64;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int n = lane & 15, j = lane >> 4;
  const Tile t = decode_tile(a);
  const int R = a.group * a.q_len;
  if (t.bad) { poison_rows<uint16_t, D>(a, t, R); return; }
  if (t.t0 >= t.L) return;

  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v_pool);
  const int32_t* __restrict__ table = a.tables + int64_t(t.b) * a.mb;

  // query rows as the B operand of QK, per 16-row tile and k-step
  u32x4 qop[NT][KS];
  int lim[NT];  // last visible position of this lane's row
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + n;
    lim[nt] = t.L - a.q_len + min(r, R - 1) / a.group;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (r < R) {
        const int i = r / a.group, h = t.g * a.group + r % a.group;
        v = *reinterpret_cast<const u32x4*>(q + (int64_t(t.b * a.q_len + i) * a.hq + h) * D + 32 * ks + 8 * j);
      }
      qop[nt][ks] = v;
    }
  }

  f32x4 acc[NT][DT];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[nt][dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  bool poisoned = false;

  const int nsteps = (t.t1 - t.t0 + 31) / 32;
  const int64_t head_stride = int64_t(BS) * D;  // elements of one (block, head) slice
  for (int s = wave; s < nsteps; s += W) {
    const int tb = t.t0 + 32 * s;
    // physical blocks of this step (uniform across the wave)
    int blk0 = table[tb / BS];
    int blk1 = blk0;
    bool have1 = true;
    if (BS == 16) {
      have1 = tb + 16 < t.L;
      blk1 = have1 ? table[tb / BS + 1] : blk0;
    }
    if (blk0 < 0 || blk0 >= a.nb || blk1 < 0 || blk1 >= a.nb) {
      poisoned = true;
      continue;
    }
    const uint16_t* kb0 = kp + (int64_t(blk0) * a.hkv + t.g) * head_stride;
    const uint16_t* kb1 = kp + (int64_t(blk1) * a.hkv + t.g) * head_stride;
    const uint16_t* vb0 = vp + (int64_t(blk0) * a.hkv + t.g) * head_stride;
    const uint16_t* vb1 = vp + (int64_t(blk1) * a.hkv + t.g) * head_stride;

    // K tiles: A operand, token of row n in tile i
    u32x4 kop[2][KS];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tok = 8 * (n >> 2) + 4 * i + (n & 3);
      const uint16_t* row;
      bool ok = true;
      if (BS == 32) {
        row = kb0 + tok * D;
      } else {
        row = (tok < 16 ? kb0 : kb1) + (tok & 15) * D;
        ok = tok < 16 || have1;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0, 0, 0, 0};
        if (ok) v = *reinterpret_cast<const u32x4*>(row + 32 * ks + 8 * j);
        kop[i][ks] = v;
      }
    }
    // V^T slices: A operand of PV, head-dim row 16*dt + n, tokens 8j..8j+7
    u32x4 vop[DT];
    {
      const uint16_t* base;
      bool ok = true;
      if (BS == 32) {
        base = vb0 + 8 * j;
      } else {
        base = (j < 2 ? vb0 : vb1) + 8 * (j & 1);
        ok = j < 2 || have1;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u32x4 v = {0, 0, 0, 0};
        if (ok) v = *reinterpret_cast<const u32x4*>(base + (16 * dt + n) * BS);
        vop[dt] = v;
      }
    }
    // tail step: zero V entries past the context so 0 * NaN never reaches the sum
    if (tb + 32 > t.L) {
      const int valid = min(max(t.L - (tb + 8 * j), 0), 8);  // tokens of this lane's 8 still valid
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        const uint32_t keep = (2 * w4 + 1 < valid) ? 0xffffffffu : (2 * w4 < valid ? 0x0000ffffu : 0u);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vop[dt][w4] &= keep;
      }
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 sc[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        sc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[i][ks]),
                                                           __builtin_bit_cast(bf16x8, qop[nt][ks]),
                                                           sc[i], 0, 0, 0);
      }
      // mask and scale; e = 4*i + r is token tb + 8j + e
      float s2[8];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = tb + 8 * j + 4 * i + r;
          const bool vis = tok < t.t1 && tok <= lim[nt];
          const float v = vis ? sc[i][r] * a.scale_log2 : -INFINITY;
          s2[4 * i + r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[nt] - m_use);
      m_run[nt] = m_new;
      uint32_t pk[4];
      float psum = 0.f;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        const float p0 = fast_exp2(s2[2 * w4] - m_use);
        const float p1 = fast_exp2(s2[2 * w4 + 1] - m_use);
        const uint32_t packed = pack_bf16x2(p0, p1);
        pk[w4] = packed;
        // the sum uses the rounded weights, so the output stays a convex combination
        psum += __uint_as_float(packed << 16) + __uint_as_float(packed & 0xffff0000u);
      }
      l_run[nt] = l_run[nt] * alpha + psum;
      const u32x4 pop = {pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        acc[nt][dt] *= alpha;
        acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop[dt]),
                                                              __builtin_bit_cast(bf16x8, pop),
                                                              acc[nt][dt], 0, 0, 0);
      }
    }
  }

  // row sums: each lane holds its 8-token share; add the 4 lanes of the row
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    l_run[nt] += __shfl_xor(l_run[nt], 16);
    l_run[nt] += __shfl_xor(l_run[nt], 32);
  }
  // park the per-wave states of the R real rows in LDS:
  // m_s[W][R], l_s[W][R], o_s[W][R][D]
  float* m_s = smem;
  float* l_s = m_s + W * R;
  float* o_s = l_s + W * R;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + n;
    if (r < R) {
      if (j == 0) {
        m_s[wave * R + r] = m_run[nt];
        l_s[wave * R + r] = l_run[nt];
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int k = 0; k < 4; ++k) o_s[(wave * R + r) * D + 16 * dt + 4 * j + k] = acc[nt][dt][k];
    }
  }
  // a bad table entry in any wave poisons the whole workgroup
  const int any_bad = __syncthreads_or(poisoned ? 1 : 0);
  merge_and_store<uint16_t, D>(a, t, R, R, W, m_s, l_s, o_s, any_bad != 0);
}

// ---------------------------------------------------------------------------
// VALU kernel (f32 or bf16)
// ---------------------------------------------------------------------------
// Per 64-token step: lane l computes the scores of token tb + l for every
// query row (query rows broadcast from LDS), the wave reduces the step maximum
// per row, probabilities go through LDS, and lane l then accumulates head-dim
// elements l and l + 64 of every row over the step's tokens from the V^T
// slices (16-byte loads of adjacent tokens).
template <typename T, int D, int BS>
__global__ __launch_bounds__(256) void valu_attn(AttnArgs a) {
  constexpr int VEC = 16 / sizeof(T);     // elements per 16-byte load
  constexpr int DPL = D / 64;             // head-dim elements per lane in P.V
  constexpr int RM = kValuMaxRows;
  extern __shared__ float smem[];
  const int W = blockDim.x / 64;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const Tile t = decode_tile(a);
  const int R = a.group * a.q_len;
  if (t.bad) { poison_rows<T, D>(a, t, R); return; }
  if (t.t0 >= t.L) return;

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ kp = static_cast<const T*>(a.k_pool);
  const T* __restrict__ vp = static_cast<const T*>(a.v_pool);
  const int32_t* __restrict__ table = a.tables + int64_t(t.b) * a.mb;

  // LDS: q_s[RM][D] | p_s[W][RM][64] ; the merge reuses the space after q_s
  float* q_s = smem;
  float* p_s = q_s + RM * D;
  for (int e = threadIdx.x; e < RM * D; e += blockDim.x) {
    const int r = e / D, c = e % D;
    float v = 0.f;
    if (r < R) {
      const int i = r / a.group, h = t.g * a.group + r % a.group;
      v = load_f<T>(q + (int64_t(t.b * a.q_len + i) * a.hq + h) * D + c) * a.scale_log2;
    }
    q_s[e] = v;
  }
  __syncthreads();

  float m_run[RM], l_run[RM], acc[RM][DPL];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[r][k] = 0.f;
  }
  bool poisoned = false;
  float* pw = p_s + wave * RM * 64;
  const int64_t head_stride = int64_t(BS) * D;
  const int nsteps = (t.t1 - t.t0 + 63) / 64;

  for (int s = wave; s < nsteps; s += W) {
    const int tb = t.t0 + 64 * s;
    const int tok = tb + lane;
    const bool in = tok < t.t1;
    // scores of this lane's token
    float sc[RM];
#pragma unroll
    for (int r = 0; r < RM; ++r) sc[r] = 0.f;
    int blk = in ? table[tok / BS] : 0;
    const bool blk_ok = blk >= 0 && blk < a.nb;
    if (in && !blk_ok) poisoned = true;
    if (in && blk_ok) {
      const T* krow = kp + (int64_t(blk) * a.hkv + t.g) * head_stride + (tok % BS) * D;
      for (int c0 = 0; c0 < D; c0 += VEC) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(krow + c0);
        float kv[VEC];
        if constexpr (sizeof(T) == 4) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) kv[e] = __uint_as_float(raw[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv[2 * e] = __uint_as_float(raw[e] << 16);
            kv[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
          }
        }
#pragma unroll
        for (int r = 0; r < RM; ++r) {
          if (r < R) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) sc[r] = fmaf(q_s[r * D + c0 + e], kv[e], sc[r]);
          }
        }
      }
    }
    // online softmax per row over the step
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r >= R) continue;
      const int lim = t.L - a.q_len + r / a.group;
      const float v = (in && blk_ok && tok <= lim) ? sc[r] : -INFINITY;
      float mx = v;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_new = fmaxf(m_run[r], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[r] - m_use);
      const float pr = fast_exp2(v - m_use);
      m_run[r] = m_new;
      l_run[r] = l_run[r] * alpha + pr;   // lane-partial sum, reduced at the end
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[r][k] *= alpha;
      pw[r * 64 + lane] = pr;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // P.V over the step's tokens, block by block
    const int ntok = min(64, t.t1 - tb);
    for (int kb = 0; kb * BS < ntok; ++kb) {
      const int tok0 = tb + kb * BS;
      const int vb = table[tok0 / BS];
      if (vb < 0 || vb >= a.nb) { poisoned = true; continue; }
      const int cnt = min(BS, t.t1 - tok0);
      const T* vslice = vp + (int64_t(vb) * a.hkv + t.g) * head_stride;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const T* vrow = vslice + int64_t(lane + 64 * k) * BS;
        for (int u0 = 0; u0 < cnt; u0 += VEC) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(vrow + u0);
          float vv[VEC];
          if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) vv[e] = __uint_as_float(raw[e]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              vv[2 * e] = __uint_as_float(raw[e] << 16);
              vv[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
            }
          }
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            if (u0 + e < cnt) {
              const int tt = kb * BS + u0 + e;
#pragma unroll
              for (int r = 0; r < RM; ++r)
                if (r < R) acc[r][k] = fmaf(pw[r * 64 + tt], vv[e], acc[r][k]);
            }
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  // reduce the lane-partial sums over the wave
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    if (r >= R) continue;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l_run[r] += __shfl_xor(l_run[r], o);
  }
  __syncthreads();  // q_s/p_s are reused below
  float* m_s = smem;
  float* l_s = m_s + W * RM;
  float* o_s = l_s + W * RM;
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    if (r >= R) continue;
    if (lane == 0) {
      m_s[wave * RM + r] = m_run[r];
      l_s[wave * RM + r] = l_run[r];
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) o_s[(wave * RM + r) * D + lane + 64 * k] = acc[r][k];
  }
  const int any_bad = __syncthreads_or(poisoned ? 1 : 0);
  merge_and_store<T, D>(a, t, R, RM, W, m_s, l_s, o_s, any_bad != 0);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partition partials
// ---------------------------------------------------------------------------
// One workgroup (D threads) per output row: M = max_p m_p, w_p = l_p 2^(m_p-M),
// out = sum_p w_p o_p / sum_p w_p over the partitions the sequence has.
template <typename T, int D>
__global__ __launch_bounds__(128) void lse_merge(AttnArgs a) {
  __shared__ float w_s[kMaxPartitions];
  __shared__ float red[D / 64 + 1];
  const int row = blockIdx.x;
  const int b = row / (a.q_len * a.hq);
  const int L = a.lens[b];
  T* out = static_cast<T*>(a.out) + int64_t(row) * D;
  const int c = threadIdx.x;
  if (L < a.q_len || L > a.max_ctx) {
    store_f<T>(out + c, NAN);
    return;
  }
  const int np = (L + a.part_tokens - 1) / a.part_tokens;
  const float* ml = a.part_ml + int64_t(row) * a.parts * 2;
  const float* po = a.part_o + int64_t(row) * a.parts * D;
  // global maximum
  float mx = -INFINITY;
  for (int p = c; p < np; p += D) mx = fmaxf(mx, ml[2 * p]);
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((c & 63) == 0) red[c / 64] = mx;
  __syncthreads();
  float M = red[0];
  for (int k = 1; k < D / 64; ++k) M = fmaxf(M, red[k]);
  __syncthreads();
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float wsum = 0.f;
  for (int p = c; p < np; p += D) {
    const float w = ml[2 * p + 1] * fast_exp2(ml[2 * p] - Mu);
    w_s[p] = w;
    wsum += w;
  }
  for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o);
  if ((c & 63) == 0) red[c / 64] = wsum;
  __syncthreads();
  float denom = 0.f;
  for (int k = 0; k < D / 64; ++k) denom += red[k];
  float acc = 0.f;
  for (int p = 0; p < np; ++p) acc = fmaf(w_s[p], po[int64_t(p) * D + c], acc);
  store_f<T>(out + c, denom > 0.f ? acc / denom : NAN);
}

// ---------------------------------------------------------------------------
// Host side: validation, planning, launch
// ---------------------------------------------------------------------------
struct Plan {
  int path, part_tokens, parts, waves, grid, merge_grid, nt, rows;
  size_t ws;
};

int ceil_div(int64_t x, int64_t y) { return int((x + y - 1) / y); }

pa_status make_plan(const pa_attn_desc* d, int32_t q_len, Plan* pl) {
  if (!d || !pl) return PA_ERR_INVALID_ARG;
  for (int k = 0; k < 5; ++k)
    if (d->reserved[k] != 0) return PA_ERR_INVALID_ARG;
  if (d->num_seqs < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->num_q_heads % d->num_kv_heads != 0 || d->max_blocks_per_seq < 1 || d->num_blocks < 1 ||
      q_len < 1 || d->max_context < 1 || d->partition_tokens < 0 || d->partition_tokens % 64 != 0)
    return PA_ERR_INVALID_ARG;
  if (d->dtype != PA_DTYPE_F32 && d->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (!pa::supported_head_dim(d->head_dim) || !pa::supported_block_size(d->block_size))
    return PA_ERR_UNSUPPORTED;
  if (int64_t(d->max_context) > int64_t(d->max_blocks_per_seq) * d->block_size ||
      q_len > d->max_context)
    return PA_ERR_INVALID_ARG;
  const int G = d->num_q_heads / d->num_kv_heads;
  const int64_t rows = int64_t(G) * q_len;
  int path = d->path;
  if (path == PA_PATH_AUTO) {
    if (d->dtype == PA_DTYPE_BF16 && rows <= kMfmaMaxRows) path = PA_PATH_MFMA;
    else path = PA_PATH_VALU;
  }
  if (path == PA_PATH_MFMA) {
    if (d->dtype != PA_DTYPE_BF16 || rows > kMfmaMaxRows) return PA_ERR_UNSUPPORTED;
  } else if (path == PA_PATH_VALU) {
    if (rows > kValuMaxRows) return PA_ERR_UNSUPPORTED;
  } else {
    return PA_ERR_INVALID_ARG;
  }
  const int waves = 4;
  const int64_t pairs = int64_t(d->num_seqs) * d->num_kv_heads;
  int pt = d->partition_tokens;
  if (pt == 0) {
    // enough waves to give every compute unit 8 of them, partitions >= 256 tokens
    const int64_t want = (int64_t(kCUs) * 8 + pairs * waves - 1) / (pairs * waves);
    const int max_parts = std::max(1, ceil_div(d->max_context, 256));
    const int parts = int(std::min<int64_t>(std::max<int64_t>(want, 1), max_parts));
    pt = ceil_div(ceil_div(d->max_context, parts), 64) * 64;
  }
  const int parts = ceil_div(d->max_context, pt);
  if (parts > kMaxPartitions) return PA_ERR_UNSUPPORTED;
  const int64_t grid = pairs * parts;
  const int64_t out_rows = int64_t(d->num_seqs) * q_len * d->num_q_heads;
  if (grid > INT32_MAX || out_rows > INT32_MAX) return PA_ERR_UNSUPPORTED;
  pl->path = path;
  pl->part_tokens = pt;
  pl->parts = parts;
  pl->waves = waves;
  pl->grid = int(grid);
  pl->merge_grid = parts > 1 ? int(out_rows) : 0;
  pl->nt = rows > 16 ? 2 : 1;
  pl->rows = int(rows);
  pl->ws = parts > 1 ? size_t(out_rows) * parts * (d->head_dim + 2) * sizeof(float) : 0;
  return PA_OK;
}

size_t lds_bytes(const Plan& pl, int D) {
  if (pl.path == PA_PATH_MFMA) return size_t(pl.waves) * pl.rows * (D + 2) * sizeof(float);
  const size_t first = size_t(kValuMaxRows) * D + size_t(pl.waves) * kValuMaxRows * 64;
  const size_t merge = size_t(pl.waves) * kValuMaxRows * (D + 2);
  return std::max(first, merge) * sizeof(float);
}

template <int D, int BS>
pa_status launch_main(const Plan& pl, int dtype, const AttnArgs& args, hipStream_t s) {
  const dim3 grid(pl.grid), block(64 * pl.waves);
  const size_t lds = lds_bytes(pl, D);
  if (pl.path == PA_PATH_MFMA) {
    if (pl.nt == 1) hipLaunchKernelGGL((mfma_attn<D, BS, 1>), grid, block, lds, s, args);
    else hipLaunchKernelGGL((mfma_attn<D, BS, 2>), grid, block, lds, s, args);
  } else if (dtype == PA_DTYPE_F32) {
    hipLaunchKernelGGL((valu_attn<float, D, BS>), grid, block, lds, s, args);
  } else {
    hipLaunchKernelGGL((valu_attn<uint16_t, D, BS>), grid, block, lds, s, args);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <int D>
pa_status launch_merge(const Plan& pl, int dtype, const AttnArgs& args, hipStream_t s) {
  if (dtype == PA_DTYPE_F32)
    hipLaunchKernelGGL((lse_merge<float, D>), dim3(pl.merge_grid), dim3(D), 0, s, args);
  else
    hipLaunchKernelGGL((lse_merge<uint16_t, D>), dim3(pl.merge_grid), dim3(D), 0, s, args);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" pa_status pa_attention_plan(const pa_attn_desc* desc, int32_t q_len, pa_attn_plan* out) {
  if (!out) return PA_ERR_INVALID_ARG;
  Plan pl;
  pa_status st = make_plan(desc, q_len, &pl);
  if (st != PA_OK) return st;
  out->path = pl.path;
  out->partition_tokens = pl.part_tokens;
  out->num_partitions = pl.parts;
  out->waves_per_group = pl.waves;
  out->grid = pl.grid;
  out->merge_grid = pl.merge_grid;
  out->workspace_bytes = pl.ws;
  return PA_OK;
}

extern "C" size_t pa_attention_workspace_size(const pa_attn_desc* desc, int32_t q_len) {
  Plan pl;
  return make_plan(desc, q_len, &pl) == PA_OK ? pl.ws : 0;
}

extern "C" pa_status pa_attention(const pa_attn_desc* desc, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables,
                                  const int32_t* context_lens, int32_t q_len, float scale,
                                  void* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  Plan pl;
  pa_status st = make_plan(desc, q_len, &pl);
  if (st != PA_OK) return st;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (pl.ws > 0 && (!workspace || workspace_bytes < pl.ws)) return PA_ERR_INVALID_ARG;
  AttnArgs args;
  args.q = q;
  args.k_pool = k_pool;
  args.v_pool = v_pool;
  args.tables = block_tables;
  args.lens = context_lens;
  args.out = out;
  const int64_t out_rows = int64_t(desc->num_seqs) * q_len * desc->num_q_heads;
  args.part_ml = pl.ws ? static_cast<float*>(workspace) : nullptr;
  args.part_o = pl.ws ? static_cast<float*>(workspace) + out_rows * pl.parts * 2 : nullptr;
  args.hq = desc->num_q_heads;
  args.hkv = desc->num_kv_heads;
  args.group = desc->num_q_heads / desc->num_kv_heads;
  args.mb = desc->max_blocks_per_seq;
  args.nb = desc->num_blocks;
  args.q_len = q_len;
  args.max_ctx = desc->max_context;
  args.parts = pl.parts;
  args.part_tokens = pl.part_tokens;
  args.scale_log2 = scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = desc->head_dim, BS = desc->block_size;
  if (D == 64) st = BS == 16 ? launch_main<64, 16>(pl, desc->dtype, args, s) : launch_main<64, 32>(pl, desc->dtype, args, s);
  else st = BS == 16 ? launch_main<128, 16>(pl, desc->dtype, args, s) : launch_main<128, 32>(pl, desc->dtype, args, s);
  if (st != PA_OK || pl.parts == 1) return st;
  return D == 64 ? launch_merge<64>(pl, desc->dtype, args, s) : launch_merge<128>(pl, desc->dtype, args, s);
}
