// Device half of writing the paged KV cache: the copy-on-write block copy and
// the scatter of new tokens' K/V rows into their physical slots.
//
// Blog #54, interview question 2: a growing sequence gets a new block per
// block_size tokens, and a write into a block shared by several sequences
// first gives the writer its own copy; the host plan (pool.cpp) takes those
// decisions, these kernels move the bytes.
//
// Pool layout: k_pool [NB][H_kv][d/32][bs][32], v_pool [NB][H_kv][d][bs];
// FP8 pools: codes k [NB][H_kv][d/64][bs][64], v [NB][H_kv][d][bs], each
// followed by fp32 scales [NB][H_kv][bs].
// Both kernels take their block ids by value (kernel arguments), so a write
// needs no device-side staging buffer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "pa_internal.h"

namespace {

constexpr int kIdsPerLaunch = 64;    // logical blocks covered by one scatter launch
constexpr int kPairsPerLaunch = 32;  // block copies per copy launch

struct BlockIds {
  int32_t id[kIdsPerLaunch];
};
struct CopyPairs {
  int32_t src[kPairsPerLaunch];
  int32_t dst[kPairsPerLaunch];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One thread per (token, kv head, 16-byte chunk of the head dim).
// Token i of this launch is sequence position pos0 + i; its logical block is
// pos / bs, found at ids.id[pos / bs - first_logical].
template <typename T>
__global__ void scatter_kernel(T* __restrict__ k_pool, T* __restrict__ v_pool,
                               const T* __restrict__ k_new, const T* __restrict__ v_new,
                               BlockIds ids, int32_t first_logical, int32_t pos0, int32_t tok0,
                               int32_t n_tok, int32_t hkv, int32_t d, int32_t bs) {
  constexpr int VEC = 16 / sizeof(T);
  const int chunks = d / VEC;
  const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(n_tok) * hkv * chunks;
  if (tid >= total) return;
  const int c = int(tid % chunks);
  const int h = int((tid / chunks) % hkv);
  const int i = int(tid / (int64_t(chunks) * hkv));
  const int pos = pos0 + i;
  const int64_t blk = ids.id[pos / bs - first_logical];
  const int off = pos % bs;
  const int64_t src = (int64_t(tok0 + i) * hkv + h) * d + int64_t(c) * VEC;
  // K: elements c*VEC .. c*VEC+VEC-1 of the row sit in slab (c*VEC)/32 at the
  // token's 32-element run (16 contiguous bytes, never straddling a slab)
  const int e0 = c * VEC;
  *reinterpret_cast<u32x4*>(k_pool + ((blk * hkv + h) * (d / 32) + e0 / 32) * (int64_t(bs) * 32) +
                            off * 32 + e0 % 32) = *reinterpret_cast<const u32x4*>(k_new + src);
  // V: element e of the chunk goes to row (c*VEC + e) of the [d][bs] slice
  T* vdst = v_pool + ((blk * hkv + h) * d + int64_t(c) * VEC) * bs + off;
#pragma unroll
  for (int e = 0; e < VEC; ++e) vdst[int64_t(e) * bs] = v_new[src + e];
}

// FP8 pools: quantise while scattering. A group of d/8 lanes holds one
// (token, KV head) row, 8 bf16 elements per lane; the group's max |x| sets
// the scale, the smallest power of two >= amax / 448 (1 for an all-zero
// row), and each element becomes the E4M3 code of x / scale (exact: a power
// of two; then round to nearest even, v_cvt_pk_fp8_f32). Lanes past the end
// still take part in the group shuffles but store nothing.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The smallest power of two >= s, for finite s > 0 (subnormals included).
__device__ __forceinline__ float pow2_ceil(float s) {
  const uint32_t b = __float_as_uint(s);
  const uint32_t m = b & 0x7fffffu;
  if (m == 0) return s;                                                   // 2^e already
  if (b >= 0x800000u) return __uint_as_float((b & 0x7f800000u) + 0x800000u);  // the next binade
  return __uint_as_float(1u << (32 - __clz(m - 1)));  // subnormal: m units of 2^-149
}

__device__ __forceinline__ float bf16_bits_to_f(uint32_t b) { return __uint_as_float(b << 16); }

template <int D>
__global__ void scatter_fp8_kernel(uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes,
                                   float* __restrict__ k_scales, float* __restrict__ v_scales,
                                   const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                                   BlockIds ids, int32_t first_logical, int32_t pos0, int32_t tok0,
                                   int32_t n_tok, int32_t hkv, int32_t bs) {
  constexpr int LPT = D / 8;  // lanes per (token, head) row
  const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t row = tid / LPT;
  const int c = int(tid % LPT);
  const bool live = row < int64_t(n_tok) * hkv;
  const int h = int(row % hkv);
  const int i = int(row / hkv);
  float kx[8], vx[8];
  float kmax = 0.f, vmax = 0.f;
  if (live) {
    const int64_t src = (int64_t(tok0 + i) * hkv + h) * D + 8 * c;
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(k_new + src);
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(v_new + src);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a = kw[e], b = vw[e];
      kx[2 * e] = bf16_bits_to_f(a & 0xffffu);
      kx[2 * e + 1] = bf16_bits_to_f(a >> 16);
      vx[2 * e] = bf16_bits_to_f(b & 0xffffu);
      vx[2 * e + 1] = bf16_bits_to_f(b >> 16);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kmax = fmaxf(kmax, fabsf(kx[e]));
      vmax = fmaxf(vmax, fabsf(vx[e]));
    }
  }
#pragma unroll
  for (int o = LPT / 2; o >= 1; o >>= 1) {
    kmax = fmaxf(kmax, __shfl_xor(kmax, o));
    vmax = fmaxf(vmax, __shfl_xor(vmax, o));
  }
  if (!live) return;
  const float ks = kmax > 0.f ? pow2_ceil(kmax / 448.f) : 1.f;
  const float vs = vmax > 0.f ? pow2_ceil(vmax / 448.f) : 1.f;
  uint32_t kc[2], vc[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int kp = __builtin_amdgcn_cvt_pk_fp8_f32(kx[4 * w] / ks, kx[4 * w + 1] / ks, 0, false);
    kp = __builtin_amdgcn_cvt_pk_fp8_f32(kx[4 * w + 2] / ks, kx[4 * w + 3] / ks, kp, true);
    int vp = __builtin_amdgcn_cvt_pk_fp8_f32(vx[4 * w] / vs, vx[4 * w + 1] / vs, 0, false);
    vp = __builtin_amdgcn_cvt_pk_fp8_f32(vx[4 * w + 2] / vs, vx[4 * w + 3] / vs, vp, true);
    kc[w] = uint32_t(kp);
    vc[w] = uint32_t(vp);
  }
  const int pos = pos0 + i;
  const int64_t blk = ids.id[pos / bs - first_logical];
  const int off = pos % bs;
  const int e0 = 8 * c;
  // K: slab e0/64 of 64 elements per token
  *reinterpret_cast<u32x2*>(k_codes + ((blk * hkv + h) * (D / 64) + e0 / 64) * (int64_t(bs) * 64) +
                            off * 64 + e0 % 64) = (u32x2){kc[0], kc[1]};
  // V: one byte in each of the head-dim rows e0 .. e0+7 of the [d][bs] slice
  uint8_t* vdst = v_codes + ((blk * hkv + h) * D + e0) * bs + off;
#pragma unroll
  for (int e = 0; e < 8; ++e) vdst[int64_t(e) * bs] = uint8_t(vc[e / 4] >> (8 * (e % 4)));
  if (c == 0) {
    k_scales[(blk * hkv + h) * bs + off] = ks;
    v_scales[(blk * hkv + h) * bs + off] = vs;
  }
}

// grid.y = pair index; each thread copies 16 bytes of the K slice and of the V
// slice of one block (both are block_elems elements long and contiguous).
template <typename T>
__global__ void copy_blocks_kernel(T* __restrict__ k_pool, T* __restrict__ v_pool, CopyPairs pairs,
                                   int64_t block_elems) {
  constexpr int VEC = 16 / sizeof(T);
  const int64_t v = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v * VEC >= block_elems) return;
  const int64_t s = pairs.src[blockIdx.y] * block_elems + v * VEC;
  const int64_t t = pairs.dst[blockIdx.y] * block_elems + v * VEC;
  *reinterpret_cast<u32x4*>(k_pool + t) = *reinterpret_cast<const u32x4*>(k_pool + s);
  *reinterpret_cast<u32x4*>(v_pool + t) = *reinterpret_cast<const u32x4*>(v_pool + s);
}

template <typename T>
pa_status launch_copies(const pa_pool* p, void* k_pool, void* v_pool, const int32_t* src_dst,
                        int32_t n_pairs, hipStream_t stream,
                        int64_t block_elems_override = 0) {
  const int64_t block_elems = block_elems_override ? block_elems_override
                                                   : int64_t(p->num_kv_heads) * p->block_size * p->head_dim;
  constexpr int VEC = 16 / sizeof(T);
  const int threads = 256;
  const unsigned gx = unsigned((block_elems / VEC + threads - 1) / threads);
  for (int32_t k0 = 0; k0 < n_pairs; k0 += kPairsPerLaunch) {
    const int32_t n = std::min<int32_t>(kPairsPerLaunch, n_pairs - k0);
    CopyPairs cp{};
    for (int32_t k = 0; k < n; ++k) {
      cp.src[k] = src_dst[2 * (k0 + k)];
      cp.dst[k] = src_dst[2 * (k0 + k) + 1];
    }
    hipLaunchKernelGGL(copy_blocks_kernel<T>, dim3(gx, n), dim3(threads), 0, stream,
                       static_cast<T*>(k_pool), static_cast<T*>(v_pool), cp, block_elems);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return pa::hip_failed(e);
  }
  return PA_OK;
}

// FP8 pools: the codes (bytes) and then the scales (one float per token and head)
pa_status launch_copies_fp8(const pa_pool* p, void* k_pool, void* v_pool, const int32_t* src_dst,
                            int32_t n_pairs, hipStream_t stream) {
  pa_status st = launch_copies<uint8_t>(p, k_pool, v_pool, src_dst, n_pairs, stream);
  if (st != PA_OK) return st;
  const int64_t codes = pa::fp8_codes_bytes(p->num_blocks, p->num_kv_heads, p->block_size, p->head_dim);
  return launch_copies<float>(p, static_cast<char*>(k_pool) + codes, static_cast<char*>(v_pool) + codes,
                              src_dst, n_pairs, stream, int64_t(p->num_kv_heads) * p->block_size);
}

pa_status launch_scatter_fp8(const pa_pool* p, void* k_pool, void* v_pool, const int32_t* table,
                             int32_t start_pos, int32_t n_tokens, const void* k_new, const void* v_new,
                             hipStream_t stream) {
  const int32_t bs = p->block_size, hkv = p->num_kv_heads, d = p->head_dim;
  const int64_t codes = pa::fp8_codes_bytes(p->num_blocks, hkv, bs, d);
  uint8_t* kc = static_cast<uint8_t*>(k_pool);
  uint8_t* vc = static_cast<uint8_t*>(v_pool);
  float* ksc = reinterpret_cast<float*>(kc + codes);
  float* vsc = reinterpret_cast<float*>(vc + codes);
  const int32_t end = start_pos + n_tokens;
  const int32_t first = start_pos / bs, last = (end - 1) / bs;
  for (int32_t lb = first; lb <= last; lb += kIdsPerLaunch) {
    const int32_t lb_end = std::min(last + 1, lb + kIdsPerLaunch);
    BlockIds ids{};
    for (int32_t j = lb; j < lb_end; ++j) ids.id[j - lb] = table[j];
    const int32_t pos0 = std::max(start_pos, lb * bs);
    const int32_t pos1 = std::min(end, lb_end * bs);
    const int32_t n = pos1 - pos0;
    const int64_t total = int64_t(n) * hkv * (d / 8);
    const int threads = 256;
    const unsigned grid = unsigned((total + threads - 1) / threads);
    const uint16_t* kn = static_cast<const uint16_t*>(k_new);
    const uint16_t* vn = static_cast<const uint16_t*>(v_new);
    if (d == 64)
      hipLaunchKernelGGL(scatter_fp8_kernel<64>, dim3(grid), dim3(threads), 0, stream, kc, vc, ksc, vsc, kn,
                         vn, ids, lb, pos0, pos0 - start_pos, n, hkv, bs);
    else
      hipLaunchKernelGGL(scatter_fp8_kernel<128>, dim3(grid), dim3(threads), 0, stream, kc, vc, ksc, vsc, kn,
                         vn, ids, lb, pos0, pos0 - start_pos, n, hkv, bs);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return pa::hip_failed(e);
  }
  return PA_OK;
}

template <typename T>
pa_status launch_scatter(const pa_pool* p, void* k_pool, void* v_pool, const int32_t* table,
                         int32_t start_pos, int32_t n_tokens, const void* k_new,
                         const void* v_new, hipStream_t stream) {
  const int32_t bs = p->block_size, hkv = p->num_kv_heads, d = p->head_dim;
  constexpr int VEC = 16 / sizeof(T);
  const int32_t end = start_pos + n_tokens;
  const int32_t first = start_pos / bs, last = (end - 1) / bs;
  for (int32_t lb = first; lb <= last; lb += kIdsPerLaunch) {
    const int32_t lb_end = std::min(last + 1, lb + kIdsPerLaunch);
    BlockIds ids{};
    for (int32_t j = lb; j < lb_end; ++j) ids.id[j - lb] = table[j];
    const int32_t pos0 = std::max(start_pos, lb * bs);
    const int32_t pos1 = std::min(end, lb_end * bs);
    const int32_t n = pos1 - pos0;
    const int64_t total = int64_t(n) * hkv * (d / VEC);
    const int threads = 256;
    const unsigned grid = unsigned((total + threads - 1) / threads);
    hipLaunchKernelGGL(scatter_kernel<T>, dim3(grid), dim3(threads), 0, stream,
                       static_cast<T*>(k_pool), static_cast<T*>(v_pool),
                       static_cast<const T*>(k_new), static_cast<const T*>(v_new), ids, lb,
                       pos0, pos0 - start_pos, n, hkv, d, bs);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return pa::hip_failed(e);
  }
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_copy_blocks(const pa_pool* pool, void* k_pool, void* v_pool,
                                    const int32_t* src_dst, int32_t n_pairs, void* stream) {
  if (!pool || n_pairs < 0 || (n_pairs > 0 && (!k_pool || !v_pool || !src_dst)))
    return PA_ERR_INVALID_ARG;
  for (int32_t k = 0; k < 2 * n_pairs; ++k)
    if (src_dst[k] < 0 || src_dst[k] >= pool->num_blocks) return PA_ERR_INVALID_ARG;
  for (int32_t k = 0; k < n_pairs; ++k)
    if (src_dst[2 * k] == src_dst[2 * k + 1]) return PA_ERR_INVALID_ARG;
  if (n_pairs == 0) return PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pool->dtype == PA_DTYPE_FP8_E4M3) return launch_copies_fp8(pool, k_pool, v_pool, src_dst, n_pairs, s);
  return pool->dtype == PA_DTYPE_F32 ? launch_copies<float>(pool, k_pool, v_pool, src_dst, n_pairs, s)
                                     : launch_copies<uint16_t>(pool, k_pool, v_pool, src_dst, n_pairs, s);
}

extern "C" pa_status pa_write_kv(pa_pool* pool, void* k_pool, void* v_pool,
                                 int32_t* block_table_host, int32_t table_capacity,
                                 int32_t* num_blocks_inout, int32_t start_pos, int32_t n_tokens,
                                 const void* k_new, const void* v_new, void* stream) {
  return pa::guarded([&]() -> pa_status {
    if (!pool || !block_table_host || !num_blocks_inout) return PA_ERR_INVALID_ARG;
    if (n_tokens > 0 && (!k_pool || !v_pool || !k_new || !v_new)) return PA_ERR_INVALID_ARG;
    std::vector<int32_t> copies;
    pa_status st = pa::plan_write(pool, block_table_host, table_capacity, num_blocks_inout,
                                  start_pos, n_tokens, &copies, INT32_MAX, nullptr);
    if (st != PA_OK || n_tokens == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t n_pairs = static_cast<int32_t>(copies.size() / 2);
    if (pool->dtype == PA_DTYPE_FP8_E4M3) {
      if (n_pairs) st = launch_copies_fp8(pool, k_pool, v_pool, copies.data(), n_pairs, s);
      if (st == PA_OK)
        st = launch_scatter_fp8(pool, k_pool, v_pool, block_table_host, start_pos, n_tokens, k_new, v_new, s);
    } else if (pool->dtype == PA_DTYPE_F32) {
      if (n_pairs) st = launch_copies<float>(pool, k_pool, v_pool, copies.data(), n_pairs, s);
      if (st == PA_OK)
        st = launch_scatter<float>(pool, k_pool, v_pool, block_table_host, start_pos, n_tokens,
                                   k_new, v_new, s);
    } else {
      if (n_pairs) st = launch_copies<uint16_t>(pool, k_pool, v_pool, copies.data(), n_pairs, s);
      if (st == PA_OK)
        st = launch_scatter<uint16_t>(pool, k_pool, v_pool, block_table_host, start_pos, n_tokens,
                                      k_new, v_new, s);
    }
    return st;
  });
}
