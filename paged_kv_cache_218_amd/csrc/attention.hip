// Paged decode / verification attention for gfx950 (MI355X).
//
// What is computed (Part 8, "Thực Thi Kernel Toán Học Trong CUDA"): for query
// row q_i, softmax(q_i K^T / sqrt(d_k)) V over the sequence's context, where
// the keys and values live in physical blocks reached through the block
// table, processed block by block with an online softmax (running maximum,
// running sum of exponentials, rescaled accumulator).
//
// Every (sequence b, KV head g) is one segment of work: all G*q_len query
// rows that read KV head g (GQA: query head h reads KV head h / G) go through
// the segment's tokens together, so each K/V byte is read from HBM once per
// sequence. A wavefront takes 32-token steps (64 in the VALU kernel) and
// keeps its own online-softmax state; the states of a workgroup's waves are
// merged through LDS.
//
// Two schedules:
//   balanced    (default) the grid is the device's resident capacity; the
//               (KV head, sequence, step) list is cut into one contiguous
//               range per workgroup, equal in steps (prefix sums of the
//               steps computed in every workgroup from context_lens), the
//               ranges of one XCD consecutive (so it holds whole KV heads). A
//               segment inside one range is written directly; a segment cut
//               by range boundaries leaves (m, l, o) partials, and the
//               workgroup that counts the last piece in merges them with the
//               log-sum-exp identity.
//   partitions  a workgroup per (sequence, KV head, partition of
//               partition_tokens tokens); partitions write partials and
//               lse_merge combines them (sequence-parallel attention: local
//               attention per KV segment, then a reduction; "Mở rộng Quy mô
//               và Triển khai", "Song song hóa Chuỗi"). When the partitions
//               alone fill the device's wave slots, a wavefront per partition
//               instead, its partial written from registers.
//
// Kernels:
//   mfma_attn_balanced, mfma_attn, mfma_attn_wave  bf16 queries. Per 32-token step, scores
//              S^T[token][row] come from v_mfma_f32_16x16x32_bf16 with the K
//              rows as the A operand and the query rows as B; the output
//              accumulator O^T[d][row] from the same instruction with the
//              V^T slice as A and the bf16 probabilities as B. Each lane owns
//              one query row (lane % 16), so the softmax rescale is
//              lane-local; only the per-step row maximum crosses lanes. One
//              or two 16-row tiles (NT). A wave keeps one K and one V
//              register buffer and refills each with the next step's loads
//              as soon as the step has consumed it (next K after the score
//              MFMAs, next V during P.V). Template variants: FP8 E4M3 pools
//              (KV8: codes converted to bf16 in registers, per-token scales on
//              the scores and the P.V weights), tree masks over the drafted
//              positions (TREE), non-temporal K/V loads (STREAM).
//   valu_attn  f32 or bf16, any row count up to 16. One lane per token for
//              the scores (query rows broadcast from LDS), probabilities
//              through LDS, one lane per head-dim element for P.V.
//   lse_merge  the partitions' merge.
// Scores are kept in the base-2 domain (scale * log2(e) folded into one
// multiplier) so every exponential is a single v_exp_f32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "pa_internal.h"

// Scratch of the entry point that allocates nothing (pa_attention_noalloc):
// one array per device, held until the process ends. Its first
// kScratchCounterBytes hold the balanced schedule's arrival counters (cleared
// by every call that uses them), the rest the partials. In host code
// `scratch` only names the symbol: its device address comes from
// scratch_base().
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchCounterBytes = size_t(256) << 10;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace pa {
namespace {
thread_local int g_last_hip_error = 0;
}
pa_status hip_failed(int hip_error) {
  g_last_hip_error = hip_error;
  return PA_ERR_HIP;
}
}  // namespace pa

extern "C" int32_t pa_last_hip_error(void) { return pa::g_last_hip_error; }

extern "C" const char* pa_hip_error_name(int32_t hip_error) {
  return hipGetErrorName(static_cast<hipError_t>(hip_error));
}

namespace {

constexpr int kMaxCUs = 256;           // compute units the workspace bound allows for (MI355X: 256)
constexpr int kMaxPartitions = 1 << 16;  // partitions per sequence
constexpr int kMfmaMaxRows = 32;       // two 16-row tiles
constexpr int kValuMaxRows = 16;
constexpr float kLog2e = 1.4426950408889634f;
// Lazy online-softmax rescaling: how far (base 2) a row's scores may exceed
// its reference maximum before the reference moves; weights stay <= 2^8.
constexpr float kLazyRescale = 8.f;

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
  float* part_ml;  // partitions: [rows_total][P][2]; balanced: [pieces][R][2] (m base-2, l)
  float* part_o;   // partitions: [rows_total][P][d]; balanced: [pieces][R][d]
  int32_t* counters;  // balanced: arrival count per segment, zero between calls
  const float* k_scales;  // FP8 pools: per (block, head, slot) scales after the codes
  const float* v_scales;
  const uint32_t* tree_mask;  // tree verification: visibility bits per drafted row, or null (causal)
  int32_t mask_stride;        // masks between consecutive sequences (0: one set for all)
  int32_t num_seqs, hq, hkv, group, mb, nb, q_len, max_ctx, parts, part_tokens;
  float scale_log2;  // scale * log2(e)
  int32_t seg_cost;  // balanced: what starting a segment costs, in steps, when ranges are cut
  int32_t run_parts;  // one wavefront per partition: consecutive partitions per wavefront (>= 1)
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

// Device-coherent accesses for data handed between workgroups of one launch
// (which may sit on different XCDs, each with its own L2): agent-scope
// relaxed atomic stores write through to the device-coherent level and
// agent-scope relaxed atomic loads read from it, so no L2 writeback or
// invalidate is needed.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 64- and 128-bit accesses with the same coherence (the sc1 cache policy) for
// the balanced schedule's partials, through buffer resources over one
// piece's (or one segment's) partials; out-of-range accesses read zero and
// write nothing.
constexpr int kCoherent = 16;  // sc1 cache-policy bit
constexpr int kRawBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, int(bytes), kRawBufferWord3);
}
__device__ __forceinline__ f32x4 load4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kCoherent));
}
__device__ __forceinline__ f32x2 load2_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, kCoherent));
}
__device__ __forceinline__ void store4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, int(off), 0, kCoherent);
}
__device__ __forceinline__ void store2_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, int(off), 0, kCoherent);
}

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

// Which drafted positions row i (0 <= i < q_len) of sequence b sees: bit j
// stands for position L - q_len + j. Plain verification is causal (bits
// 0..i); a tree of drafted tokens passes one mask per row, whose own bit is
// always taken as set (speculative decoding variants: parallel decoding
// verifies a whole tree of candidates in one pass; "Mở rộng Quy mô và Triển
// khai", "Giải mã Suy đoán"). Every position before L - q_len is context,
// visible to every row.
__device__ __forceinline__ uint32_t row_mask(const AttnArgs& a, int b, int i) {
  if (a.tree_mask) return a.tree_mask[int64_t(b) * a.mask_stride + i] | (1u << i);
  return (2u << i) - 1u;  // i = 31 wraps to all ones
}

// Row r of a (b, g) group: draft position i = r / G, query head g*G + r % G.
// Flat output row index (matches out[B][q_len][H_q][d]).
__device__ __forceinline__ int out_row(const AttnArgs& a, int b, int g, int r) {
  const int i = r / a.group, hh = r % a.group;
  return (b * a.q_len + i) * a.hq + g * a.group + hh;
}

// Cross-wave merge of per-wave online-softmax states kept in LDS, then the
// final or partial write. m_s/l_s: [W][rows_pad]; o_s: [W][rows_pad][O_STRIDE].
template <typename T, int D, int O_STRIDE = D>
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
      o += f * o_s[(w * rows_pad + r) * O_STRIDE + c];
    }
    const float val = poisoned ? NAN : (l > 0.f ? o / l : 0.f);
    const int row = out_row(a, t.b, t.g, r);
    if (t.L <= a.part_tokens) {  // the sequence has this one partition: final output
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
// MFMA path (bf16)
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
constexpr int kStep = 32;  // tokens per MFMA step

// 16-byte K/V load. STREAM: each block is read once per call (no sharing), so
// the load carries the non-temporal hint and the bytes do not displace the
// tables, queries and partials in the caches; otherwise (blocks shared by
// several sequences, e.g. a common prompt) the load is cached normally.
template <bool STREAM>
__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

template <bool STREAM>
__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}
template <bool STREAM>
__device__ __forceinline__ u32x2 load8(const uint8_t* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  else return *reinterpret_cast<const u32x2*>(p);
}
template <bool STREAM>
__device__ __forceinline__ f32x4 load16f(const float* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  else return *reinterpret_cast<const f32x4*>(p);
}

// two E4M3 codes (the low or high 16 bits of w) -> two bf16, exactly
template <bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, HIGH));
}

// Maximum over the four lanes n, n+16, n+32, n+48 of a wavefront (the lanes
// holding one MFMA row), returned in all four: two lane-swap steps between
// 16-lane rows and between 32-lane halves, VALU work with no LDS round trip.
__device__ __forceinline__ float row_max4(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

template <int D>
struct StepBuf {
  u32x4 k[2][D / 32];  // two 16-token K tiles, D/32 k-steps each
  u32x4 v[D / 16];     // V^T head-dim tiles
};

// FP8 pools: 16 K codes per lane per 64-element slab (two MFMA k-steps), 8 V
// codes per lane per head-dim tile, and the K and V scales of the lane's 8
// tokens (8j .. 8j+7 of the step).
template <int D>
struct StepBuf8 {
  u32x4 k[2][D / 64];
  u32x2 v[D / 16];
  f32x4 ks[2], vs[2];
};

// Online-softmax state of one wavefront: lane (n, j) holds row 16*nt + n,
// head-dim elements 16*dt + 4*j .. +3 of the accumulator.
template <int D, int NT>
struct WaveState {
  f32x4 acc[NT][D / 16];
  float m[NT], l[NT];
  bool poisoned;
};

template <int D, int NT>
__device__ __forceinline__ void wave_state_init(WaveState<D, NT>& st) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    st.m[nt] = -INFINITY;
    st.l[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) st.acc[nt][dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  st.poisoned = false;
}

// One wavefront's share of a piece: steps first, first+W, ... < end of
// sequence b (context L), KV head g. Every step covers 32 tokens; tokens at
// or past L, and tokens after a row's causal limit, are masked.
// next_step(s) gives the wave's step after s (>= end: none left).
// on_step(s) runs after each of the wave's steps except its last, once step
// s is in the state (its loads for the next step already issued).
struct NoStepHook {
  __device__ void operator()(int) const {}
};
template <int D, int BS, int NT, bool STREAM, bool KV8, bool TREE, typename NextStep, typename OnStep = NoStepHook>
__device__ void mfma_wave_steps(const AttnArgs& a, int b, int g, int L, int first, int end,
                                WaveState<D, NT>& st, NextStep next_step, OnStep on_step = {}) {
  constexpr int KS = D / 32;  // k-steps over the head dim for QK
  constexpr int DT = D / 16;  // 16-row tiles of the head dim for PV
  const int lane = threadIdx.x % 64;
  const int n = lane & 15, j = lane >> 4;
  const int R = a.group * a.q_len;
  // The segment and the step range are the same in every lane of the wave
  // (they come from LDS, so the compiler cannot see it): held in scalar
  // registers, the table entries become scalar loads, which never wait on
  // the K/V loads in flight.
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  L = __builtin_amdgcn_readfirstlane(L);
  first = __builtin_amdgcn_readfirstlane(first);
  end = __builtin_amdgcn_readfirstlane(end);
  if (first >= end) return;

  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v_pool);
  const int32_t* __restrict__ table = a.tables + int64_t(b) * a.mb;

  // query rows as the B operand of QK, per 16-row tile and k-step. The k
  // elements of lane j in k-step ks: d = 32ks + 8j .. +7 (bf16 pools), or
  // d = 64(ks/2) + 16j + 8(ks%2) .. +7 (FP8 pools, where one 16-byte load
  // holds two k-steps of a token's 64-element slab)
  u32x4 qop[NT][KS];
  // causal rows: last visible position; tree rows: the drafted positions seen
  int lim[NT];
  uint32_t vbits[NT];
  const int ctx_end = L - a.q_len;  // first drafted position
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + n;
    const int row_i = min(r, R - 1) / a.group;
    if constexpr (TREE)
      vbits[nt] = row_mask(a, b, row_i) & (a.q_len >= 32 ? ~0u : (1u << a.q_len) - 1u);
    else lim[nt] = ctx_end + row_i;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (r < R) {
        const int i = r / a.group, h = g * a.group + r % a.group;
        const int d0 = KV8 ? 64 * (ks >> 1) + 16 * j + 8 * (ks & 1) : 32 * ks + 8 * j;
        v = *reinterpret_cast<const u32x4*>(q + (int64_t(b * a.q_len + i) * a.hq + h) * D + d0);
      }
      qop[nt][ks] = v;
    }
  }

  // Tree rows: visibility of the lane's 8 tokens tb + 8j .. +7 as bits 0..7,
  // read from a 64-bit word whose low half stands for the 32 positions
  // before the drafted ones (context) and whose high half is the row's mask
  // (bits at or past q_len cleared, so positions at or past L are hidden).
  auto tree_bits = [&](int tb, int nt) -> uint32_t {
    const int off0 = tb + 8 * j - ctx_end;  // drafted index of the lane's first token
    if (off0 < -32) return 0xFFu;
    if (off0 >= 32) return 0u;
    const uint64_t w = (uint64_t(vbits[nt]) << 32) | 0xFFFFFFFFull;
    return uint32_t(w >> (off0 + 32)) & 0xFFu;
  };
  // token tok (= tb + 8j + e) is visible to this lane's row of tile nt
  auto visible = [&](int tok, int nt, uint32_t tbits, int e) -> bool {
    if constexpr (TREE) return (tbits >> e) & 1u;
    else return tok < L && tok <= lim[nt];
  };

  // Where one 32-token step's K and V live (wave-uniform). The table is never
  // written during a launch: read through the constant address space, its
  // entries are scalar loads, which never wait on the K/V loads in flight.
  struct StepLoc {
    int tb;          // first token of the step
    int64_t s0, s1;  // (block, head) slices of tokens 0-15 and 16-31
    bool ok;         // block ids in range
  };
  const __attribute__((address_space(4))) int32_t* ctable =
      (const __attribute__((address_space(4))) int32_t*)(table);
  auto locate = [&](int step) {
    StepLoc s;
    s.tb = kStep * step;
    const int blk0 = ctable[s.tb / BS];
    const bool have1 = BS == 32 || s.tb + 16 < L;  // block size 16: tokens 16-31 exist
    const int blk1 = (BS == 16 && have1) ? ctable[s.tb / BS + 1] : blk0;
    s.ok = blk0 >= 0 && blk0 < a.nb && blk1 >= 0 && blk1 < a.nb;
    s.s0 = s.ok ? int64_t(blk0) * a.hkv + g : 0;
    s.s1 = s.ok ? int64_t(blk1) * a.hkv + g : 0;
    return s;
  };
  // The accumulator rescale of the online softmax, skipped (a wave-uniform
  // branch) in steps where no row's reference maximum moved.
  auto rescale = [&](const float (&alpha)[NT]) {
    bool moved = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) moved |= alpha[nt] != 1.f;
    if (__ballot(moved) != 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) st.acc[nt][dt] *= alpha[nt];
    }
  };

  // Both step loops below keep one K and one V buffer per wave and refill
  // each with the next step's loads as soon as the current step has consumed
  // it: the next K right after the score MFMAs, the next V during P.V. A wave
  // thus keeps about a step's bytes in flight while it computes, in the
  // registers of one buffer (loads complete in issue order, so waiting for K
  // leaves V in flight and waiting for V leaves the next K in flight).
  //
  // The loads are unconditional (a branch per load would leave the compiler
  // unable to count them, and it would wait for every load in flight), and
  // always in bounds: a bad block id reads slice 0, the step is computed on
  // it and the wave is marked poisoned (its rows are written as NaN); a
  // missing second block (block size 16, tokens 16-31 past the context)
  // re-reads the first, whose tokens are then masked: scores by a select, V
  // entries zeroed before P.V. The last step is peeled off the loop, so the
  // loop body is straight-line.

  if constexpr (KV8) {
    const uint8_t* __restrict__ kc = static_cast<const uint8_t*>(a.k_pool);
    const uint8_t* __restrict__ vc = static_cast<const uint8_t*>(a.v_pool);
    const int64_t slice = int64_t(BS) * D;  // bytes of one (block, head) code slice
    // the lane's 8 tokens 8j..8j+7 of the step: their block and offset in it
    const bool second8 = BS == 16 && j >= 2;
    const int toff = BS == 32 ? 8 * j : 8 * (j & 1);
    // K codes (same lane layout as the bf16 tiles, 16 codes per 64-element
    // slab) and the K scales of the lane's 8 tokens
    auto load_k8 = [&](StepBuf8<D>& buf, const StepLoc& s) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int tok = 8 * (n >> 2) + 4 * i + (n & 3);
        const bool second = BS == 16 && tok >= 16;
        const uint8_t* row = kc + (second ? s.s1 : s.s0) * slice + (tok & (BS - 1)) * 64 + 16 * j;
#pragma unroll
        for (int sl = 0; sl < D / 64; ++sl) buf.k[i][sl] = load16<STREAM>(row + sl * (BS * 64));
      }
      const int64_t si = second8 ? s.s1 : s.s0;
#pragma unroll
      for (int h = 0; h < 2; ++h) buf.ks[h] = load16f<STREAM>(a.k_scales + si * BS + toff + 4 * h);
    };
    // V^T codes (8 per lane per head-dim tile) and the V scales of the lane's 8 tokens
    auto load_v8 = [&](StepBuf8<D>& buf, const StepLoc& s) {
      const int64_t si = second8 ? s.s1 : s.s0;
      const uint8_t* base = vc + si * slice + toff + n * BS;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) buf.v[dt] = load8<STREAM>(base + 16 * dt * BS);
#pragma unroll
      for (int h = 0; h < 2; ++h) buf.vs[h] = load16f<STREAM>(a.v_scales + si * BS + toff + 4 * h);
    };
    // Scores of every row tile, each times its token's K scale (exact: the
    // scale multiplies the dot product): the step's only use of K.
    auto qk8 = [&](const StepBuf8<D>& buf, f32x4 (&sc)[NT][2]) {
      // each token's K scale times scale * log2(e): the scores come out in base 2
      const f32x4 ks[2] = {buf.ks[0] * a.scale_log2, buf.ks[1] * a.scale_log2};
      // codes -> bf16 (exact); K: slab sl gives k-steps 2sl (codes 0-7) and 2sl+1 (8-15)
      u32x4 kop[2][KS];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int sl = 0; sl < D / 64; ++sl)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const uint32_t w0 = buf.k[i][sl][2 * hh], w1 = buf.k[i][sl][2 * hh + 1];
            kop[i][2 * sl + hh] = (u32x4){fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                                          fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1)};
          }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          sc[nt][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            sc[nt][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[i][ks]),
                                                                 __builtin_bit_cast(bf16x8, qop[nt][ks]),
                                                                 sc[nt][i], 0, 0, 0);
          // e = 4i + r is token tb + 8j + e
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[nt][i][r] *= ks[i][r];
        }
    };
    // Online softmax. Each weight is rounded to bf16 once (the row sum adds
    // the rounded weights, so the output stays a convex combination of the
    // dequantised V rows); its token's V scale, a power of two, then
    // multiplies it exactly, so P.V takes the scaled weights as bf16 numbers
    // with no further rounding.
    // FULL: a step every row sees whole (no masking work).
    auto softmax8 = [&](auto FULL, const f32x4 (&sc)[NT][2], const StepBuf8<D>& buf, int tb, u32x4 (&pop)[NT],
                        float (&alpha)[NT]) {
      constexpr bool kFull = decltype(FULL)::value;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float s2[8];
        bool vis[8];
        float mx = -INFINITY;
        const uint32_t tbits = (TREE && !kFull) ? tree_bits(tb, nt) : 0u;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * i + r;
            vis[e] = kFull || visible(tb + 8 * j + e, nt, tbits, e);
            const float v = vis[e] ? sc[nt][i][r] : -INFINITY;  // K scales carry scale * log2(e)
            s2[e] = v;
            mx = fmaxf(mx, v);
          }
        mx = row_max4(mx);
        // Lazy rescaling: the row's reference maximum m moves only when a
        // score exceeds it by more than kLazyRescale (base 2), so weights
        // stay below 2^kLazyRescale and the accumulator is rescaled only in
        // the rare steps where some row's maximum jumps (the result does not
        // depend on which reference is used: l and o are scaled alike).
        const bool grow = mx > st.m[nt] + kLazyRescale;
        const float m_new = grow ? mx : st.m[nt];
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        alpha[nt] = grow ? fast_exp2(st.m[nt] - m_use) : 1.f;
        st.m[nt] = m_new;
        uint32_t pk[4];
        float psum = 0.f;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const int e0 = 2 * w4, e1 = 2 * w4 + 1;
          const uint32_t pr = pack_bf16x2(fast_exp2(s2[e0] - m_use), fast_exp2(s2[e1] - m_use));
          const float p0 = __uint_as_float(pr << 16), p1 = __uint_as_float(pr & 0xffff0000u);
          psum += p0 + p1;
          // masked tokens: the select keeps a scale past the context (any
          // bits) out of the weight
          const float q0 = vis[e0] ? p0 * buf.vs[e0 / 4][e0 % 4] : 0.f;
          const float q1 = vis[e1] ? p1 * buf.vs[e1 / 4][e1 % 4] : 0.f;
          pk[w4] = pack_bf16x2(q0, q1);
        }
        st.l[nt] = st.l[nt] * alpha[nt] + psum;
        pop[nt] = (u32x4){pk[0], pk[1], pk[2], pk[3]};
      }
    };
    // P.V of one step (the step's only use of the V codes).
    auto accumulate8 = [&](const StepBuf8<D>& buf, int tb, const u32x4 (&pop)[NT], const float (&alpha)[NT],
                           bool last) {
      // tokens past the context hold the NaN code: zeroed by a select on the
      // wave's last step, the only one that can hold the sequence's tail
      const int valid = last ? min(max(L - (tb + 8 * j), 0), 8) : 8;
      uint32_t keep[4];
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4)
        keep[w4] = (2 * w4 + 1 < valid) ? 0xffffffffu : (2 * w4 < valid ? 0x0000ffffu : 0u);
      rescale(alpha);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint32_t w0 = buf.v[dt][0], w1 = buf.v[dt][1];
        const u32x4 vop = {fp8x2_to_bf16x2<false>(w0) & keep[0], fp8x2_to_bf16x2<true>(w0) & keep[1],
                           fp8x2_to_bf16x2<false>(w1) & keep[2], fp8x2_to_bf16x2<true>(w1) & keep[3]};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          st.acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop),
                                                                   __builtin_bit_cast(bf16x8, pop[nt]),
                                                                   st.acc[nt][dt], 0, 0, 0);
      }
    };
    StepBuf8<D> buf;
    StepLoc cur = locate(first);
    load_k8(buf, cur);
    load_v8(buf, cur);
    for (int sn = next_step(first); sn < end; sn = next_step(sn)) {
      const StepLoc nxt = locate(sn);
      f32x4 sc[NT][2];
      u32x4 pop[NT];
      float alpha[NT];
      qk8(buf, sc);
      __builtin_amdgcn_sched_barrier(0);
      load_k8(buf, nxt);
      __builtin_amdgcn_sched_barrier(0);
      if (cur.tb + kStep <= ctx_end) softmax8(std::true_type{}, sc, buf, cur.tb, pop, alpha);
      else softmax8(std::false_type{}, sc, buf, cur.tb, pop, alpha);
      accumulate8(buf, cur.tb, pop, alpha, false);
      load_v8(buf, nxt);
      st.poisoned |= !cur.ok;
      on_step(cur.tb / kStep);
      cur = nxt;
    }
    f32x4 sc[NT][2];
    u32x4 pop[NT];
    float alpha[NT];
    qk8(buf, sc);
    softmax8(std::false_type{}, sc, buf, cur.tb, pop, alpha);
    accumulate8(buf, cur.tb, pop, alpha, true);
    st.poisoned |= !cur.ok;
  } else {
    const int64_t head_stride = int64_t(BS) * D;  // elements of one (block, head) slice
    // K tiles: A operand, token of row n in tile i. K slab ks holds head-dim
    // elements 32ks..32ks+31 of the block's tokens back to back (64 B each),
    // so one load instruction reads tokens {0-3, 8-11, 16-19, 24-27} (tile 0)
    // or {4-7, ...} (tile 1) of slab ks: four runs of 256 contiguous bytes.
    auto load_k = [&](StepBuf<D>& buf, const StepLoc& s) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int tok = 8 * (n >> 2) + 4 * i + (n & 3);
        const bool second = BS == 16 && tok >= 16;
        const uint16_t* row = kp + (second ? s.s1 : s.s0) * head_stride + (tok & (BS - 1)) * 32 + 8 * j;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) buf.k[i][ks] = load16<STREAM>(row + ks * (BS * 32));
      }
    };
    // V^T slices: A operand of PV, head-dim row 16*dt + n, tokens 8j..8j+7
    auto load_v = [&](StepBuf<D>& buf, const StepLoc& s) {
      const bool second = BS == 16 && j >= 2;
      const uint16_t* base = vp + (second ? s.s1 : s.s0) * head_stride + (BS == 32 ? 8 * j : 8 * (j & 1)) + n * BS;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) buf.v[dt] = load16<STREAM>(base + 16 * dt * BS);
    };

    // Scores of every row tile: the step's only use of K.
    auto qk = [&](const StepBuf<D>& buf, f32x4 (&sc)[NT][2]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          sc[nt][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            sc[nt][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf.k[i][ks]),
                                                                 __builtin_bit_cast(bf16x8, qop[nt][ks]),
                                                                 sc[nt][i], 0, 0, 0);
        }
    };
    // Online softmax of the scores: leaves the bf16 probabilities and the
    // rescale factors for P.V.
    // FULL: a step every row sees whole (no masking work).
    auto softmax = [&](auto FULL, const f32x4 (&sc)[NT][2], int tb, u32x4 (&pop)[NT], float (&alpha)[NT]) {
      constexpr bool kFull = decltype(FULL)::value;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // mask and scale; e = 4*i + r is token tb + 8j + e
        float s2[8];
        float mx = -INFINITY;
        const uint32_t tbits = (TREE && !kFull) ? tree_bits(tb, nt) : 0u;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool vis = kFull || visible(tb + 8 * j + 4 * i + r, nt, tbits, 4 * i + r);
            const float v = vis ? sc[nt][i][r] * a.scale_log2 : -INFINITY;
            s2[4 * i + r] = v;
            mx = fmaxf(mx, v);
          }
        mx = row_max4(mx);
        // Lazy rescaling: the row's reference maximum m moves only when a
        // score exceeds it by more than kLazyRescale (base 2), so weights
        // stay below 2^kLazyRescale and the accumulator is rescaled only in
        // the rare steps where some row's maximum jumps (the result does not
        // depend on which reference is used: l and o are scaled alike).
        const bool grow = mx > st.m[nt] + kLazyRescale;
        const float m_new = grow ? mx : st.m[nt];
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        alpha[nt] = grow ? fast_exp2(st.m[nt] - m_use) : 1.f;
        st.m[nt] = m_new;
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
        st.l[nt] = st.l[nt] * alpha[nt] + psum;
        pop[nt] = (u32x4){pk[0], pk[1], pk[2], pk[3]};
      }
    };

    // P.V of one step (the step's only use of V).
    // last: the wave's last step, the only one that can hold the sequence's
    // tail (every earlier step of the wave is followed by one inside the
    // context, so it is full); a compile-time constant at each call.
    auto accumulate = [&](StepBuf<D>& buf, int tb, const u32x4 (&pop)[NT], const float (&alpha)[NT], bool last) {
      // zero V entries past the context so 0 * NaN never reaches the sum (a
      // select, not a branch)
      const int valid = last ? min(max(L - (tb + 8 * j), 0), 8) : 8;  // tokens of this lane's 8 still valid
      uint32_t keep[4];
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4)
        keep[w4] = (2 * w4 + 1 < valid) ? 0xffffffffu : (2 * w4 < valid ? 0x0000ffffu : 0u);
      rescale(alpha);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x4 vm = {buf.v[dt][0] & keep[0], buf.v[dt][1] & keep[1], buf.v[dt][2] & keep[2],
                          buf.v[dt][3] & keep[3]};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          st.acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vm),
                                                                   __builtin_bit_cast(bf16x8, pop[nt]),
                                                                   st.acc[nt][dt], 0, 0, 0);
        }
      }
    };

    // One K and one V buffer per wave, each refilled with the next step's
    // loads as soon as the current step has consumed it: the next K goes out
    // after the scores, the next V after P.V, so the wave keeps about a
    // step's bytes in flight while it computes, in the registers of a single
    // buffer. (Loads complete in issue order, so the wait for K before the
    // scores leaves V in flight, and the wait for V before P.V leaves the
    // next K in flight.)
    StepBuf<D> buf;
    StepLoc cur = locate(first);
    load_k(buf, cur);
    load_v(buf, cur);
    for (int sn = next_step(first); sn < end; sn = next_step(sn)) {
      const StepLoc nxt = locate(sn);
      f32x4 sc[NT][2];
      u32x4 pop[NT];
      float alpha[NT];
      qk(buf, sc);
      // the next K loads go out right after the score MFMAs, before the softmax
      __builtin_amdgcn_sched_barrier(0);
      load_k(buf, nxt);
      __builtin_amdgcn_sched_barrier(0);
      if (cur.tb + kStep <= ctx_end) softmax(std::true_type{}, sc, cur.tb, pop, alpha);
      else softmax(std::false_type{}, sc, cur.tb, pop, alpha);
      accumulate(buf, cur.tb, pop, alpha, false);
      load_v(buf, nxt);
      st.poisoned |= !cur.ok;
      on_step(cur.tb / kStep);
      cur = nxt;
    }
    f32x4 sc[NT][2];
    u32x4 pop[NT];
    float alpha[NT];
    qk(buf, sc);
    softmax(std::false_type{}, sc, cur.tb, pop, alpha);
    accumulate(buf, cur.tb, pop, alpha, true);
    st.poisoned |= !cur.ok;
  }
}

// Floats per parked row of a partition run: m, the 4 lanes' l, the poisoned
// flag, 2 unused, the D columns and 4 more, which make the stride (D + 12,
// 16-byte aligned) step 12 banks a row, so that the 16 rows a row tile
// writes at once fall in distinct banks (3n mod 16 takes every value).
__host__ __device__ constexpr int run_slot_row(int D) { return D + 12; }

// Row stride of the parked o rows: D + kParkPad floats. The 16 lanes of a
// row tile that hold the same columns write 16 rows at once; with a stride of
// D floats (a multiple of the 64 LDS banks) all 16 land in the same 4 banks,
// while 4 more floats per row move each row 4 banks on, over all 64.
constexpr int kParkPad = 4;

// Park each wave's state of the R real rows in LDS (m_s[W][R], l_s[W][R],
// o_s[W][R][D + kParkPad]) and return whether any wave of the workgroup saw a
// bad block.
template <int D, int NT>
__device__ bool park_states(const WaveState<D, NT>& st, int R, float* smem) {
  const int W = blockDim.x / 64;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int n = lane & 15, j = lane >> 4;
  float l_row[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {  // row sums: add the 4 lanes of the row
    l_row[nt] = st.l[nt] + __shfl_xor(st.l[nt], 16);
    l_row[nt] += __shfl_xor(l_row[nt], 32);
  }
  float* m_s = smem;
  float* l_s = m_s + W * R;
  float* o_s = l_s + W * R;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + n;
    if (r < R) {
      if (j == 0) {
        m_s[wave * R + r] = st.m[nt];
        l_s[wave * R + r] = l_row[nt];
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int k = 0; k < 4; ++k) o_s[(wave * R + r) * (D + kParkPad) + 16 * dt + 4 * j + k] = st.acc[nt][dt][k];
    }
  }
  return __syncthreads_or(st.poisoned ? 1 : 0) != 0;
}

// Combine the W parked wave states of a piece (log-sum-exp identity) in two
// passes: per-row weights first (one thread per row: M = max_w m_w, l = sum_w 2^(m_w - M) l_w, and
// weight_w = 2^(m_w - M) / l into wt [R][W]; M and l into row_ml [R][2]),
// then any 4-column chunk of a row is sum_w weight_w o_w (park_chunk). Ends
// with a barrier, after which every thread may read wt and row_ml.
__device__ void park_row_weights(const float* park, int W, int R, float* wt, float* row_ml) {
  const float* m_s = park;
  const float* l_s = m_s + W * R;
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    float M = -INFINITY;
    for (int w = 0; w < W; ++w) M = fmaxf(M, m_s[w * R + r]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float l = 0.f;
    for (int w = 0; w < W; ++w) {
      const float f = fast_exp2(m_s[w * R + r] - Mu);
      wt[r * W + w] = f;
      l += f * l_s[w * R + r];
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    for (int w = 0; w < W; ++w) wt[r * W + w] *= inv;
    row_ml[2 * r] = M;
    row_ml[2 * r + 1] = l;
  }
  __syncthreads();
}

// Columns c..c+3 of row r of the parked states combined (o = acc / l).
__device__ __forceinline__ f32x4 park_chunk(const float* park, int W, int R, int D, const float* wt, int r, int c) {
  const float* o_s = park + 2 * W * R;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int w = 0; w < W; ++w)
    acc += wt[r * W + w] * *reinterpret_cast<const f32x4*>(o_s + (w * R + r) * (D + kParkPad) + c);
  return acc;
}

// Fixed partitions: workgroup = (sequence, KV head, partition); partitions
// that do not cover the whole sequence leave partials for lse_merge.
template <int D, int BS, int NT, bool STREAM, bool KV8, bool TREE>
__global__ __launch_bounds__(256, 2) void mfma_attn(AttnArgs a) {
  extern __shared__ float smem[];
  const int W = blockDim.x / 64, wave = threadIdx.x / 64;
  const Tile t = decode_tile(a);
  const int R = a.group * a.q_len;
  if (t.bad) { poison_rows<uint16_t, D>(a, t, R); return; }
  if (t.t0 >= t.L) return;
  WaveState<D, NT> st;
  wave_state_init(st);
  const int s0 = t.t0 / kStep, s1 = (t.t1 + kStep - 1) / kStep;
  mfma_wave_steps<D, BS, NT, STREAM, KV8, TREE>(a, t.b, t.g, t.L, s0 + wave, s1, st,
                                                [W](int s) { return s + W; });
  const bool bad = park_states(st, R, smem);
  merge_and_store<uint16_t, D, D + kParkPad>(a, t, R, R, W, smem, smem + W * R, smem + 2 * W * R, bad);
}

// Fixed partitions, one wavefront per partition (chosen when the partitions
// fill the device on their own): wave w of workgroup k takes partition
// (k % gpw) * W + w of the (sequence, KV head) pair k / gpw, gpw =
// ceil(parts / W). It streams the partition's steps back to back through the
// step pipeline and writes the partition's (m, l, o = acc / l) partial, or
// the final rows of a one-partition sequence, straight from its registers:
// no LDS, no barrier. lse_merge combines the partials as for mfma_attn.
//
// Runs (run_parts > 1, when there are more partitions than wave slots):
// each pair's partitions are cut into runs of run_parts consecutive ones
// (the last run of a pair may be shorter), one wavefront per run, which
// streams its run as one step sequence, so the step pipeline stays full
// across partition boundaries (a partition's start would otherwise wait for its first loads,
// and its end for its last). At each boundary the finished partition's
// partial is parked in the wave's LDS slots (no global store inside the step
// loop, whose load waits count exactly) and the state starts over; the
// parked partials and the last one go to memory after the loop. Each
// partition is still computed on its own: the same partials as one wavefront
// per partition, bit for bit.
template <int D, int BS, int NT, bool STREAM, bool KV8, bool TREE, bool RUNS>
__global__ __launch_bounds__(256, NT == 1 ? 3 : 2) void mfma_attn_wave(AttnArgs a) {
  extern __shared__ float smem[];  // runs: [W][run_parts - 1][R][run_slot_row(D)] parked states
  const int W = blockDim.x / 64, wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int n = lane & 15, j = lane >> 4;
  const int R = a.group * a.q_len;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  // the partial of partition `part` of (b, g) from the state, or the final
  // rows of a one-partition sequence
  auto emit = [&](const WaveState<D, NT>& st, int b, int g, int part, bool final_rows) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float l = st.l[nt] + __shfl_xor(st.l[nt], 16);  // row sum: the 4 lanes of the row
      l += __shfl_xor(l, 32);
      const int r = nt * 16 + n;
      if (r >= R) continue;
      const int row = out_row(a, b, g, r);
      const int64_t pi = int64_t(row) * a.parts + part;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        f32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = st.poisoned ? NAN : (l > 0.f ? st.acc[nt][dt][k] / l : 0.f);
        const int c = 16 * dt + 4 * j;
        if (final_rows) {
#pragma unroll
          for (int k = 0; k < 4; ++k) store_f<uint16_t>(out + int64_t(row) * D + c + k, o[k]);
        } else {
          *reinterpret_cast<f32x4*>(a.part_o + pi * D + c) = o;
        }
      }
      if (!final_rows && j == 0) {
        a.part_ml[pi * 2 + 0] = st.poisoned ? NAN : st.m[nt];
        a.part_ml[pi * 2 + 1] = st.poisoned ? NAN : l;
      }
    }
  };
  if constexpr (!RUNS) {
    const int gpw = (a.parts + W - 1) / W;
    const int pair = blockIdx.x / gpw;
    const int part = (blockIdx.x % gpw) * W + wave;
    if (part >= a.parts) return;
    const int g = pair % a.hkv, b = pair / a.hkv;
    const int L = a.lens[b];
    if (L < a.q_len || L > a.max_ctx) {  // NaN rows: here for one partition, else by the merge kernel
      if (part == 0 && a.parts == 1)
        for (int e = lane; e < R * D; e += 64)
          store_f<uint16_t>(out + int64_t(out_row(a, b, g, e / D)) * D + e % D, NAN);
      return;
    }
    const int t0 = part * a.part_tokens;
    if (t0 >= L) return;  // past the sequence: the merge kernel reads only its partitions
    const int t1 = min(t0 + a.part_tokens, L);
    WaveState<D, NT> st;
    wave_state_init(st);
    mfma_wave_steps<D, BS, NT, STREAM, KV8, TREE>(a, b, g, L, t0 / kStep, (t1 + kStep - 1) / kStep, st,
                                                  [](int s) { return s + 1; });
    emit(st, b, g, part, L <= a.part_tokens);
    return;
  }
  // runs (partials, or the final rows of a one-partition sequence). A parked
  // partial keeps, per row, m, the 4 lanes' partial row sums, a poison flag
  // and the raw accumulator; the flush forms l and o = acc / l exactly as
  // emit does.
  constexpr int kSlotRow = run_slot_row(D);
  const int spp = a.part_tokens / kStep;  // steps per partition
  const int rpp = (a.parts + a.run_parts - 1) / a.run_parts;  // runs per pair
  const int64_t wid = int64_t(blockIdx.x) * W + wave;
  if (wid >= int64_t(a.num_seqs) * a.hkv * rpp) return;
  const int pair = int(wid / rpp);
  const int p0 = int(wid % rpp) * a.run_parts, p1 = min(a.parts, p0 + a.run_parts);  // partitions p0 .. p1 - 1
  float* slots = smem + int64_t(wave) * (a.run_parts - 1) * R * kSlotRow;
  {
    const int g = pair % a.hkv, b = pair / a.hkv;
    const int L = a.lens[b];
    if (L < a.q_len || L > a.max_ctx) return;  // NaN rows: by the merge kernel
    const int s0 = p0 * spp, s1 = min(p1 * spp, (L + kStep - 1) / kStep);
    if (s0 >= s1) return;  // partitions past the sequence
    WaveState<D, NT> st;
    wave_state_init(st);
    int parked = 0;
    int part_end = s0 + spp - 1;  // the last step of the partition in progress
    // a partition ends after step s: park its state, start the next one
    auto boundary = [&](int s) {
      if (s != part_end) return;
      part_end += spp;
      float* slot = slots + int64_t(parked) * R * kSlotRow;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + n;
        if (r >= R) continue;
        float* dst = slot + r * kSlotRow;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(dst + 8 + 16 * dt + 4 * j) = st.acc[nt][dt];
        dst[1 + j] = st.l[nt];
        if (j == 0) {
          dst[0] = st.m[nt];
          dst[5] = st.poisoned ? 1.f : 0.f;
        }
      }
      ++parked;
      wave_state_init(st);
    };
    mfma_wave_steps<D, BS, NT, STREAM, KV8, TREE>(a, b, g, L, s0, s1, st, [](int s) { return s + 1; }, boundary);
    emit(st, b, g, (s1 - 1) / spp, L <= a.part_tokens);  // a one-partition sequence: its final rows
    for (int i = 0; i < parked; ++i) {  // the parked partials, partitions p0, p0 + 1, ...
      const float* slot = slots + int64_t(i) * R * kSlotRow;
      for (int e = lane; e < R * (D / 4); e += 64) {
        const int r = e / (D / 4), c = 4 * (e % (D / 4));
        const float* row = slot + r * kSlotRow;
        const float l = (row[1] + row[2]) + (row[3] + row[4]);  // as emit sums the 4 lanes
        const bool bad = row[5] != 0.f;
        const f32x4 acc = *reinterpret_cast<const f32x4*>(row + 8 + c);
        f32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = bad ? NAN : (l > 0.f ? acc[k] / l : 0.f);
        const int64_t pi = int64_t(out_row(a, b, g, r)) * a.parts + p0 + i;
        *reinterpret_cast<f32x4*>(a.part_o + pi * D + c) = o;
        if (c == 0) {
          a.part_ml[pi * 2 + 0] = bad ? NAN : row[0];
          a.part_ml[pi * 2 + 1] = bad ? NAN : l;
        }
      }
    }
  }
}

// Balanced schedule. The work of the batch is the list of segments
// s = b * H_kv + g, each ceil(L_b / 32) steps long, laid end to end; the grid
// (sized to the resident capacity) splits that list into equal contiguous
// ranges, one per workgroup. The part of a segment inside one workgroup's
// range is a piece; a segment covered by one piece is written directly,
// otherwise every piece writes (m, l, o) partials at index
// (workgroup + segment) and the workgroup that completes a segment's last
// piece, by an atomic arrival count per segment, merges them.
__device__ __forceinline__ int64_t range_start(int64_t k, int64_t S, int64_t N) { return k * S / N; }

// workgroup whose range contains position x (0 <= x < S)
__device__ __forceinline__ int64_t owner(int64_t x, int64_t S, int64_t N) {
  int64_t k = x * N / S;
  while (k + 1 < N && range_start(k + 1, S, N) <= x) ++k;
  while (k > 0 && range_start(k, S, N) > x) --k;
  return k;
}

constexpr int kMergeBatch = 8;   // pieces whose partial loads a thread has in flight at once
// What a workgroup spends on a segment beyond its steps (the first step's
// loads in flight, and at its end parking, combining and storing the rows)
// is counted as work by the balanced partition, in steps (Plan::seg_cost),
// so that ranges holding many short segments get fewer steps.
constexpr int kMinGroupSteps = 8;  // fewest steps a workgroup's range holds
constexpr int kXcds = 8;           // accelerator complex dies (each with its own L2)

// The workgroup that completed a segment merges its npieces partials, which
// start at piece p0 (log-sum-exp identity: out = sum_p w_p o_p / sum_p w_p
// with w_p = l_p 2^(m_p - M), M = max_p m_p). Each thread owns 4-column
// chunks of the output rows and folds the pieces into a running (max, sum,
// weighted o) in piece order; the (m, l) and o loads of kMergeBatch pieces
// are issued together, so a merge of up to kMergeBatch pieces costs one
// round trip to memory. out0: the segment's first output row.
template <int D>
__device__ void merge_pieces(const AttnArgs& a, int64_t p0, int npieces, int R, uint16_t* out0) {
  // The opaque copy keeps the thread-index arithmetic below inside this
  // function: hoisted out of the caller's loop it would stay live across
  // the attention steps and cost registers there.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int T = blockDim.x;
  const auto ml_r = partial_rsrc(a.part_ml + p0 * R * 2, uint32_t(npieces) * R * 8);
  const auto o_r = partial_rsrc(a.part_o + p0 * R * D, uint32_t(npieces) * R * D * 4);
  const int nc = R * D / 4;
  for (int ch = tid; ch < nc; ch += T) {
    const int r = ch / (D / 4), c = 4 * (ch % (D / 4));
    float M = -INFINITY, den = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int pb = 0; pb < npieces; pb += kMergeBatch) {
      // loads past the last piece fall outside the buffer range and read 0
      f32x2 ml[kMergeBatch];
      f32x4 o[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        ml[u] = load2_coherent(ml_r, uint32_t((pb + u) * R + r) * 8);
        o[u] = load4_coherent(o_r, uint32_t(((pb + u) * R + r) * D + c) * 4);
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        if (pb + u < npieces) {
          const float m = ml[u][0], l = ml[u][1];
          const float m_new = fmaxf(M, m);
          const float mu = m_new == -INFINITY ? 0.f : m_new;
          const float f_old = fast_exp2(M - mu), w = l * fast_exp2(m - mu);
          den = den * f_old + w;
          acc = acc * f_old + w * o[u];
          M = m_new;
        }
      }
    }
    const int i = r / a.group, hh = r % a.group;  // drafted token, head within the group
    uint16_t* dst = out0 + (int64_t(i) * a.hq + hh) * D + c;
#pragma unroll
    for (int u = 0; u < 4; ++u) store_f<uint16_t>(dst + u, den > 0.f ? acc[u] / den : NAN);
  }
}

// Resident waves per compute unit for NT row tiles (registers allow three
// waves per SIMD with one tile, two with two).
constexpr int balanced_waves(int nt) { return nt == 1 ? 12 : 8; }

template <int D, int BS, int NT, bool STREAM, bool KV8, bool TREE>
__global__ __launch_bounds__(64 * balanced_waves(NT)) void mfma_attn_balanced(AttnArgs a) {
  extern __shared__ float smem[];  // [B+1] step prefix sums, then the parked states
  const int W = blockDim.x / 64, wave = threadIdx.x / 64;
  const int R = a.group * a.q_len;
  const int B = a.num_seqs;
  int32_t* pre = reinterpret_cast<int32_t*>(smem);
  float* park = smem + ((B + 1 + 3) & ~3);
  // steps per sequence (0 for an out-of-range length) and their prefix sums:
  // thread t owns a contiguous chunk of sequences; chunk totals are scanned
  // across the workgroup with wave shuffles and per-wave totals in LDS
  {
    const int T = blockDim.x, tid = threadIdx.x;
    const int chunk = (B + T - 1) / T;
    const int b0 = min(B, tid * chunk), b1 = min(B, b0 + chunk);
    // work units of each of the sequence's segments: its steps plus the
    // cost of starting it (0 for an out-of-range length)
    auto steps_of = [&](int b) {
      const int L = a.lens[b];
      return (L < a.q_len || L > a.max_ctx) ? 0 : (L + kStep - 1) / kStep + a.seg_cost;
    };
    int local = 0;
    for (int b = b0; b < b1; ++b) local += steps_of(b);
    int incl = local;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if ((tid & 63) >= o) incl += v;
    }
    __shared__ int wave_tot[16];  // one per wavefront (at most 1024 threads)
    if ((tid & 63) == 63) wave_tot[tid >> 6] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < (tid >> 6); ++w) run += wave_tot[w];
    for (int b = b0; b < b1; ++b) {
      pre[b] = run;
      run += steps_of(b);
    }
    if (b1 == B && b0 < b1) pre[B] = run;
    if (B <= tid * chunk && tid == 0) pre[B] = 0;
    __syncthreads();
  }
  // Units in head-major order: KV head g's segments fill [g P, (g + 1) P),
  // P = pre[B], sequence b's segment [g P + pre[b], g P + pre[b + 1]).
  // Segments are numbered in the same order (seg = g B + b) for the arrival
  // counters and the partials.
  const int64_t P = pre[B];
  const int64_t S = P * a.hkv;
  // sequences with an out-of-range length: NaN rows, spread over the grid
  for (int b = int(blockIdx.x); b < B; b += int(gridDim.x)) {
    const int L = a.lens[b];
    if (L < a.q_len || L > a.max_ctx)
      for (int e = threadIdx.x; e < a.q_len * a.hq * D; e += blockDim.x)
        store_f<uint16_t>(static_cast<uint16_t*>(a.out) + int64_t(b) * a.q_len * a.hq * D + e, NAN);
  }
  // With no more workgroups than steps every range is non-empty, so the
  // pieces of a segment are exactly the workgroups from its first owner to
  // its last.
  const int64_t N = min(int64_t(gridDim.x), (S + kMinGroupSteps - 1) / kMinGroupSteps);
  if (int64_t(blockIdx.x) >= N) return;
  // Range k of workgroup blockIdx.x. Workgroups go to the XCDs in turn
  // (workgroup i to XCD i mod kXcds): with N a multiple of kXcds, each XCD
  // takes N / kXcds consecutive ranges, i.e. whole KV heads, so that blocks
  // several sequences share (a common prompt) are fetched into its L2 once
  // and then read there by the XCD's other workgroups.
  const int64_t k = N % kXcds == 0 ? int64_t(blockIdx.x % kXcds) * (N / kXcds) + blockIdx.x / kXcds
                                   : int64_t(blockIdx.x);
  const int64_t x0 = range_start(k, S, N), x1 = range_start(k + 1, S, N);
  // the head and the first sequence whose segment reaches past x0
  int g = int(x0 / P), b = 0;
  {
    const int64_t xr = x0 - int64_t(g) * P;
    int lo = 0, hi = B - 1;  // largest b with pre[b] <= xr
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (pre[mid] <= xr) lo = mid; else hi = mid - 1;
    }
    b = lo;
  }
  __shared__ int64_t duty_seg[2], duty_p0[2];
  __shared__ int duty_n[2];
  __shared__ int n_duty;
  if (threadIdx.x == 0) n_duty = 0;
  __syncthreads();
  // A segment occupies seg_cost units for its start, then one unit per
  // step; a range holds the steps of the units it covers (possibly none of
  // a segment whose start units it ends in).
  int64_t x = x0;
  while (x < x1) {
    if (b >= B) {  // on to the next head
      ++g;
      b = 0;
      continue;
    }
    const int nu = pre[b + 1] - pre[b];  // units of sequence b's segment
    const int64_t seg_start = int64_t(g) * P + pre[b], seg_end = seg_start + nu;
    if (nu == 0 || seg_end <= x) { ++b; continue; }
    const int64_t real_start = seg_start + a.seg_cost;  // unit of the segment's first step
    const int nb = nu - a.seg_cost;
    if (min(x1, seg_end) <= real_start) { x = min(x1, seg_end); continue; }  // only start units here
    const int first = int(max(x, real_start) - real_start), last = int(min(x1, seg_end) - real_start);
    const int L = a.lens[b];
    WaveState<D, NT> st;
    wave_state_init(st);
    mfma_wave_steps<D, BS, NT, STREAM, KV8, TREE>(a, b, g, L, first + wave, last, st,
                                                  [W](int s) { return s + W; });
    const bool bad = park_states(st, R, park);
    const int64_t seg = int64_t(g) * B + b;
    const bool whole = first == 0 && last == nb;
    uint16_t* out = static_cast<uint16_t*>(a.out);
    __shared__ float wt[kMfmaMaxRows * 16], row_ml[kMfmaMaxRows * 2];  // per-row wave weights, (M, l)
    park_row_weights(park, W, R, wt, row_ml);
    if (whole) {  // the rows, 4 columns (8 bytes) per store
      for (int e = threadIdx.x; e < R * D / 4; e += blockDim.x) {
        const int r = e / (D / 4), c = 4 * (e % (D / 4));
        const f32x4 o = park_chunk(park, W, R, D, wt, r, c);
        const u32x2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(out + int64_t(out_row(a, b, g, r)) * D + c) =
            bad ? (u32x2){0x7fc07fc0u, 0x7fc07fc0u} : packed;
      }
    } else {
      const int64_t piece = k + seg;
      // this piece's (m, l) per row and o per row, 4 columns per store
      const auto ml_r = partial_rsrc(a.part_ml + piece * R * 2, uint32_t(R) * 8);
      const auto o_r = partial_rsrc(a.part_o + piece * R * D, uint32_t(R) * D * 4);
      for (int e = threadIdx.x; e < R * D / 4; e += blockDim.x) {
        const int r = e / (D / 4), c = 4 * (e % (D / 4));
        f32x4 v = park_chunk(park, W, R, D, wt, r, c);
        if (bad) v = (f32x4){NAN, NAN, NAN, NAN};
        store4_coherent(o_r, uint32_t(r * D + c) * 4, v);
        if (c == 0)
          store2_coherent(ml_r, uint32_t(r) * 8, bad ? (f32x2){NAN, NAN} : (f32x2){row_ml[2 * r], row_ml[2 * r + 1]});
      }
      // Every wave waits until its partial stores are complete at the
      // coherent level, then one thread counts the piece in. The workgroup
      // that brings the count to the number of pieces read the others'
      // partials after seeing their increments, and merges.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const int64_t k_first = owner(real_start, S, N), k_last = owner(seg_end - 1, S, N);
      const int npieces = int(k_last - k_first + 1);
      __shared__ int arrived;
      if (threadIdx.x == 0)
        arrived = __hip_atomic_fetch_add(&a.counters[seg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (arrived == npieces - 1 && threadIdx.x == 0) {  // this workgroup merges the segment
        duty_seg[n_duty] = seg;
        duty_p0[n_duty] = k_first + seg;
        duty_n[n_duty] = npieces;
        ++n_duty;
      }
    }
    __syncthreads();  // the park area is reused by the next piece
    x = real_start + last;
  }
  // Merges after the steps (only a range's first and last piece can be
  // partial, so at most two), kept out of the step loop's registers.
  for (int d = 0; d < n_duty; ++d) {
    const int64_t seg = duty_seg[d];
    const int bb = int(seg % B), gg = int(seg / B);
    merge_pieces<D>(a, duty_p0[d], duty_n[d], R,
                    static_cast<uint16_t*>(a.out) + int64_t(out_row(a, bb, gg, 0)) * D);
    if (threadIdx.x == 0)  // ready for the next call
      __hip_atomic_store(&a.counters[seg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// VALU kernel (f32 or bf16)
// ---------------------------------------------------------------------------
// Per 64-token step: lane l computes the scores of token tb + l for every
// query row (query rows broadcast from LDS), the wave reduces the step maximum
// per row, probabilities go through LDS, and lane l then accumulates head-dim
// elements l and l + 64 of every row over the step's tokens from the V^T
// slices (16-byte loads of adjacent tokens).
// bf16: both contractions use v_dot2_f32_bf16 on packed pairs: q.k on the raw
// bf16 pairs of q (LDS) and of the K row (no unpacking), P.V on pairs of
// adjacent tokens, with the probabilities rounded to bf16 (the row sum uses
// the rounded values). f32: plain FMAs.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

template <typename T, int D, int BS>
__global__ __launch_bounds__(256) void valu_attn(AttnArgs a) {
  constexpr bool BF = sizeof(T) == 2;
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

  // LDS: q_s (f32: [RM][D] pre-scaled; bf16: [RM][D/2] raw pairs) | p_s per
  // wave (f32: [RM][64] floats; bf16: [RM][64] bf16); the merge reuses it all
  float* q_s = smem;
  float* p_s = q_s + RM * D;
  const uint32_t* q2 = reinterpret_cast<const uint32_t*>(q_s);
  if constexpr (BF) {
    uint32_t* qw = reinterpret_cast<uint32_t*>(q_s);
    for (int e = threadIdx.x; e < RM * D / 2; e += blockDim.x) {
      const int r = e / (D / 2), c2 = e % (D / 2);
      uint32_t v = 0;
      if (r < R) {
        const int i = r / a.group, h = t.g * a.group + r % a.group;
        v = reinterpret_cast<const uint32_t*>(q + (int64_t(t.b * a.q_len + i) * a.hq + h) * D)[c2];
      }
      qw[e] = v;
    }
  } else {
    for (int e = threadIdx.x; e < RM * D; e += blockDim.x) {
      const int r = e / D, c = e % D;
      float v = 0.f;
      if (r < R) {
        const int i = r / a.group, h = t.g * a.group + r % a.group;
        v = load_f<T>(q + (int64_t(t.b * a.q_len + i) * a.hq + h) * D + c) * a.scale_log2;
      }
      q_s[e] = v;
    }
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
  uint32_t vbits[RM];  // drafted positions each row sees
#pragma unroll
  for (int r = 0; r < RM; ++r) vbits[r] = row_mask(a, t.b, min(r, R - 1) / a.group);
  const int ctx_end = t.L - a.q_len;
  float* pw = p_s + wave * RM * 64;                              // f32 probabilities
  uint16_t* pwh = reinterpret_cast<uint16_t*>(pw);               // bf16 probabilities
  const uint32_t* pw2 = reinterpret_cast<const uint32_t*>(pw);   // ... as token pairs
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
      // K slice: 32-element head-dim slabs, each [bs][32]
      const T* krow = kp + (int64_t(blk) * a.hkv + t.g) * head_stride + (tok % BS) * 32;
      for (int c0 = 0; c0 < D; c0 += VEC) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(krow + (c0 / 32) * (BS * 32) + c0 % 32);
        if constexpr (BF) {
#pragma unroll
          for (int r = 0; r < RM; ++r) {
            if (r < R) {
              const u32x4 qq = *reinterpret_cast<const u32x4*>(q2 + r * (D / 2) + c0 / 2);
#pragma unroll
              for (int e = 0; e < 4; ++e) sc[r] = dot2_bf16(qq[e], raw[e], sc[r]);
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < RM; ++r) {
            if (r < R) {
#pragma unroll
              for (int e = 0; e < VEC; ++e) sc[r] = fmaf(q_s[r * D + c0 + e], __uint_as_float(raw[e]), sc[r]);
            }
          }
        }
      }
      if constexpr (BF) {
#pragma unroll
        for (int r = 0; r < RM; ++r) sc[r] *= a.scale_log2;
      }
    }
    // online softmax per row over the step
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r >= R) continue;
      const int off = tok - ctx_end;
      const bool vis = off < 0 || ((vbits[r] >> (off & 31)) & 1u);
      const float v = (in && blk_ok && vis) ? sc[r] : -INFINITY;
      float mx = v;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_new = fmaxf(m_run[r], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[r] - m_use);
      float pr = fast_exp2(v - m_use);
      if constexpr (BF) {
        const uint16_t pb = f_to_bf16(pr);
        pwh[r * 64 + lane] = pb;
        pr = bf16_to_f(pb);   // the row sum uses the rounded weight
      } else {
        pw[r * 64 + lane] = pr;
      }
      m_run[r] = m_new;
      l_run[r] = l_run[r] * alpha + pr;   // lane-partial sum, reduced at the end
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[r][k] *= alpha;
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
          u32x4 raw = *reinterpret_cast<const u32x4*>(vrow + u0);
          if constexpr (BF) {
            // tokens past the context keep their pool bytes (NaN in tests): zero them
            const int valid = cnt - u0;
            if (valid < 8) {
#pragma unroll
              for (int w4 = 0; w4 < 4; ++w4)
                raw[w4] &= (2 * w4 + 1 < valid) ? 0xffffffffu : (2 * w4 < valid ? 0x0000ffffu : 0u);
            }
#pragma unroll
            for (int r = 0; r < RM; ++r) {
              if (r < R) {
                const u32x4 pp = *reinterpret_cast<const u32x4*>(pw2 + r * 32 + (kb * BS + u0) / 2);
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) acc[r][k] = dot2_bf16(pp[w4], raw[w4], acc[r][k]);
              }
            }
          } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              if (u0 + e < cnt) {
                const int tt = kb * BS + u0 + e;
                const float vv = __uint_as_float(raw[e]);
#pragma unroll
                for (int r = 0; r < RM; ++r)
                  if (r < R) acc[r][k] = fmaf(pw[r * 64 + tt], vv, acc[r][k]);
              }
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
// One workgroup of kMergeWaves wavefronts per output row of a sequence that
// has more than one partition: M = max_p m_p, w_p = l_p 2^(m_p - M),
// out = sum_p w_p o_p / sum_p w_p. Wave w takes partitions w, w+4, ...; each
// lane holds D/64 head-dim elements; the waves' sums meet in LDS.
constexpr int kMergeWaves = 4;

template <typename T, int D>
__global__ __launch_bounds__(256) void lse_merge(AttnArgs a) {
  constexpr int DPL = D / 64;
  __shared__ float red_m[kMergeWaves];
  __shared__ float red_o[kMergeWaves][D + 1];
  const int row = blockIdx.x;
  const int b = row / (a.q_len * a.hq);
  const int L = a.lens[b];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  T* out = static_cast<T*>(a.out) + int64_t(row) * D;
  if (L < a.q_len || L > a.max_ctx) {
    for (int c = threadIdx.x; c < D; c += blockDim.x) store_f<T>(out + c, NAN);
    return;
  }
  const int np = (L + a.part_tokens - 1) / a.part_tokens;
  if (np == 1) return;  // written by the partition kernel
  const float* ml = a.part_ml + int64_t(row) * a.parts * 2;
  const float* po = a.part_o + int64_t(row) * a.parts * D;
  // global maximum over the partitions
  float mx = -INFINITY;
  for (int p = threadIdx.x; p < np; p += blockDim.x) mx = fmaxf(mx, ml[2 * p]);
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red_m[wave] = mx;
  __syncthreads();
  float M = red_m[0];
  for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, red_m[w]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  // weighted sums; four partitions in flight per wave
  float acc[DPL], wsum = 0.f;
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  int p = wave;
  for (; p + 3 * kMergeWaves < np; p += 4 * kMergeWaves) {
    float w4[4], o4[4][DPL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pu = p + u * kMergeWaves;
      w4[u] = ml[2 * pu + 1] * fast_exp2(ml[2 * pu] - Mu);
#pragma unroll
      for (int k = 0; k < DPL; ++k) o4[u][k] = po[int64_t(pu) * D + lane + 64 * k];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wsum += w4[u];
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[k] = fmaf(w4[u], o4[u][k], acc[k]);
    }
  }
  for (; p < np; p += kMergeWaves) {
    const float w = ml[2 * p + 1] * fast_exp2(ml[2 * p] - Mu);
    wsum += w;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = fmaf(w, po[int64_t(p) * D + lane + 64 * k], acc[k]);
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) red_o[wave][lane + 64 * k] = acc[k];
  if (lane == 0) red_o[wave][D] = wsum;
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int w = 0; w < kMergeWaves; ++w) {
      num += red_o[w][c];
      den += red_o[w][D];
    }
    store_f<T>(out + c, den > 0.f ? num / den : NAN);
  }
}

// ---------------------------------------------------------------------------
// Host side: validation, planning, launch
// ---------------------------------------------------------------------------
struct Plan {
  int path, sched, part_tokens, parts, waves, grid, merge_grid, nt, rows;
  bool stream;  // K/V loads with the non-temporal hint
  bool kv8;     // FP8 pools
  bool tree;    // per-row visibility masks over the drafted positions
  int64_t segments, pieces;  // balanced schedule: segments, partial slots
  int seg_cost;              // balanced schedule: a segment start's cost in steps
  int run_parts = 1;         // one wavefront per partition: consecutive partitions per wavefront
  // Workspace layout, the same for every schedule: the balanced schedule's
  // arrival counters (ws_counters bytes, reserved by every layout so that no
  // other schedule ever writes them), then the partials: (m, l) pairs at
  // offset 0 of the partial area, o from offset ws_o_off.
  size_t ws_counters, ws_o_off, ws_partials;
  size_t ws;  // total: ws_counters + ws_partials, or 0 when nothing is split
};

constexpr int kMaxBalancedSeqs = 8192;  // step prefix sums live in LDS
constexpr int kWavesPerCu = 12;          // resident waves of the one-tile MFMA kernels (3 per SIMD)

int ceil_div(int64_t x, int64_t y) { return int((x + y - 1) / y); }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr size_t kMaxLdsBytes = 160 * 1024;  // LDS of one compute unit (gfx950)
constexpr size_t kStaticLdsReserve = 4096;    // the kernels' fixed __shared__ arrays
constexpr int kPerCuMinContext = 2048;  // one workgroup per CU once the longest context reaches this

size_t lds_bytes(const Plan& pl, int D, int num_seqs) {
  if (pl.path == PA_PATH_MFMA) {
    const size_t park = size_t(pl.waves) * pl.rows * (D + 2 + kParkPad) * sizeof(float);
    // runs: each wave's parked partials
    if (pl.sched == PA_SCHED_PARTITIONS_WAVE)
      return size_t(pl.waves) * (pl.run_parts - 1) * pl.rows * run_slot_row(D) * sizeof(float);
    if (pl.sched == PA_SCHED_PARTITIONS) return park;
    return size_t((num_seqs + 1 + 3) & ~3) * sizeof(int32_t) + park;  // step prefix sums, then the park area
  }
  const size_t first = size_t(kValuMaxRows) * D + size_t(pl.waves) * kValuMaxRows * 64;
  const size_t merge = size_t(pl.waves) * kValuMaxRows * (D + 2);
  return std::max(first, merge) * sizeof(float);
}

// Default wavefronts per workgroup. Balanced schedule: one workgroup of 8
// waves per compute unit, so the compute unit's waves share one range
// (workgroups dispatched earlier on a compute unit otherwise run ahead of the
// later ones and finish early); with one row tile the registers would allow
// 12 resident waves, but 8 measure faster (the 70B layer by 1%), except where
// measurement favours smaller workgroups: contexts shorter than
// kPerCuMinContext tokens (many segment boundaries, where all of a
// workgroup's waves wait for its slowest one) and the FP8 two-tile step (two
// workgroups of four waves keep its conversions busier than one of eight).
int default_waves(const Plan& pl, int max_context) {
  if (pl.sched != PA_SCHED_BALANCED || max_context < kPerCuMinContext) return 4;
  if (pl.nt == 2 && pl.kv8) return 4;
  return 8;
}

// Cost of starting a segment in the balanced partition, in steps (the
// measured optimum per pool format: an FP8 step moves half the bytes, so a
// boundary weighs more steps).
int default_segment_cost(const Plan& pl) {
  return pl.kv8 ? 16 : 8;
}

// Compute units of the current device, queried once per device and kept
// (kMaxCUs when no device can be queried). Used to size partitions; the
// workspace bound does not depend on it.
constexpr int kMaxDevices = 64;
int device_cus() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kMaxCUs;
  }
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return kMaxCUs;
  }
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

pa_status make_plan(const pa_attn_desc* d, int32_t q_len, Plan* pl) {
  if (!d || !pl) return PA_ERR_INVALID_ARG;
  for (int k = 0; k < 2; ++k)
    if (d->reserved[k] != 0) return PA_ERR_INVALID_ARG;
  if (d->kv_shared != 0 && d->kv_shared != 1) return PA_ERR_INVALID_ARG;
  if (d->kv_format != PA_KV_SAME && d->kv_format != PA_KV_FP8_E4M3) return PA_ERR_INVALID_ARG;
  if (d->waves_per_group != 0 && d->waves_per_group != 1 && d->waves_per_group != 2 &&
      d->waves_per_group != 4 && d->waves_per_group != 8 && d->waves_per_group != 12)
    return PA_ERR_INVALID_ARG;
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
    if (d->kv_format == PA_KV_FP8_E4M3) return PA_ERR_UNSUPPORTED;  // FP8 pools: MFMA path only
  } else {
    return PA_ERR_INVALID_ARG;
  }
  if (d->kv_format == PA_KV_FP8_E4M3 && d->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  const int64_t pairs = int64_t(d->num_seqs) * d->num_kv_heads;
  const int64_t out_rows = int64_t(d->num_seqs) * q_len * d->num_q_heads;
  if (out_rows > INT32_MAX) return PA_ERR_UNSUPPORTED;
  pl->path = path;
  pl->nt = rows > 16 ? 2 : 1;
  pl->rows = int(rows);
  pl->stream = d->kv_shared == 0;
  pl->kv8 = d->kv_format == PA_KV_FP8_E4M3;
  pl->tree = false;  // set by the tree entry point
  const bool balanced = path == PA_PATH_MFMA && d->partition_tokens == 0 &&
                        d->num_seqs <= kMaxBalancedSeqs;
  pl->sched = balanced ? PA_SCHED_BALANCED : PA_SCHED_PARTITIONS;
  const int max_waves = balanced ? balanced_waves(pl->nt) : 4;
  if (d->waves_per_group > max_waves) return PA_ERR_UNSUPPORTED;
  pl->waves = d->waves_per_group ? d->waves_per_group : default_waves(*pl, d->max_context);
  while (lds_bytes(*pl, d->head_dim, d->num_seqs) > kMaxLdsBytes - kStaticLdsReserve) {
    if (d->waves_per_group || pl->waves == 1) return PA_ERR_UNSUPPORTED;
    pl->waves = pl->waves > 4 ? 4 : pl->waves / 2;
  }
  const int waves = pl->waves;
  if (balanced) {
    // grid = resident capacity; the workspace is sized for the largest one
    // (every compute unit full of single-workgroup waves)
    const int64_t grid_max = int64_t(kMaxCUs) * std::max(1, 32 / waves);
    pl->part_tokens = 0;
    pl->parts = 0;
    pl->grid = int(grid_max);
    pl->merge_grid = 0;
    pl->segments = pairs;
    pl->pieces = grid_max + pairs;
    pl->seg_cost = default_segment_cost(*pl);
    pl->ws_counters = align256(size_t(pairs) * sizeof(int32_t));
    pl->ws_o_off = align256(size_t(pl->pieces) * rows * 2 * sizeof(float));
    pl->ws_partials = pl->ws_o_off + size_t(pl->pieces) * rows * d->head_dim * sizeof(float);
    pl->ws = pl->ws_counters + pl->ws_partials;
    return PA_OK;
  }
  const int cus = device_cus();
  int pt = d->partition_tokens;
  if (pt == 0) {
    // enough waves for two full rounds of the kernel's occupancy (the VALU
    // kernel runs 16 waves per compute unit; the MFMA one 12), partitions of
    // at least 256 tokens
    const int64_t target = int64_t(cus) * (path == PA_PATH_VALU ? 32 : 24);
    const int64_t want = (target + pairs * waves - 1) / (pairs * waves);
    const int max_parts = std::max(1, ceil_div(d->max_context, 256));
    const int parts = int(std::min<int64_t>(std::max<int64_t>(want, 1), max_parts));
    pt = ceil_div(ceil_div(d->max_context, parts), 64) * 64;
  }
  const int parts = ceil_div(d->max_context, pt);
  if (parts > kMaxPartitions) return PA_ERR_UNSUPPORTED;
  // MFMA path with enough partitions to fill every wave slot of the device
  // (3 per SIMD) on their own: one wavefront per partition, which streams the
  // partition without waiting for other waves and writes its partial from
  // registers; with fewer, the waves of a workgroup share a partition.
  if (path == PA_PATH_MFMA && pairs * parts >= int64_t(cus) * kWavesPerCu) pl->sched = PA_SCHED_PARTITIONS_WAVE;
  int64_t grid = pl->sched == PA_SCHED_PARTITIONS_WAVE ? pairs * ceil_div(parts, waves) : pairs * parts;
  // More partitions than resident waves: runs of consecutive partitions per
  // wave, so that every wave is resident from the start and its step
  // pipeline runs on across partition boundaries. A run parks all but its
  // last partial in LDS: the run is as long as full occupancy leaves room for.
  pl->run_parts = 1;
  if (pl->sched == PA_SCHED_PARTITIONS_WAVE && parts > 1 && pt % kStep == 0) {
    const int per_cu = pl->nt == 1 ? kWavesPerCu : balanced_waves(2);
    const int64_t total = pairs * parts;
    const size_t slot = size_t(rows) * run_slot_row(d->head_dim) * sizeof(float);
    const int kmax = 1 + int((kMaxLdsBytes - kStaticLdsReserve) / (size_t(per_cu) * slot));
    const int k = std::min<int64_t>(kmax, (total + int64_t(cus) * per_cu - 1) / (int64_t(cus) * per_cu));
    if (k > 1) {
      pl->run_parts = k;
      grid = (pairs * ceil_div(parts, k) + waves - 1) / waves;
    }
  }
  if (grid > INT32_MAX) return PA_ERR_UNSUPPORTED;
  pl->part_tokens = pt;
  pl->parts = parts;
  pl->grid = int(grid);
  pl->merge_grid = parts > 1 ? int(out_rows) : 0;
  pl->segments = 0;
  pl->pieces = 0;
  // partials: (m, l) per row and partition, then o (from a 256-byte boundary,
  // 16-byte stores), after the counter area of the balanced schedule, which
  // this schedule leaves untouched
  if (parts > 1) {
    pl->ws_counters = align256(size_t(pairs) * sizeof(int32_t));
    pl->ws_o_off = align256(size_t(out_rows) * parts * 2 * sizeof(float));
    pl->ws_partials = pl->ws_o_off + size_t(out_rows) * parts * d->head_dim * sizeof(float);
  } else {
    pl->ws_counters = pl->ws_o_off = pl->ws_partials = 0;
  }
  pl->ws = pl->ws_counters + pl->ws_partials;
  return PA_OK;
}


// Workgroups of `kernel` that fit on the device at once (0 if unknown). The
// occupancy query runs once per (kernel, threads, LDS bytes, device); later
// calls read the kept answer.
int resident_groups(const void* kernel, int threads, size_t lds) {
  struct Entry { const void* kernel; int threads; size_t lds; int dev, per_cu; };
  static std::mutex mu;
  static Entry seen[256];
  static int n_seen = 0, next_slot = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int cus = device_cus();
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_seen; ++i)
      if (seen[i].kernel == kernel && seen[i].threads == threads && seen[i].lds == lds && seen[i].dev == dev)
        return seen[i].per_cu * cus;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  std::lock_guard<std::mutex> lock(mu);
  seen[next_slot] = Entry{kernel, threads, lds, dev, per_cu};  // a full table recycles its oldest entry
  next_slot = (next_slot + 1) % 256;
  n_seen = std::min(n_seen + 1, 256);
  return per_cu * cus;
}

// The main kernel a plan launches (one template instance per shape; sched is
// the plan's schedule, or kSchedRuns for one wavefront per partition in runs).
constexpr int kSchedRuns = -1;
template <int D, int BS, int NT, bool STREAM, bool KV8, bool TREE>
const void* mfma_kernel(int sched) {
  if (sched == PA_SCHED_BALANCED) return reinterpret_cast<const void*>(mfma_attn_balanced<D, BS, NT, STREAM, KV8, TREE>);
  if (sched == PA_SCHED_PARTITIONS_WAVE) return reinterpret_cast<const void*>(mfma_attn_wave<D, BS, NT, STREAM, KV8, TREE, false>);
  if (sched == kSchedRuns) return reinterpret_cast<const void*>(mfma_attn_wave<D, BS, NT, STREAM, KV8, TREE, true>);
  return reinterpret_cast<const void*>(mfma_attn<D, BS, NT, STREAM, KV8, TREE>);
}

template <int D, int BS, int NT, bool TREE>
const void* mfma_kernel(const Plan& pl) {
  const int sc = pl.sched == PA_SCHED_PARTITIONS_WAVE && pl.run_parts > 1 ? kSchedRuns : pl.sched;
  if (pl.kv8)
    return pl.stream ? mfma_kernel<D, BS, NT, true, true, TREE>(sc) : mfma_kernel<D, BS, NT, false, true, TREE>(sc);
  return pl.stream ? mfma_kernel<D, BS, NT, true, false, TREE>(sc) : mfma_kernel<D, BS, NT, false, false, TREE>(sc);
}

template <int D, int BS, int NT>
const void* mfma_kernel(const Plan& pl) {
  return pl.tree ? mfma_kernel<D, BS, NT, true>(pl) : mfma_kernel<D, BS, NT, false>(pl);
}

template <int D, int BS>
const void* main_kernel(const Plan& pl, int dtype) {
  if (pl.path == PA_PATH_MFMA) return pl.nt == 1 ? mfma_kernel<D, BS, 1>(pl) : mfma_kernel<D, BS, 2>(pl);
  return dtype == PA_DTYPE_F32 ? reinterpret_cast<const void*>(valu_attn<float, D, BS>)
                               : reinterpret_cast<const void*>(valu_attn<uint16_t, D, BS>);
}

const void* main_kernel_for(const Plan& pl, int dtype, int D, int BS) {
  if (D == 64) return BS == 16 ? main_kernel<64, 16>(pl, dtype) : main_kernel<64, 32>(pl, dtype);
  return BS == 16 ? main_kernel<128, 16>(pl, dtype) : main_kernel<128, 32>(pl, dtype);
}

// Workgroups the main kernel is launched with: for the balanced schedule the
// device's resident capacity for that kernel (capped by the plan's bound).
int launch_grid(const Plan& pl, const pa_attn_desc* d) {
  if (pl.sched != PA_SCHED_BALANCED) return pl.grid;
  const void* k = main_kernel_for(pl, d->dtype, d->head_dim, d->block_size);
  const int fit = resident_groups(k, 64 * pl.waves, lds_bytes(pl, d->head_dim, d->num_seqs));
  return std::max(1, std::min(pl.grid, fit > 0 ? fit : pl.grid));
}

pa_status launch_main(const Plan& pl, const pa_attn_desc* d, const AttnArgs& args, hipStream_t s) {
  const void* k = main_kernel_for(pl, d->dtype, d->head_dim, d->block_size);
  const size_t lds = lds_bytes(pl, d->head_dim, d->num_seqs);
  const int grid = launch_grid(pl, d);
  void* kargs[] = {const_cast<AttnArgs*>(&args)};
  if (const hipError_t e = hipLaunchKernel(k, dim3(grid), dim3(64 * pl.waves), kargs, lds, s); e != hipSuccess) {
    (void)hipGetLastError();
    return pa::hip_failed(e);
  }
  return PA_OK;
}

template <int D>
pa_status launch_merge(const Plan& pl, int dtype, const AttnArgs& args, hipStream_t s) {
  const dim3 block(64 * kMergeWaves);
  if (dtype == PA_DTYPE_F32)
    hipLaunchKernelGGL((lse_merge<float, D>), dim3(pl.merge_grid), block, 0, s, args);
  else
    hipLaunchKernelGGL((lse_merge<uint16_t, D>), dim3(pl.merge_grid), block, 0, s, args);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : pa::hip_failed(e);
}

}  // namespace

extern "C" pa_status pa_attention_plan(const pa_attn_desc* desc, int32_t q_len, pa_attn_plan* out) {
  if (!out) return PA_ERR_INVALID_ARG;
  Plan pl;
  pa_status st = make_plan(desc, q_len, &pl);
  if (st != PA_OK) return st;
  out->path = pl.path;
  out->schedule = pl.sched;
  out->partition_tokens = pl.part_tokens;
  out->num_partitions = pl.parts;
  out->waves_per_group = pl.waves;
  out->grid = launch_grid(pl, desc);
  out->merge_grid = pl.merge_grid;
  out->tiles_per_wave = pl.path == PA_PATH_MFMA ? pl.nt : 0;
  out->partitions_per_wave = pl.sched == PA_SCHED_PARTITIONS_WAVE ? pl.run_parts : 0;
  out->segment_cost = pl.sched == PA_SCHED_BALANCED ? pl.seg_cost : 0;
  out->workspace_bytes = pl.ws;
  return PA_OK;
}

extern "C" size_t pa_attention_workspace_size(const pa_attn_desc* desc, int32_t q_len) {
  Plan pl;
  return make_plan(desc, q_len, &pl) == PA_OK ? pl.ws : 0;
}

namespace {

// This device's copy of `scratch`, looked up once per device (with that
// device current), or null with the HIP error recorded.
void* scratch_base() {
  static std::mutex mu;
  static void* base[kMaxDevices];
  int dev = 0;
  if (const hipError_t e = hipGetDevice(&dev); e != hipSuccess) {
    (void)hipGetLastError();
    pa::hip_failed(e);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!base[dev]) {
    void* p = nullptr;
    if (const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess || !p) {
      (void)hipGetLastError();
      pa::hip_failed(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return nullptr;
    }
    base[dev] = p;
  }
  return base[dev];
}

__global__ __launch_bounds__(256) void zero_words(int32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0;
}

// Where the split-KV state of a call lives: the caller's workspace, or this
// library's scratch.
enum class Ws { caller, scratch };

pa_status attention_impl(const pa_attn_desc* desc, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t q_len, const uint32_t* tree_mask,
                         int32_t mask_stride, float scale, void* out, void* workspace,
                         size_t workspace_bytes, Ws ws_kind, void* stream) {
  Plan pl;
  pa_status st = make_plan(desc, q_len, &pl);
  if (st != PA_OK) return st;
  pl.tree = tree_mask != nullptr;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  char* counters_at = nullptr;  // arrival counters (balanced schedule)
  char* partials_at = nullptr;  // (m, l) partials; o follows at pl.ws_o_off
  if (ws_kind == Ws::caller) {
    if (pl.ws > 0 && (!workspace || workspace_bytes < pl.ws)) return PA_ERR_INVALID_ARG;
    if (pl.ws > 0 && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return PA_ERR_INVALID_ARG;  // 16-byte partial stores
    counters_at = static_cast<char*>(workspace);
    partials_at = counters_at + pl.ws_counters;
  } else if (pl.ws > 0) {
    if (pl.ws_counters > kScratchCounterBytes || pl.ws_partials > kScratchBytes - kScratchCounterBytes)
      return PA_ERR_TOO_LARGE;
    char* base = static_cast<char*>(scratch_base());
    if (!base) return PA_ERR_HIP;
    counters_at = base;
    partials_at = base + kScratchCounterBytes;
  }
  AttnArgs args;
  args.q = q;
  args.k_pool = k_pool;
  args.v_pool = v_pool;
  args.tables = block_tables;
  args.lens = context_lens;
  args.out = out;
  args.counters = nullptr;
  args.part_ml = nullptr;
  args.part_o = nullptr;
  args.k_scales = nullptr;
  args.v_scales = nullptr;
  args.tree_mask = tree_mask;
  args.mask_stride = mask_stride;
  if (pl.kv8) {
    const int64_t codes = pa::fp8_codes_bytes(desc->num_blocks, desc->num_kv_heads, desc->block_size,
                                              desc->head_dim);
    args.k_scales = reinterpret_cast<const float*>(static_cast<const char*>(k_pool) + codes);
    args.v_scales = reinterpret_cast<const float*>(static_cast<const char*>(v_pool) + codes);
  }
  if (pl.ws) {
    if (pl.sched == PA_SCHED_BALANCED) args.counters = reinterpret_cast<int32_t*>(counters_at);
    args.part_ml = reinterpret_cast<float*>(partials_at);
    args.part_o = reinterpret_cast<float*>(partials_at + pl.ws_o_off);
  }
  args.num_seqs = desc->num_seqs;
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
  args.seg_cost = pl.sched == PA_SCHED_BALANCED ? pl.seg_cost : 0;
  args.run_parts = pl.run_parts;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ws_kind == Ws::scratch && pl.sched == PA_SCHED_BALANCED) {
    // the scratch's counters start every call at zero (a fill kernel, not a
    // memset node, so that a captured graph replays it correctly)
    hipLaunchKernelGGL(zero_words, dim3(std::min<int64_t>(64, (pl.segments + 255) / 256)), dim3(256), 0, s,
                       args.counters, int64_t(pl.segments));
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return pa::hip_failed(e);
  }
  st = launch_main(pl, desc, args, s);
  if (st != PA_OK || pl.merge_grid == 0) return st;
  return desc->head_dim == 64 ? launch_merge<64>(pl, desc->dtype, args, s)
                              : launch_merge<128>(pl, desc->dtype, args, s);
}

}  // namespace

extern "C" pa_status pa_attention(const pa_attn_desc* desc, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables,
                                  const int32_t* context_lens, int32_t q_len, float scale,
                                  void* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return attention_impl(desc, q, k_pool, v_pool, block_tables, context_lens, q_len, nullptr, 0,
                        scale, out, workspace, workspace_bytes, Ws::caller, stream);
}

extern "C" pa_status pa_attention_noalloc(const pa_attn_desc* desc, const void* q, const void* k_pool,
                                          const void* v_pool, const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t q_len, float scale,
                                          void* out, void* stream) {
  return attention_impl(desc, q, k_pool, v_pool, block_tables, context_lens, q_len, nullptr, 0,
                        scale, out, nullptr, 0, Ws::scratch, stream);
}

extern "C" pa_status pa_attention_tree(const pa_attn_desc* desc, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* block_tables,
                                       const int32_t* context_lens, int32_t q_len,
                                       const uint32_t* tree_mask, int32_t mask_stride, float scale,
                                       void* out, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (!tree_mask || q_len < 1 || q_len > PA_TREE_MAX_NODES) return PA_ERR_INVALID_ARG;
  if (mask_stride != 0 && mask_stride < q_len) return PA_ERR_INVALID_ARG;
  if (desc && int64_t(mask_stride) * (desc->num_seqs - 1) + q_len > INT32_MAX) return PA_ERR_INVALID_ARG;
  return attention_impl(desc, q, k_pool, v_pool, block_tables, context_lens, q_len, tree_mask,
                        mask_stride, scale, out, workspace, workspace_bytes, Ws::caller, stream);
}
