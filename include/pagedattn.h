/*
 * pagedattn.h -- C ABI of libpagedattn.so: a paged KV cache and paged decode
 * attention for one AMD Instinct MI355X (gfx950).
 *
 * The problem, as the pages state it:
 *   - The KV cache of every sequence is cut into fixed-size physical blocks of
 *     16 or 32 tokens that may sit anywhere in device memory; a per-sequence
 *     block table maps logical block j (tokens j*bs .. j*bs+bs-1) to a
 *     physical block, and the attention kernel reads that table itself.
 *     [Part 8 (vLLM), "PagedAttention: Ảo Hóa Phân Trang Bộ Nhớ Cho Key và
 *     Value" and the block-table diagram of "Phân Tích Cơ Cấu Bộ Nhớ Của KV
 *     Cache"; Blog #54, section 2.2 and its address diagram]
 *   - A sequence takes one block from the shared free pool each time it grows
 *     past a multiple of the block size; sequences sharing a prompt point at
 *     the same blocks with a reference count; a write into a shared block
 *     first gives the writer a private copy (copy-on-write); a block whose
 *     count reaches 0 is free again.
 *     [Blog #54, interview question 2; Part 8, "RadixAttention"]
 *   - Attention output for query row q_i is softmax(q_i K^T / sqrt(d_k)) V
 *     over the sequence's context, computed block by block with an online
 *     softmax. [Part 8, "Thực Thi Kernel Toán Học Trong CUDA", eqs. for A_i,
 *     A_{i,j} and o_i]
 *
 * Conventions for every call:
 *   - Every call returns a pa_status; nothing throws or aborts across the ABI.
 *     Argument errors are detected on the host before any state change or
 *     launch. Device work is asynchronous on the given stream (a hipStream_t
 *     passed as void*, NULL = the null stream); a fault in it surfaces as
 *     PA_ERR_HIP from a later launch check or from the caller's own
 *     synchronisation.
 *   - "host" pointers are CPU memory, "device" pointers are GPU memory on the
 *     current HIP device; all buffers are owned by the caller unless stated.
 *   - Host bookkeeping memory is allocated when a pool or prefix cache is
 *     made and by the calls that plan a write, match or insert a prefix, each
 *     before it changes anything (PA_ERR_NO_MEMORY if that fails). Block
 *     allocation, fork and release, eviction, the queries and destroying a
 *     handle allocate nothing.
 *   - A pool and its prefix cache are not safe for concurrent use: calls on
 *     one pool are serialised by the caller. Distinct pools are independent.
 *   - Pool layout (device memory, caller-owned, element type = pool dtype):
 *       k_pool: [num_blocks][num_kv_heads][head_dim/32][block_size][32]
 *       v_pool: [num_blocks][num_kv_heads][head_dim][block_size]
 *     One (block, kv head) slice of K or V is contiguous (block_size*head_dim
 *     elements). Within a K slice the head dimension is cut into 32-element
 *     slabs, each holding the block's tokens back to back; within a V slice
 *     each head-dimension element keeps the block's tokens adjacent. Element
 *     (token t, dim c) of block b, KV head h is at
 *       K: (((b*H_kv + h)*(head_dim/32) + c/32)*block_size + t)*32 + c%32
 *       V: ((b*H_kv + h)*head_dim + c)*block_size + t
 *   - bf16 is IEEE bfloat16 stored as uint16; f32 is IEEE binary32.
 *   - FP8 pools (PA_DTYPE_FP8_E4M3; the pages name FP8 KV quantisation as the
 *     capacity lever: Blog #54 section 4, Part 8 quantisation section) hold
 *     OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *     largest finite 448) plus one fp32 scale per (token, KV head); the value
 *     of a code is decode(code) * scale. Each buffer is the codes followed by
 *     the scales, pa_pool_buffer_bytes long:
 *       k_pool: codes [num_blocks][num_kv_heads][head_dim/64][block_size][64],
 *               then scales [num_blocks][num_kv_heads][block_size]
 *       v_pool: codes [num_blocks][num_kv_heads][head_dim][block_size],
 *               then scales [num_blocks][num_kv_heads][block_size]
 *     Rows are written as bf16 and quantised per (token, KV head): scale =
 *     the smallest power of two >= max|x| / 448 (the quotient in fp32; 1 for
 *     an all-zero row), code = round-to-nearest-even(x / scale) in fp32 (the
 *     division is exact). Power-of-two scales keep every weight times its
 *     token's V scale a bf16 number, so attention applies them exactly.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;
enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,   /* bad pointer, shape, range or size */
  PA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head_dim, block_size, dtype, rows) */
  PA_ERR_NO_FREE_BLOCK = 3, /* the pool cannot supply the blocks asked for */
  PA_ERR_BAD_BLOCK = 4,     /* refcount underflow, fork/free of a free block */
  PA_ERR_HIP = 5,           /* a HIP runtime call or kernel launch failed */
  PA_ERR_NO_MEMORY = 6,     /* host memory for the bookkeeping could not be allocated;
                               the call changed nothing */
  PA_ERR_TOO_LARGE = 7      /* the call needs more scratch than pa_attention_noalloc
                               holds; nothing launched */
};

enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1, PA_DTYPE_FP8_E4M3 = 2 };

/* K/V storage of the pools read by pa_attention (pa_attn_desc.kv_format). */
enum { PA_KV_SAME = 0, PA_KV_FP8_E4M3 = 1 };

/* Kernel selection for pa_attention. AUTO picks by dtype and row count. */
enum { PA_PATH_AUTO = 0, PA_PATH_VALU = 1, PA_PATH_MFMA = 2 };

/* How pa_attention splits the batch's work (reported by pa_attention_plan).
 * PARTITIONS: one workgroup per (sequence, KV head, fixed-length token
 *   partition); sequences longer than a partition are finished by a second,
 *   log-sum-exp merge kernel.
 * BALANCED: the grid holds as many workgroups as the GPU runs at once and
 *   each takes an equal share of all (sequence, KV head, 32-token step) work
 *   items; a sequence split between workgroups is merged by the workgroup
 *   that finishes its last share (one kernel, no second launch).
 * PARTITIONS_WAVE: fixed-length partitions as PARTITIONS, one wavefront per
 *   (sequence, KV head, partition), each writing its partial from registers;
 *   chosen instead of PARTITIONS on the MFMA path when the partitions alone
 *   fill every wave slot of the device. The same merge kernel follows.
 * Split-KV on one GPU as on the pages: attention local to each partition of
 * the sequence, then a reduction of the partitions' results ("Mở rộng Quy mô
 * và Triển khai", "Song song hóa Chuỗi"; the reduction is the log-sum-exp
 * merge). */
enum { PA_SCHED_PARTITIONS = 0, PA_SCHED_BALANCED = 1, PA_SCHED_PARTITIONS_WAVE = 2 };

/* Largest tree of drafted tokens pa_attention_tree takes: one 32-bit
 * visibility mask per node. */
enum { PA_TREE_MAX_NODES = 32 };

/* Human-readable name of a status code (static string, never NULL). */
const char* pa_status_string(pa_status s);

/* ------------------------------------------------------------------------ */
/* Block pool (host metadata only)                                          */
/* ------------------------------------------------------------------------ */

typedef struct pa_pool pa_pool;
typedef struct pa_prefix_cache pa_prefix_cache;

/* Create the host-side bookkeeping of a pool of num_blocks physical blocks:
 * a reference count per block (all 0) and a LIFO free list. The free list's
 * initial order is initial_free_order[0..num_blocks) (host, a permutation of
 * 0..num_blocks-1; the first entry is handed out first), or ascending ids
 * when NULL. block_size must be 16 or 32, head_dim 64 or 128, dtype
 * PA_DTYPE_F32, PA_DTYPE_BF16 or PA_DTYPE_FP8_E4M3 (PA_ERR_UNSUPPORTED
 * otherwise). The device
 * arrays k_pool/v_pool are not allocated here: the caller owns them.
 * *out receives the handle (PA_ERR_INVALID_ARG if out is NULL or the order
 * is not a permutation). [Blog #54 question 2: the free block pool] */
pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, int32_t dtype, const int32_t* initial_free_order,
                         pa_pool** out);

/* Release the handle (NULL is a no-op). Device memory is not touched. */
void pa_pool_destroy(pa_pool* pool);

/* Bytes of one pool buffer (k_pool or v_pool; both have this size) for the
 * given shape and storage dtype, scales included for FP8. -1 for an invalid
 * or unsupported shape. */
int64_t pa_pool_buffer_bytes(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                             int32_t head_dim, int32_t dtype);

/* Bytes of K plus V that one token occupies: 2 * num_layers * num_kv_heads *
 * head_dim * elem_bytes; at 16-bit storage this is 4 * L * H_kv * d_k
 * [Part 8, "Phân Tích Cơ Cấu Bộ Nhớ Của KV Cache": 327,680 B for 80 layers,
 * 8 KV heads, d_k 128]. Returns -1 if any argument is <= 0. */
int64_t pa_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                              int32_t elem_bytes);

/* Pop the head of the free list into *block_id and set its count to 1: a
 * sequence that grows past a multiple of the block size asks the free pool
 * for one more physical block [Blog #54 question 2: a new block is requested
 * from the free block pool each time the current one fills; Part 8,
 * "PagedAttention: Ảo Hóa Phân Trang Bộ Nhớ Cho Key và Value": blocks are
 * handed out on demand]. With a prefix cache attached, an empty free list
 * evicts the least recently used unreferenced cached block instead.
 * PA_ERR_NO_FREE_BLOCK when no block can be supplied (state unchanged);
 * PA_ERR_INVALID_ARG for a NULL pool or block_id. */
pa_status pa_block_alloc(pa_pool* pool, int32_t* block_id);

/* Share a live block: count += 1 [Blog #54 question 2: sharers point at the
 * same block; Part 8 "RadixAttention": ref_count++ on reuse].
 * PA_ERR_INVALID_ARG if out of range, PA_ERR_BAD_BLOCK if the block is free. */
pa_status pa_block_fork(pa_pool* pool, int32_t block_id);

/* Drop one reference; at 0 the block is pushed on the head of the free list
 * [Part 8 "RadixAttention": blocks with ref_count 0 are reclaimable].
 * PA_ERR_BAD_BLOCK if the block is already free (state unchanged). */
pa_status pa_block_free(pa_pool* pool, int32_t block_id);

/* Read-only queries. */
pa_status pa_block_refcount(const pa_pool* pool, int32_t block_id, int32_t* refcount);
pa_status pa_pool_num_free(const pa_pool* pool, int32_t* num_free);
/* Copy the free list, head first, into out[0..capacity) (host); *n receives
 * its full length. PA_ERR_INVALID_ARG if capacity < length. */
pa_status pa_pool_free_list(const pa_pool* pool, int32_t* out, int32_t capacity, int32_t* n);

/* ------------------------------------------------------------------------ */
/* Writing keys and values                                                  */
/* ------------------------------------------------------------------------ */

/* Host-only planning of a write of tokens [start_pos, start_pos + n_tokens)
 * of one sequence. block_table (host, table_capacity entries) holds the
 * sequence's physical block ids, the first *num_blocks_inout of them live.
 * For each logical block the write touches, in ascending order:
 *   - a block past the live ones is taken from the free list and appended
 *     [Blog #54 question 2: one new block per block_size tokens];
 *   - a live block whose count is > 1 is copied into a fresh block, the old
 *     block loses one reference and the table entry is patched
 *     (copy-on-write) [Blog #54 question 2: only the diverging part gets a
 *     new block].
 * Outputs (host, each nullable): copies_out[2*k], copies_out[2*k+1] = (src,
 * dst) of the k-th copy, at most max_copies pairs (*n_copies_out = count,
 * PA_ERR_INVALID_ARG before any change if more would be needed);
 * slots_out[i] = physical slot (block*block_size + offset) of token
 * start_pos+i. No device work: the caller must perform the copies before
 * storing tokens (pa_write_kv does both).
 * Errors, all before any change: PA_ERR_INVALID_ARG for negative sizes, a
 * start past the live blocks' end (a hole), or a table too small;
 * PA_ERR_BAD_BLOCK if a touched live entry names a free block;
 * PA_ERR_NO_FREE_BLOCK if the pool cannot supply every block needed. */
pa_status pa_write_plan(pa_pool* pool, int32_t* block_table, int32_t table_capacity,
                        int32_t* num_blocks_inout, int32_t start_pos, int32_t n_tokens,
                        int32_t* copies_out, int32_t max_copies, int32_t* n_copies_out,
                        int32_t* slots_out);

/* Append or overwrite tokens of one sequence: pa_write_plan on the host, then
 * on `stream` the copy-on-write block copies and one scatter of k_new/v_new
 * (device, [n_tokens][num_kv_heads][head_dim], pool dtype) into k_pool/v_pool
 * (device, pool layout above). The host table and live count are updated in
 * place; the caller re-uploads the table before attention reads it.
 * Same errors as pa_write_plan (nothing launched), PA_ERR_INVALID_ARG for
 * NULL device pointers, PA_ERR_HIP if a launch fails (the host state has
 * then already changed). */
pa_status pa_write_kv(pa_pool* pool, void* k_pool, void* v_pool, int32_t* block_table_host,
                      int32_t table_capacity, int32_t* num_blocks_inout, int32_t start_pos,
                      int32_t n_tokens, const void* k_new, const void* v_new, void* stream);

/* Copy whole physical blocks (every KV head, K and V, and their scales in an
 * FP8 pool) on `stream`:
 * block src_dst[2k] -> block src_dst[2k+1] for k < n_pairs (host array).
 * The device half of copy-on-write. PA_ERR_INVALID_ARG for an id out of
 * range or src == dst. */
pa_status pa_copy_blocks(const pa_pool* pool, void* k_pool, void* v_pool, const int32_t* src_dst,
                         int32_t n_pairs, void* stream);

/* ------------------------------------------------------------------------ */
/* Attention                                                                */
/* ------------------------------------------------------------------------ */

typedef struct pa_attn_desc {
  int32_t num_seqs;           /* B */
  int32_t num_q_heads;        /* H_q, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* H_kv; query head h reads KV head h / (H_q/H_kv) */
  int32_t head_dim;           /* d: 64 or 128 */
  int32_t block_size;         /* bs: 16 or 32 */
  int32_t max_blocks_per_seq; /* MB: row stride of block_tables */
  int32_t num_blocks;         /* NB: pool size; table entries must be in [0, NB) */
  int32_t dtype;              /* PA_DTYPE_F32 or PA_DTYPE_BF16 (q, pools, out) */
  int32_t max_context;        /* upper bound on context_lens, <= MB*bs */
  int32_t path;               /* PA_PATH_* (AUTO unless testing a path) */
  int32_t partition_tokens;   /* 0 = chosen by the library (BALANCED on the MFMA path
                                 for up to 8192 sequences, else PARTITIONS); otherwise
                                 PARTITIONS of this many tokens, a multiple of 64 */
  int32_t waves_per_group;    /* wavefronts per workgroup of the main kernel: 0 = chosen
                                 by the library; else 1, 2 or 4 for the PARTITIONS
                                 schedules, and 1, 2, 4, 8 or 12 for BALANCED (12 with
                                 one 16-row query tile, G*q_len <= 16; at most 8 with
                                 two). Larger values than the schedule allows give
                                 PA_ERR_UNSUPPORTED, values outside the list
                                 PA_ERR_INVALID_ARG */
  int32_t kv_shared;          /* cache hint, results do not depend on it: 0 = every
                                 physical block is read by one sequence only, so K/V
                                 loads stream past the caches; 1 = some blocks are
                                 shared (a common prompt), so K/V loads stay cacheable */
  int32_t kv_format;          /* PA_KV_SAME: pools in dtype; PA_KV_FP8_E4M3: FP8 pools
                                 (dtype must be PA_DTYPE_BF16, MFMA path only) */
  int32_t reserved[2];        /* must be 0 */
} pa_attn_desc;

/* What pa_attention launches for a descriptor (for tests and profiling). */
typedef struct pa_attn_plan {
  int32_t path;               /* PA_PATH_VALU or PA_PATH_MFMA */
  int32_t schedule;           /* PA_SCHED_PARTITIONS, PA_SCHED_BALANCED or
                                 PA_SCHED_PARTITIONS_WAVE */
  int32_t partition_tokens;   /* PARTITIONS*: tokens per partition (0 for BALANCED) */
  int32_t num_partitions;     /* PARTITIONS*: partitions per sequence (1 = no merge pass) */
  int32_t waves_per_group;    /* wavefronts per workgroup of the main kernel */
  int32_t grid;               /* workgroups of the main kernel; BALANCED: the resident
                                 capacity of the current device for that kernel (an
                                 upper bound when no device is available) */
  int32_t merge_grid;         /* workgroups of the merge kernel (0 if none) */
  int32_t tiles_per_wave;     /* MFMA: 16-row query tiles each wavefront holds (1, or 2
                                 when G*q_len > 16); 0 for the VALU path */
  int32_t partitions_per_wave; /* PARTITIONS_WAVE: consecutive partitions of one (sequence,
                                 KV head) each wavefront streams: 1, or a run of several
                                 when the partitions outnumber the device's wave slots;
                                 0 for the other schedules */
  int32_t segment_cost;       /* BALANCED: steps a (sequence, KV head) segment's start
                                 counts for when the (KV head, sequence, step) list is
                                 cut into equal ranges: S = H_kv * sum over valid
                                 sequences of (ceil(L/32) + segment_cost) units, and
                                 min(grid, ceil(S / 8)) ranges; 0 for the other
                                 schedules */
  size_t workspace_bytes;     /* workspace pa_attention needs */
} pa_attn_plan;

/* Fill *plan for this descriptor and q_len; PA_ERR_INVALID_ARG /
 * PA_ERR_UNSUPPORTED exactly where pa_attention would fail validation. */
pa_status pa_attention_plan(const pa_attn_desc* desc, int32_t q_len, pa_attn_plan* plan);

/* Workspace bytes pa_attention needs for this descriptor and q_len: the
 * split-KV partials of sequence-parallel attention, each partition's (m, l, o)
 * kept until the log-sum-exp reduction combines them ["Mở rộng Quy mô và
 * Triển khai", "Song song hóa Chuỗi": attention local to each KV segment,
 * then a reduction; Part 8, "Thực Thi Kernel Toán Học Trong CUDA": the
 * running maximum and sum of the online softmax are what a partial carries].
 * 0 when nothing is split, or for an invalid descriptor. The size does not
 * depend on the device: the balanced schedule's share is bounded for at most
 * 256 compute units (a larger device runs that many resident workgroups at
 * most). Layout, the same for every schedule: align256(4*num_seqs*
 * num_kv_heads) bytes of arrival counters, written by the BALANCED schedule
 * only; then the (m, l) partials; then, from a 256-byte boundary, the o
 * partials. */
size_t pa_attention_workspace_size(const pa_attn_desc* desc, int32_t q_len);

/* Paged attention for q_len query rows per sequence [Part 8, "Thực Thi
 * Kernel Toán Học Trong CUDA": A_i = softmax(q_i K^T / sqrt(d_k)), computed
 * block by block over the blocks B_1..B_m the block table names, with the
 * running maximum, running sum and rescaled output of an online softmax;
 * Blog #54 section 2.2: the kernel reads the block table itself; Blog #54
 * section 2.4 and Part 8's speculative-decoding diagram: q_len > 1 scores all
 * drafted tokens in one pass].
 *   q            device [B][q_len][H_q][d]
 *   k_pool       device pool layout above; v_pool likewise
 *   block_tables device int32 [B][max_blocks_per_seq]; entries past a
 *                sequence's ceil(L_b/bs) blocks are never read
 *   context_lens device int32 [B]; L_b counts the q_len new tokens, whose
 *                K/V must already be written at positions L_b-q_len..L_b-1
 *   q_len        query rows per sequence (1 = decode; > 1 = verification of
 *                drafted tokens: row i attends to positions 0..L_b-q_len+i)
 *   scale        multiplies q.k (1/sqrt(d) for standard attention)
 *   out          device [B][q_len][H_q][d], same dtype as q
 *   workspace    device, >= pa_attention_workspace_size bytes, 16-byte aligned
 *                (may be NULL when that size is 0); holds split-KV partials, no
 *                hidden allocation.
 *                Its first align256(4*B*H_kv) bytes are the BALANCED
 *                schedule's arrival counters, which must be zero when such a
 *                call starts. Only that schedule writes them, and every
 *                completed call leaves them zero; every other layout starts
 *                its partials after them. So a workspace zero-filled once
 *                serves any sequence of calls (any schedule, path or q_len)
 *                whose B*H_kv never grows; after a call with a smaller B*H_kv
 *                wrote partials there, zero-fill it again before a BALANCED
 *                call with a larger one. Calls that share one workspace must
 *                not run concurrently.
 * Output row (b, i, h) = softmax(scale * q[b,i,h] . K_b[t], t visible) . V_b.
 * Requirements (else PA_ERR_INVALID_ARG / PA_ERR_UNSUPPORTED, nothing
 * launched): H_q % H_kv == 0, d in {64,128}, bs in {16,32}, 1 <= q_len,
 * max_context <= MB*bs, (H_q/H_kv)*q_len rows within the chosen path's limit.
 * A sequence whose context_lens entry lies outside [q_len, max_context], or
 * whose table names a block outside [0, NB), gets NaN in all its output rows;
 * the kernels never read outside the pools or past a table row. */
pa_status pa_attention(const pa_attn_desc* desc, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_tables,
                       const int32_t* context_lens, int32_t q_len, float scale, void* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* pa_attention for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as pa_attention, without the workspace:
 * split-KV state lives in a scratch array inside this library, one per GPU,
 * PA_NOALLOC_SCRATCH_BYTES long, held from the first call on that GPU until
 * the process ends. Its first 256 KiB are the balanced schedule's arrival
 * counters (up to 65,536 (sequence, KV head) pairs), zeroed on the stream by
 * a small kernel at the start of every call that uses them; the rest holds
 * the partials (at most pa_attention_workspace_size minus its counter area).
 * A call needing more returns PA_ERR_TOO_LARGE before any device work. The
 * call allocates nothing, host or device. Every call on one GPU shares that
 * GPU's scratch and leaves its contents there: calls that may overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller. */
enum { PA_NOALLOC_SCRATCH_BYTES = 64 << 20 };
pa_status pa_attention_noalloc(const pa_attn_desc* desc, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t q_len, float scale,
                               void* out, void* stream);

/* Tree-structured verification ("Mở rộng Quy mô và Triển khai", section
 * "Giải mã Suy đoán", its variants: parallel decoding drafts a tree of
 * candidate continuations and the target verifies the whole tree in one
 * pass). The q_len drafted tokens are the nodes of a tree, node j at position
 * L_b-q_len+j (its K/V written there); node i sees the context (positions
 * 0..L_b-q_len-1) and the nodes whose bit is set in its mask:
 *   tree_mask    device uint32 [B][mask_stride] (mask_stride > 0) or [q_len]
 *                shared by every sequence (mask_stride == 0); bit j of
 *                tree_mask[b*mask_stride + i] lets row i of sequence b see
 *                node j. Bit i is taken as set (a node always sees itself);
 *                bits at or above q_len are ignored. pa_tree_masks turns
 *                parent indices into ancestor masks.
 *   mask_stride  0, or >= q_len
 * Everything else is pa_attention's, which this equals when every mask is
 * the causal one (bits 0..i). PA_ERR_INVALID_ARG for a null tree_mask,
 * q_len > PA_TREE_MAX_NODES or a bad stride, besides pa_attention's checks.
 * Mask contents are not validated: any 32-bit value is a valid mask. */
pa_status pa_attention_tree(const pa_attn_desc* desc, const void* q, const void* k_pool,
                            const void* v_pool, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t q_len,
                            const uint32_t* tree_mask, int32_t mask_stride, float scale,
                            void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Radix prefix cache (Part 8, "RadixAttention"; "Mở rộng Quy mô và
 * Triển khai", "Cache Tiền tố") -------------------------------------------
 * Host bookkeeping attached to a pool: the KV blocks of earlier requests are
 * kept in a prefix tree, a request whose tokens match a cached prefix reuses
 * those physical blocks (reference count + 1, no prefill for them), and under
 * memory pressure unreferenced cached blocks are reclaimed least recently
 * used first. Mechanics (this library's reading):
 *   - one tree node per full block, keyed by its block_size token ids;
 *   - a cached block whose count falls to 0 stays in the tree, unreferenced,
 *     stamped by a counter bumped at each such event; it is not on the free
 *     list (pa_pool_num_free does not count it);
 *   - pa_block_alloc and pa_write_kv take the free list first, then evict the
 *     unreferenced leaf with the oldest stamp; a block is reclaimable when it
 *     and its whole subtree are unreferenced, and availability checks count
 *     those (so a write either fits or changes nothing);
 *   - a write into a cached block copies it first, even at count 1.
 * Tokens are host int32 ids; tables are host int32 block ids. */

/* Attach a prefix cache to `pool` (one per pool; PA_ERR_INVALID_ARG if it
 * already has one). pa_pool_destroy also destroys an attached cache. */
pa_status pa_prefix_cache_create(pa_pool* pool, pa_prefix_cache** out);

/* Detach and delete: reclaimable blocks go to the free list in eviction
 * order, then every other unreferenced cached block in stamp order; blocks
 * still referenced return to the free list when released. */
void pa_prefix_cache_destroy(pa_prefix_cache* cache);

/* Longest cached prefix of whole blocks of tokens[0..n_tokens), at most
 * `capacity` blocks: writes them to table[0..*n_blocks) and forks each
 * (an unreferenced one is referenced again). The caller continues writing at
 * position *n_blocks * block_size. */
pa_status pa_prefix_match(pa_prefix_cache* cache, const int32_t* tokens, int32_t n_tokens,
                          int32_t* table, int32_t capacity, int32_t* n_blocks);

/* Cache a request's full blocks: tokens[0..n_tokens) held in table[0..n_blocks)
 * (only final tokens: a cached block is never written again). Walking the
 * tree, an existing node with the same tokens is followed; otherwise the
 * request's block becomes that node. *n_new (nullable) = nodes added.
 * PA_ERR_INVALID_ARG if a block to add is out of range or already cached
 * under another prefix, PA_ERR_BAD_BLOCK if it is free; nothing changes then. */
pa_status pa_prefix_insert(pa_prefix_cache* cache, const int32_t* tokens, int32_t n_tokens,
                           const int32_t* table, int32_t n_blocks, int32_t* n_new);

/* Evict up to max_blocks reclaimable blocks (LRU leaves first) onto the free
 * list's head; their ids in eviction order go to `evicted` (nullable). */
pa_status pa_prefix_evict(pa_prefix_cache* cache, int32_t max_blocks, int32_t* evicted,
                          int32_t* n_evicted);

/* Counts of cached, unreferenced cached, and reclaimable blocks (nullable). */
pa_status pa_prefix_cache_stats(const pa_prefix_cache* cache, int32_t* cached,
                                int32_t* unreferenced, int32_t* reclaimable);

/* Every cached block in ascending id order with its parent block (-1: child
 * of the root) and unreferenced stamp (-1: referenced). *n = the count;
 * PA_ERR_INVALID_ARG if capacity is smaller (only *n is written then). */
pa_status pa_prefix_cache_dump(const pa_prefix_cache* cache, int32_t* blocks, int32_t* parents,
                               int64_t* stamps, int32_t capacity, int32_t* n);

/* Speculative decoding's accept / resample step (Blog #54, interview
 * question 3; Part 8, "Thuật Toán Chấp Nhận & Từ Chối Phỏng Đoán"): drafted
 * token x_k is kept with probability min(1, p_k(x_k) / q_k(x_k)); at the
 * first rejection the later drafts are dropped and one token is drawn from
 * max(0, p_k - q_k) renormalised; when all K are kept one more token is drawn
 * from p_{K+1} (Blog #54, section 2.4 example). Per sequence b, all device:
 *   p             float32 [B][K+1][vocab] target probabilities
 *   q             float32 [B][K][vocab] draft probabilities (may be NULL if K = 0)
 *   draft         int32 [B][K] drafted tokens
 *   u_accept      float32 [B][K] uniforms in [0, 1), one per acceptance test
 *   u_draw        uint32 [B] uniform 32-bit integers, one per draw
 *   num_accepted  int32 [B] out: drafts kept (0..K), or -1 when a drafted
 *                 token lies outside [0, vocab) (tokens then all -1)
 *   tokens        int32 [B][K+1] out: the kept drafts, then the drawn token,
 *                 then -1
 * The test is taken in float32: keep iff p >= q or u * q < p (one rounding).
 * The draw: weights w = max(0, p - q) (p - q rounded once; p itself for the
 * extra token, or when every residual weight is below 2^-32) become
 * integers floor(w * 2^32); with S their sum and T = floor(U * S / 2^32)
 * the token drawn is the smallest x whose running sum exceeds T (-1 if
 * S = 0). Bit-exact and independent of summation order. Asynchronous on
 * `stream`; PA_ERR_INVALID_ARG for bad sizes, missing pointers or a
 * workspace smaller than pa_spec_accept_workspace_size. */
pa_status pa_spec_accept(const float* p, const float* q, const int32_t* draft,
                         const float* u_accept, const uint32_t* u_draw, int32_t num_seqs,
                         int32_t num_draft, int32_t vocab, int32_t* num_accepted, int32_t* tokens,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes pa_spec_accept needs (device, caller-owned: per-chunk
 * weight sums and per-sequence arrival counters). It must be zero-filled
 * before its first use; every completed call leaves the counters zero again.
 * Calls sharing a workspace must not run concurrently. 0 for bad sizes. */
size_t pa_spec_accept_workspace_size(int32_t num_seqs, int32_t vocab);

/* The hipError_t of this thread's last HIP call that made a pa_* function
 * return PA_ERR_HIP (0 if none yet), and the HIP runtime's name for a
 * hipError_t value. Diagnostics only. */
int32_t pa_last_hip_error(void);
const char* pa_hip_error_name(int32_t hip_error);

/* Host helper: ancestor masks of a tree given by parent indices.
 *   parents  host int32 [n]; parents[i] is -1 (node i continues the context)
 *            or an earlier node (0 <= parents[i] < i)
 *   masks    host uint32 [n] out; bit j of masks[i] is set iff node j is node
 *            i or one of its ancestors
 * PA_ERR_INVALID_ARG for null pointers, n outside [1, PA_TREE_MAX_NODES] or a
 * parent that is not an earlier node (masks then unspecified). */
pa_status pa_tree_masks(const int32_t* parents, int32_t n, uint32_t* masks);

/* Read-bandwidth probe, a measurement aid for the HBM roofline of the
 * attention kernels (not part of the attention path): reads num_blocks
 * blocks of block_bytes of `buf` in the order given, the access pattern of a
 * pool's (block, KV head) slices, with non-temporal loads.
 *   buf               device, >= num_blocks * block_bytes bytes
 *   block_bytes       4096 or 8192 (a slice at block size 16 or 32, head
 *                     dimension 128, bf16)
 *   order             device int32 [num_blocks]: block ids to read (a
 *                     permutation for a full pass; ids outside
 *                     [0, num_blocks) are clamped, never read past buf)
 *   blocks_in_flight  1, 2 or 4 blocks per wavefront loaded together
 *   workgroups        grid size (256 threads each)
 *   sink              device uint32 [1]: written only for one unlikely
 *                     checksum, so that the loads are kept
 * Asynchronous on `stream`; time it with events around the call.
 * PA_ERR_INVALID_ARG for null pointers or bad sizes, PA_ERR_HIP if the launch
 * fails. */
pa_status pa_read_probe(const void* buf, int64_t num_blocks, int32_t block_bytes, const int32_t* order,
                        int32_t blocks_in_flight, int32_t workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
