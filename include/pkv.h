/*
 * pkv.h -- C ABI of libpkv: paged KV-cache decode attention for MI355X (gfx950).
 *
 * What the library computes
 *   The KV cache of every sequence is cut into fixed-size blocks of
 *   block_size tokens that may sit anywhere in a pool; a per-sequence block
 *   table maps logical block j to its physical block ("AI Engineering
 *   Visualised: KV cache", intro; "KV cache and PagedAttention in serving",
 *   section "PagedAttention: virtual memory for GPUs").  The attention
 *   kernel computes attention directly over those blocks through the block
 *   table, never gathering them into a contiguous copy (same section; "Paged
 *   KV Cache" tutorial, section "Block Tables and Sharing").  Decode attends
 *   one new query token per sequence over the cached K/V of the tokens
 *   processed so far ("KV cache and PagedAttention in serving", section
 *   "What the KV cache actually is").
 *
 *   Attention here is softmax(scale * q . K^T) . V per query head, scale
 *   defaulting to 1/sqrt(head_dim); query head g reads KV head
 *   g / (h_q / h_kv) (grouped-query attention, "Paged KV Cache" tutorial,
 *   section "Reproduce Bytes per Token": query heads share KV heads).
 *
 * Conventions for every entry point
 *   - All tensors are dense, row-major, in device memory owned by the caller.
 *     The library allocates no device memory and keeps no pointer after a
 *     call returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *     stream).  Buffers must stay valid until the stream has passed the call.
 *     No call synchronizes the stream.
 *   - The return value is a pkv_status; nothing throws across the ABI.
 *     Scalar arguments are validated before anything is launched; on error
 *     nothing is launched and no memory is touched.
 *   - Device-resident data (block ids, context lengths, slots) is not read
 *     by the host.  The kernels bound every access: a block id outside
 *     [0, num_blocks) or a slot outside the pool is skipped rather than
 *     followed, and a context length is clamped to
 *     [0, max_blocks_per_seq * block_size].  Such inputs give undefined
 *     numbers, never an out-of-bounds access.
 *   - Thread-safe: the only global state is read-only after first use.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* Element types a tensor can hold. */
typedef enum {
  PKV_F32 = 0,      /* IEEE binary32 */
  PKV_F16 = 1,      /* IEEE binary16 */
  PKV_BF16 = 2,     /* bfloat16: the upper half of a binary32 */
  PKV_FP8_E4M3 = 3  /* OCP E4M3 (no infinities, max 448), one fp32 scale per tensor */
} pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* a scalar argument is out of range or a pointer is NULL */
  PKV_EUNSUPPORTED = 2,  /* valid, but this dtype / group / block-size combination is not built */
  PKV_ENOSPC = 3,        /* block manager: the pool cannot supply the blocks (state unchanged) */
  PKV_EWORKSPACE = 4,    /* workspace smaller than the sizing call returns */
  PKV_EHIP = 5           /* the HIP runtime reported an error at launch */
} pkv_status;

/* Human-readable name of a status code (static string; "unknown ..." for
 * a value outside the enum). */
const char* pkv_status_str(pkv_status status);

/* ABI version of this header (bumped on any signature change). */
#define PKV_ABI_VERSION 2
int pkv_abi_version(void);

/* ------------------------------------------------------------------------
 * Paged decode attention
 *
 * Shapes (S = num_seqs, Hq = h_q, Hkv = h_kv, D = head_dim, B = block_size,
 * NB = num_blocks, MB = max_blocks_per_seq):
 *   out          [S, Hq, D]       out_dtype in {F32, F16, BF16}
 *   q            [S, Hq, D]       q_dtype in {F32, F16, BF16}
 *   k_cache      [NB, Hkv, B, D]  kv_dtype
 *   v_cache      [NB, Hkv, B, D]  kv_dtype
 *   block_tables [S, MB] int32    physical block of logical block j of seq s;
 *                                  entries j >= ceil(ctx_s / B) are never read
 *   context_lens [S] int32        ctx_s: tokens attended by seq s; positions
 *                                  t >= ctx_s are never read (their bytes may
 *                                  be anything, NaN included)
 * A 16-bit out_dtype receives the fp32 result rounded to nearest-even.
 * Semantics: for each seq s and query head g (kv head h = g / (Hq / Hkv)):
 *   out[s, g, :] = sum_t softmax_t(scale * q[s, g, :] . K_s[h, t, :]) V_s[h, t, :]
 * over t in [0, ctx_s), where K_s[h, t, :] = k_cache[block_tables[s, t / B],
 * h, t % B, :] (times k_scale for FP8) and likewise for V.  ctx_s = 0 gives 0.
 *
 * Supported combinations (others return PKV_EUNSUPPORTED):
 *   1 <= Hq / Hkv <= 16; B >= 1;
 *   (q, kv) in {(F32, F32), (F16, F16), (BF16, BF16), (BF16, FP8_E4M3),
 *   (F16, FP8_E4M3)}.  The matrix-core path serves the 16-bit and FP8 caches
 *   when B is 16 times a power of two; everything else takes the vector path.
 *   D must be 64 or 128 (another D is PKV_EINVAL).
 *
 * max_context_len: an upper bound the host knows for max_s ctx_s (used only
 *   to size the split over blocks; a longer ctx_s is still computed exactly).
 * scale: logit scale; pass 0 (or a negative value) for 1/sqrt(D).
 * k_scale, v_scale: per-tensor FP8 scales (ignored for other kv dtypes).
 *
 * Workspace: device memory of at least
 *   pkv_decode_workspace_bytes(S, Hq, D, max_context_len, B) bytes.  It must
 *   be zero-filled before its FIRST use; every call leaves it ready for the
 *   next (its counters return to zero), so it is reused without clearing.
 *   Two calls in flight at once must not share a workspace.
 * Errors: PKV_EINVAL (NULL pointer, S < 0, Hq % Hkv != 0, B < 1, D not in
 *   {64, 128}, max_context_len > MB * B, ...), PKV_EUNSUPPORTED,
 *   PKV_EWORKSPACE, PKV_EHIP.
 * ------------------------------------------------------------------------ */

/* Workspace bytes for any decode call (pkv_paged_attention_decode or
 * pkv_decode_step) with these sizes and any h_kv that divides h_q, the
 * library choosing the split count; 0 for invalid sizes. */
size_t pkv_decode_workspace_bytes(int num_seqs, int h_q, int head_dim, int max_context_len, int block_size);

pkv_status pkv_paged_attention_decode(void* out, pkv_dtype out_dtype,
                                      const void* q, pkv_dtype q_dtype,
                                      const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                      float k_scale, float v_scale,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int num_seqs, int h_q, int h_kv, int head_dim, int block_size,
                                      int num_blocks, int max_blocks_per_seq, int max_context_len,
                                      float scale, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* ------------------------------------------------------------------------
 * Split-count tuning (tests, sweeps): the same decode with a forced count of
 * workgroups per (sequence, KV head).
 *
 * num_splits: 0 lets the library choose (exactly the calls above); a
 *   positive value forces that count.
 * pkv_decode_workspace_bytes_splits: the workspace such a call needs (h_kv
 *   given); 0 for invalid sizes.
 * pkv_decode_num_splits: the split count the library will use for these
 *   sizes (>= 1), or 0 if invalid.
 * ------------------------------------------------------------------------ */
size_t pkv_decode_workspace_bytes_splits(int num_seqs, int h_q, int h_kv, int head_dim, int block_size,
                                         int max_context_len, int num_splits);

int pkv_decode_num_splits(int num_seqs, int h_q, int h_kv, int head_dim, int block_size,
                          int max_context_len, int num_splits);

pkv_status pkv_paged_attention_decode_splits(void* out, pkv_dtype out_dtype,
                                             const void* q, pkv_dtype q_dtype,
                                             const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                             float k_scale, float v_scale,
                                             const int32_t* block_tables, const int32_t* context_lens,
                                             int num_seqs, int h_q, int h_kv, int head_dim, int block_size,
                                             int num_blocks, int max_blocks_per_seq, int max_context_len,
                                             float scale, int num_splits,
                                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops or harnesses that forbid allocation): the
 * same computation, bits and arguments as pkv_paged_attention_decode, with
 * no workspace argument.  The library uses its own workspace instead, a
 * device array of 64 MiB that each GPU the library runs on holds from the
 * first such call until the process ends; the call allocates nothing.
 * Its counters take at most 65,536 (sequence, KV head) pairs, and the
 * partial states of the split over blocks must fit the rest of the array
 * (about num_seqs * h_q * splits * (head_dim + 2) * 4 bytes, splits being
 * the library's choice); larger calls return PKV_EWORKSPACE before any
 * launch.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (on different streams, or from different threads)
 * race and give undefined results.  The first call on each GPU also clears
 * the counters with a small kernel on `stream`.
 * Errors: as for pkv_paged_attention_decode.
 * ------------------------------------------------------------------------ */
pkv_status pkv_paged_attention_decode_noalloc(void* out, pkv_dtype out_dtype,
                                              const void* q, pkv_dtype q_dtype,
                                              const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                              float k_scale, float v_scale,
                                              const int32_t* block_tables, const int32_t* context_lens,
                                              int num_seqs, int h_q, int h_kv, int head_dim, int block_size,
                                              int num_blocks, int max_blocks_per_seq, int max_context_len,
                                              float scale, hipStream_t stream);

/* ------------------------------------------------------------------------
 * One decode step in one launch: each sequence's new token is written into
 * its slot and attention runs over the context that includes it.
 *
 * Same result, bit for bit, as pkv_reshape_and_cache of new_k / new_v into
 * the slots of positions context_lens[s] - 1 followed by
 * pkv_paged_attention_decode, without the separate launch: the workgroup
 * that reads a sequence's last position writes the new token there itself,
 * and uses the rows it wrote for that position.
 *   new_k, new_v  [S, Hkv, D] in new_dtype: the K/V of each sequence's new
 *                 token, which is position context_lens[s] - 1 (its slot
 *                 comes from block_tables; the block holding it must not be
 *                 shared with another sequence, which copy-on-write ensures).
 *                 new_dtype == kv_dtype copies the bits; an FP8_E4M3 pool
 *                 takes F32 / F16 / BF16 with the scatter's rounding
 *                 (x / k_scale or x / v_scale).  A sequence with context
 *                 length 0 has no new token and gets output 0.  A sequence
 *                 whose context length exceeds MB * B (its table cannot hold
 *                 the position) is attended over its MB * B cached tokens and
 *                 its new token is not written.
 *   other arguments as for pkv_paged_attention_decode (same workspace).
 * Supported: the matrix-core combinations of decode, with new_k / new_v
 *   under 2 GiB each; others return PKV_EUNSUPPORTED (use the two calls).
 *   Errors as for decode, plus PKV_EINVAL for NULL new_k / new_v with S > 0.
 * pkv_decode_step_splits forces the split count as
 *   pkv_paged_attention_decode_splits does (its workspace sizing too).
 * ------------------------------------------------------------------------ */
pkv_status pkv_decode_step(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                           const void* new_k, const void* new_v, pkv_dtype new_dtype,
                           void* k_cache, void* v_cache, pkv_dtype kv_dtype, float k_scale, float v_scale,
                           const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int h_q,
                           int h_kv, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                           int max_context_len, float scale, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

pkv_status pkv_decode_step_splits(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                  const void* new_k, const void* new_v, pkv_dtype new_dtype,
                                  void* k_cache, void* v_cache, pkv_dtype kv_dtype, float k_scale, float v_scale,
                                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int h_q,
                                  int h_kv, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                                  int max_context_len, float scale, int num_splits, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Paged attention for several new query tokens per sequence (a chunk of a
 * prompt recomputed over a cached prefix, or the lookahead tokens of
 * speculative decoding), with a causal mask.
 *
 * Every token already processed keeps its K/V so that later tokens can
 * attend to it ("AI Engineering Visualised: KV cache", intro); a prompt
 * whose prefix is found in the cache recomputes only its trailing tokens
 * over that prefix ("KV cache and PagedAttention in serving", section
 * "Beyond paging: radix trees and continuous batching"); speculative
 * decoding places lookahead tokens in slots past the committed ones ("Paged
 * KV Cache" tutorial, section "Internal Fragmentation").
 *
 * Shapes (T = num_query_tokens, others as for decode):
 *   out, q        [T, Hq, D]   rows query_start[s] .. query_start[s+1]-1 are
 *                              the m_s new tokens of sequence s, in order
 *   query_start   [S + 1] int32, device memory, non-decreasing; entries are
 *                              clamped into [0, T] and m_s to max_query_len,
 *                              so no row outside [0, T) is read or written
 *                              (rows cut off this way are left untouched)
 *   k_cache ...   as for decode; context_lens[s] counts the cached tokens
 *                              INCLUDING the m_s new ones, whose K/V must
 *                              already be in their slots (reshape_and_cache)
 * Semantics: query token i of sequence s sits at position
 *   p = ctx_s - m_s + i and attends to positions [0, p] (itself included):
 *   out[q0 + i, g, :] = sum_{t <= p} softmax_t(scale q . K_s[h, t]) V_s[h, t]
 * with q0 = query_start[s] and h = g / (Hq / Hkv).  A row with p < 0 (more
 * new tokens than cached ones) attends over nothing and gets 0.  m_s = 1 and
 * query_start[s] = s give exactly the decode call.
 *
 * Supported: the matrix-core combinations of decode (16-bit or FP8 caches,
 * B a multiple of 16 with B / 16 a power of two, 1 <= Hq / Hkv <= 16);
 * others return PKV_EUNSUPPORTED.  D must be 64 or 128, as for decode.  The
 * (query token, head) rows of one (sequence, KV head) are processed 16 at a
 * time.
 * max_query_len: 1 <= max_query_len <= 2^24, an upper bound of every m_s.
 * Workspace: pkv_multi_workspace_bytes(...) bytes for the same sizes, zeroed
 *   before first use and reusable afterwards, as for decode.
 * Errors: PKV_EINVAL (as decode, plus NULL query_start with S > 0, T < 0,
 *   max_query_len out of range), PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_EHIP.
 * ------------------------------------------------------------------------ */
size_t pkv_multi_workspace_bytes(int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int max_query_len,
                                 int max_context_len, int num_splits);

/* The split count the library will use for these sizes (>= 1), or 0 if invalid. */
int pkv_multi_num_splits(int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int max_query_len,
                         int max_context_len, int num_splits);

pkv_status pkv_paged_attention_multi(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                     const int32_t* query_start, int num_query_tokens, int max_query_len,
                                     const void* k_cache, const void* v_cache, pkv_dtype kv_dtype, float k_scale,
                                     float v_scale, const int32_t* block_tables, const int32_t* context_lens,
                                     int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int num_blocks,
                                     int max_blocks_per_seq, int max_context_len, float scale, int num_splits,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * reshape_and_cache: write each new token's K and V into its slot.
 *
 * A slot is physical_block * block_size + offset_in_block; token i's K for
 * KV head h lands at k_cache[slot_i / B, h, slot_i % B, :] (same for V).  A
 * sequence grows by claiming free blocks without moving earlier ones ("Paged
 * KV Cache" tutorial, section "Answer Key", question 2), so a new token only
 * ever writes its own slot.
 *   key, value    [T, Hkv, D] in in_dtype (T = num_tokens)
 *   slot_mapping  [T] int64; slot < 0 marks padding (skipped); a slot outside
 *                 [0, NB * B) is skipped too.  Two tokens must not share a slot.
 *   k_cache ...   [NB, Hkv, B, D] in kv_dtype
 * Conversion: in_dtype == kv_dtype copies the bits; kv_dtype FP8_E4M3 takes
 *   in_dtype F32 / F16 / BF16 and stores round-to-nearest-even(x / scale) with
 *   one correctly rounded binary32 division, saturating to +-448, NaN -> 0x7F.
 * D must be a multiple of 8.  Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP.
 * ------------------------------------------------------------------------ */
pkv_status pkv_reshape_and_cache(const void* key, const void* value, pkv_dtype in_dtype,
                                 void* k_cache, void* v_cache, pkv_dtype kv_dtype,
                                 float k_scale, float v_scale,
                                 const int64_t* slot_mapping, int num_tokens,
                                 int h_kv, int head_dim, int block_size, int num_blocks, hipStream_t stream);

/* ------------------------------------------------------------------------
 * copy_blocks: the block copy of copy-on-write.
 *
 * Sequences share prefix blocks by reference; a sequence that appends into a
 * shared block that is only partly filled moves onto a fresh block first
 * ("Paged KV Cache" tutorial, section "Block Tables and Sharing"; "KV cache
 * and PagedAttention in serving", section "The bonus: sharing via
 * copy-on-write").  pkv_bm_append reports that move as (cow_src, cow_dst);
 * this call copies block src to block dst, every KV head and slot, in both
 * pools, so that the sequence's tokens are in its new block before its new
 * token is written (call it before pkv_reshape_and_cache on the same stream).
 *   block_pairs  [num_pairs, 2] int32 in device memory: (src, dst) per row.
 *                All rows see the pools as they were before the call: a
 *                block must not be both a source and a destination, and a
 *                destination must not repeat (caller error, not checked).
 *                A row with an id outside [0, num_blocks) is skipped.
 *   k_cache ...  [NB, Hkv, B, D] in kv_dtype; h_kv * B * D * element bytes
 *                must be a multiple of 16.
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP.
 * ------------------------------------------------------------------------ */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, pkv_dtype kv_dtype, const int32_t* block_pairs,
                           int num_pairs, int h_kv, int head_dim, int block_size, int num_blocks,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * swap_blocks: move whole blocks between two pools, typically a device pool
 * and a pool in pinned host memory.
 *
 * When the device pool fills, a sequence can be preempted by moving its KV
 * blocks to host memory over PCIe and paging them back later instead of
 * recomputing them ("KV cache and PagedAttention in serving", section
 * "Beyond paging: radix trees and continuous batching"); every such transfer
 * costs interconnect bandwidth and time ("Paged KV Cache" tutorial, section
 * "Offload").  One call moves any number of scattered blocks in one launch:
 * block src of the source pools goes to block dst of the destination pools,
 * every KV head and slot, K and V.
 *   dst_k, dst_v  [dst_num_blocks, Hkv, B, D] in kv_dtype
 *   src_k, src_v  [src_num_blocks, Hkv, B, D] in kv_dtype
 *   block_pairs   [num_pairs, 2] int32: (src block, dst block) per row; a
 *                 row with an id outside its pool is skipped; a destination
 *                 must not repeat, and the two pools must not overlap
 *                 (caller errors, not checked).
 * Every pointer must be memory of the current device or pinned host memory
 * (hipHostMalloc, or a tensor allocated pinned); pageable memory and other
 * devices' memory return PKV_EINVAL before anything is launched.  The copy
 * is ordered on `stream`; host memory it writes is complete once the stream
 * has been synchronised.  h_kv * B * D * element bytes must be a multiple of
 * 16.  Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP.
 * ------------------------------------------------------------------------ */
pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, int dst_num_blocks, const void* src_k, const void* src_v,
                           int src_num_blocks, pkv_dtype kv_dtype, const int32_t* block_pairs, int num_pairs,
                           int h_kv, int head_dim, int block_size, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Host block manager (no device memory; pure host bookkeeping)
 *
 * Blocks are handed out only as a sequence grows ("AI Engineering
 * Visualised: KV cache", intro), one by one, and a sequence's earlier blocks
 * never move ("Paged KV Cache" tutorial, "Answer Key", question 2); a block
 * returns to the free list once nothing references it, and sequences share
 * prefix blocks by reference count, a sequence that appends into a shared,
 * partly filled last block first moving to a block of its own (same
 * tutorial, "Block Tables and Sharing"; "KV cache and PagedAttention in
 * serving", "The bonus: sharing via copy-on-write").
 *
 * Policy: the free list is FIFO (take from the front, released blocks go to
 * the back, a freed sequence releases in block-table order), seeded by
 * `free_order` (a permutation of [0, num_blocks); NULL means ascending).
 * Sequence ids are any non-negative int32.  Not thread-safe per manager.
 * ------------------------------------------------------------------------ */
typedef struct pkv_bm pkv_bm;

/* Create a manager; *out receives it.  PKV_EINVAL on bad sizes or a
 * free_order that is not a permutation. */
pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pkv_bm** out);
void pkv_bm_destroy(pkv_bm* bm);

/* Append n_tokens tokens to seq (created empty if new).  slots_out (may be
 * NULL) receives the n_tokens slots in order.  If the sequence's last block
 * is partly filled and shared, the sequence first moves to a fresh block:
 * *cow_src / *cow_dst (may be NULL) receive the old and new block ids and
 * the caller must copy the filled slots of src into dst; otherwise both are
 * -1.  PKV_ENOSPC if the pool cannot supply every block needed (nothing
 * changes); PKV_EINVAL for seq < 0 or n_tokens < 0. */
pkv_status pkv_bm_append(pkv_bm* bm, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                         int32_t* cow_src, int32_t* cow_dst);

/* child becomes a copy of parent sharing all its blocks (refcounts + 1).
 * PKV_EINVAL if parent is unknown or child exists. */
pkv_status pkv_bm_fork(pkv_bm* bm, int32_t parent, int32_t child);

/* Drop seq; blocks whose refcount reaches zero go to the back of the free
 * list in block-table order.  PKV_EINVAL if seq is unknown. */
pkv_status pkv_bm_free(pkv_bm* bm, int32_t seq);

/* Copy seq's block table (up to cap entries) into out; *n_blocks and
 * *n_tokens receive its length in blocks and tokens.  PKV_EINVAL if unknown
 * or cap is too small. */
pkv_status pkv_bm_block_table(const pkv_bm* bm, int32_t seq, int32_t* out, int32_t cap,
                              int32_t* n_blocks, int32_t* n_tokens);

/* Fill the device-bound metadata of a batch: tables [num_seqs, max_blocks]
 * (unused entries -1) and context_lens [num_seqs] for the listed sequences.
 * PKV_EINVAL if a sequence is unknown or longer than max_blocks blocks. */
pkv_status pkv_bm_export(const pkv_bm* bm, const int32_t* seqs, int32_t num_seqs,
                         int32_t* tables, int32_t max_blocks, int32_t* context_lens);

int32_t pkv_bm_num_free(const pkv_bm* bm);
/* Reference count of a block (0 = free), or -1 for an id outside the pool. */
int32_t pkv_bm_refcount(const pkv_bm* bm, int32_t block);
/* Copy the free list, front first (up to cap entries); *n receives its length. */
pkv_status pkv_bm_free_list(const pkv_bm* bm, int32_t* out, int32_t cap, int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
