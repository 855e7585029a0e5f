// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kDecodeWaves = 4;        // waves per decode workgroup
constexpr int kDecodeThreads = 64 * kDecodeWaves;
constexpr int kTileTokens = 16;        // tokens per matrix-core tile
constexpr int kMaxGroup = 16;          // query heads per KV head handled by one workgroup
// Waves per SIMD the matrix-core decode kernel is built for (its register
// budget: 512 / this many VGPRs per lane).
constexpr int kDecodeWavesPerSimd = 3;
// Balanced ranges (decode over few (sequence, KV head) pairs with long
// contexts): at most this many sequences (their tile counts' prefix sums sit
// in LDS), and ranges of at least this many 16-token tiles.
constexpr int kBalancedMaxSeqs = 1024;
constexpr int kBalancedMinRange = 64;
// Compute units of an MI355X (the work-split models assume a whole GPU;
// pacing checks that the device reports this many).
constexpr int kComputeUnits = 256;
// Longest pairs first (decode grids that do not fit on the GPU at once): at
// most this many sequences, ranked by tile count in this many bins (LDS).
constexpr int kLptMaxSeqs = 1024;
constexpr int kLptBins = 2048;
static_assert(kLptMaxSeqs % kDecodeThreads == 0 && kLptBins % kDecodeThreads == 0,
              "the ranking gives every thread the same number of sequences and bins");
static_assert(kDecodeWaves <= 4, "the ranking's workgroup scan keeps one partial per wave in 4 LDS slots");

struct DecodeLaunch {
  void* out;
  int out_dtype;
  const void* q;
  int q_dtype;
  const void* k_cache;
  const void* v_cache;
  int kv_dtype;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs, h_q, h_kv, head_dim, block_size, num_blocks, max_blocks_per_seq;
  int num_splits;       // workgroups per (sequence, KV head)
  int tiles_per_split;  // upper bound of 16-token tiles per workgroup
  float scale_log2;     // logit scale * log2(e), times k_scale for FP8 caches
  float v_scale;        // output scale (FP8 V), else 1
  void* workspace;
  bool matrix_core;     // MFMA path (else the vector path)
  // Several query tokens per sequence (query_start != nullptr; matrix-core
  // path only): q and out are [num_query_tokens, h_q, head_dim], the rows of
  // sequence s are [query_start[s], query_start[s + 1]), at most max_query_len.
  const int32_t* query_start;
  int num_query_tokens, max_query_len;
  // Decode step that appends the new tokens itself (new_k != nullptr;
  // matrix-core path, one query token): new_k, new_v [num_seqs, h_kv,
  // head_dim] in new_dtype are written to position context_lens[s] - 1, FP8
  // pools dividing by k_scale_enc / v_scale_enc as the scatter does.
  const void* new_k;
  const void* new_v;
  int new_dtype;
  float k_scale_enc, v_scale_enc;
  // Balanced ranges (decode only, matrix-core path; 0 = one workgroup per
  // (sequence, KV head, split)): the grid, every workgroup one equal range of
  // all pairs' tiles.
  int balanced_workgroups;
  // Longest pairs first (decode, one workgroup per (sequence, KV head,
  // split)): -1 = workgroups take pairs in (sequence, KV head) order; else
  // sequences are taken in decreasing order of their tile count shifted
  // right by this many bits (ties in index order).
  int lpt_shift = -1;
  // Pacing (one workgroup per pair, split and row group): when the
  // grid holds more workgroups than the GPU has CUs but fewer than twice as
  // many, the dispatcher puts workgroups 0 .. kComputeUnits - 1 on CUs of
  // their own and the rest beside the first ones, so workgroups grid -
  // kComputeUnits .. kComputeUnits - 1 have a CU to themselves.  Those
  // pace their tiles, leaving HBM to the CUs that hold two workgroups; the
  // launch does so for grids of at most 1.5 times the CUs (at most half of
  // them shared: beyond that pacing measured no gain) whose pairs hold at
  // least 8 tiles per wave.  This flag says the call's kernel kind may be
  // paced; the launch checks the rest.
  bool pace = false;
  // Counters region of the workspace, in int32 slots: 0 sizes it for this
  // call's units; a fixed capacity (the library's own workspace) keeps the
  // partial states of every call clear of the counters of any other.
  int counter_slots = 0;
  // K/V tiles straight into an LDS ring (one-row-tile kernels over 16-bit
  // caches with head_dim 128, one workgroup per (sequence, KV head, split)):
  // chosen for grids that run in several rounds anyway.
  bool lds_ring = false;
};

// 16-row tiles of (query token, query head) rows per (sequence, KV head).
inline int multi_row_tiles(int h_q, int h_kv, int max_query_len) {
  return (int)(((int64_t)max_query_len * (h_q / h_kv) + 15) / 16);
}

// Row tiles one workgroup holds with several query tokens: two (one walk of
// the K/V for 32 rows) when there are two or more, else one.
inline int multi_tiles_per_workgroup(int row_tiles) { return row_tiles >= 2 ? 2 : 1; }

// Workgroups per (sequence, KV head, split) with several query tokens.
inline int multi_row_groups(int row_tiles) {
  const int t = multi_tiles_per_workgroup(row_tiles);
  return (row_tiles + t - 1) / t;
}

// Byte layout of the decode workspace.
struct WorkspaceLayout {
  size_t counters;  // int32 [units]
  size_t ml;        // float2 [units, splits, G]  (running max, running sum)
  size_t acc;       // float [units, splits, G, D]
  size_t total;
};

// balanced_workgroups > 0: the layout of balanced ranges (two partial-state
// slots per workgroup) instead of one per (sequence, KV head, split).
// counter_slots > 0: a counters region of that many int32 slots (at least the
// call's units) instead of one sized for the call.
WorkspaceLayout decode_workspace_layout(int num_seqs, int h_q, int h_kv, int head_dim, int num_splits,
                                        int balanced_workgroups = 0, int counter_slots = 0);

// The library's own decode workspace for callers that cannot allocate: a
// file-scope device array of kStaticWorkspaceBytes per GPU, whose first
// kStaticCounterSlots int32 slots are the counters (zeroed once, on the
// first use on each device, by a fill kernel on `stream`; every call leaves
// them zero) and the rest the partial states.  *ptr receives this device's
// address of the array.
constexpr size_t kStaticWorkspaceBytes = size_t(64) << 20;
constexpr int kStaticCounterSlots = 1 << 16;
hipError_t static_workspace(hipStream_t stream, void** ptr);

// Workspace of a call with several query tokens per sequence: one counter
// and 16 partial-state rows per split for each (sequence, KV head, row tile),
// (sequence, KV head) pairs counted in whole groups of 8; with balanced
// ranges (balanced_workgroups > 0, one row group), one counter per (pair,
// row tile) and two partial-state slots of 16 rows per row tile per range.
WorkspaceLayout multi_workspace_layout(int num_seqs, int h_kv, int head_dim, int row_tiles, int num_splits,
                                       int balanced_workgroups = 0);

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, int in_dtype, void* k_cache, void* v_cache,
                                    int kv_dtype, float k_scale, float v_scale, const int64_t* slot_mapping,
                                    int num_tokens, int h_kv, int head_dim, int block_size, int num_blocks,
                                    hipStream_t stream);

// Block copies between pools (the same pools for copy-on-write): row i of
// pairs is (src block, dst block); ids outside their pool are skipped.
hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int32_t* pairs,
                              int num_pairs, int64_t block_bytes, int src_blocks, int dst_blocks,
                              hipStream_t stream);

}  // namespace pkv
