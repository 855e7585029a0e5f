// C ABI of libpkv: argument validation, work-split choice and kernel dispatch.
// The declarations in include/pkv.h document every entry point.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

// Workgroups the split model lets run at once: two per CU.  A CU holds
// three of the decode kernel's, but a third walking K/V beside two slows them
// more than the smaller ranges gain (32K-token FP8 batch, 256 (sequence, KV
// head) pairs: 2 splits 261.6 us, 3 splits 277.8 us per launch), and the
// kernel with two row tiles per workgroup holds two.
constexpr int64_t kResidentWorkgroups = 256 * 2;

bool valid_dtype(int d) { return d >= PKV_F32 && d <= PKV_FP8_E4M3; }

// Compute units of the current device, queried once per device (0 if the
// query fails).  Pacing rests on the dispatch placement and the shares
// measured on a whole MI355X (pkv::kComputeUnits CUs): a device that reports
// another count (a partition of the GPU, say) runs unpaced.
int current_device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0: not queried yet
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of workgroups that share one (sequence, KV head): minimise
// (rounds of resident workgroups) x (time of one workgroup), the time counted
// in 16-token tiles per wave plus fixed costs measured on MI355X: about two
// tiles' worth for a workgroup's start (context length, block ids, first
// tile) and about six for the cross-split merge of partial states.  Ties go
// to the smaller count.
constexpr int64_t kStartCost = 2;
constexpr int64_t kMergeCost = 6;

int choose_splits(int64_t units, int64_t max_tiles) {
  if (max_tiles <= 1 || units <= 0) return 1;
  const int64_t cap = std::max<int64_t>(1, std::min<int64_t>(64, ceil_div(max_tiles, 8)));
  const int64_t padded_units = ceil_div(units, 8) * 8;
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int64_t n = 1; n <= cap; ++n) {
    const int64_t rounds = ceil_div(padded_units * n, kResidentWorkgroups);
    const int64_t per_wave = ceil_div(ceil_div(max_tiles, n), pkv::kDecodeWaves);
    const int64_t cost = rounds * (per_wave + kStartCost + (n > 1 ? kMergeCost : 0));
    if (cost < best_cost) {
      best_cost = cost;
      best = (int)n;
    }
  }
  return best;
}

// Balanced ranges for decode (the grid, or 0 for one workgroup per
// (sequence, KV head, split)): when few pairs (at most two per CU) carry long
// contexts (256 tiles or more), one workgroup per pair and split leaves the
// work as uneven as the context lengths; equal ranges of all pairs' tiles do
// not (32K-token FP8 batch: the longest wave had twice the median's tiles).
// Only when the split count is the library's choice, for at most
// kBalancedMaxSeqs sequences, and with all tiles countable in an int.
int balanced_workgroups(int num_seqs, int h_kv, int max_context_len, int num_splits) {
  const int64_t units = (int64_t)num_seqs * h_kv;
  const int64_t max_tiles = ceil_div(std::max(max_context_len, 0), pkv::kTileTokens);
  if (num_splits > 0 || num_seqs > pkv::kBalancedMaxSeqs || units > kResidentWorkgroups || max_tiles < 256) return 0;
  if (units * max_tiles >= INT32_MAX) return 0;
  return (int)std::min<int64_t>(kResidentWorkgroups, ceil_div(units * max_tiles, pkv::kBalancedMinRange));
}

// Workgroups of a decode launch with one workgroup per (sequence, KV head,
// row group, split), the pairs counted in whole groups of 8.
int64_t decode_grid(int num_seqs, int h_kv, int row_groups, int splits) {
  return ceil_div((int64_t)num_seqs * h_kv, 8) * 8 * row_groups * splits;
}

// Longest pairs first (the bin shift, or -1 for pairs in order): when a
// decode grid of one workgroup per (sequence, KV head, split) does not fit on
// the GPU at once, workgroups that start late should hold the short pairs.
// Only when the split count is the library's choice, for at most
// kLptMaxSeqs sequences (every workgroup ranks them all).
int longest_first_shift(int num_seqs, int h_kv, int max_context_len, int num_splits, int chosen_splits,
                        int row_groups, int waves_per_simd) {
  const int64_t grid = decode_grid(num_seqs, h_kv, row_groups, chosen_splits);
  if (num_splits > 0 || num_seqs > pkv::kLptMaxSeqs || grid <= (int64_t)pkv::kComputeUnits * waves_per_simd)
    return -1;
  const int64_t max_tiles = ceil_div(std::max(max_context_len, 0), pkv::kTileTokens);
  int shift = 0;
  while ((max_tiles >> shift) >= pkv::kLptBins) ++shift;
  return shift;
}

// The kernels with an LDS ring for K/V (one row tile, 16-bit caches, rows of
// 128 elements, no balanced ranges).  Their ring takes 64 KiB of LDS per
// workgroup, so two workgroups share a CU instead of three: they are taken
// only for grids that need several rounds at three per CU, where they
// measured faster (8B mixed-length and MHA batches, 2,048 workgroups); on a
// grid resident in one round the register ring measured as fast or faster.
bool lds_ring_fits(bool matrix_core, int balanced, int kv_dtype, int head_dim, bool multi, int row_tiles) {
  const bool one_row_tile = !multi || pkv::multi_tiles_per_workgroup(row_tiles) == 1;
  return matrix_core && balanced == 0 && (kv_dtype == PKV_BF16 || kv_dtype == PKV_F16) && head_dim == 128 &&
         one_row_tile;
}

int resolve_splits(int num_seqs, int h_kv, int max_context_len, int num_splits) {
  const int64_t max_tiles = ceil_div(std::max(max_context_len, 0), pkv::kTileTokens);
  int n = num_splits > 0 ? num_splits : choose_splits((int64_t)num_seqs * h_kv, max_tiles);
  return std::max(1, n);
}

// Attention kernels are built for these head dims; another one is an
// invalid argument, not a combination left out.
bool attention_head_dim(int head_dim) { return head_dim == 64 || head_dim == 128; }

bool decode_shape_ok(int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int max_context_len,
                     int num_splits) {
  return num_seqs >= 0 && h_q >= 1 && h_kv >= 1 && h_q % h_kv == 0 && attention_head_dim(head_dim) &&
         block_size >= 1 && max_context_len >= 0 && num_splits >= 0;
}

// The address a kernel on the current device uses for p: p itself for memory
// of that device, the mapped address for pinned host memory; false for
// pageable host memory, other devices' memory, or anything unknown.
bool device_address(const void* p, void** out) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // keep the failed query from surfacing at the next launch
    return false;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (a.type == hipMemoryTypeDevice && a.device == dev && a.devicePointer != nullptr) {
    *out = const_cast<void*>(p);
    return true;
  }
  if (a.type == hipMemoryTypeHost && a.devicePointer != nullptr) {
    // the mapped address of p itself, whether the runtime reports the two
    // addresses at p or at the start of the allocation
    const char* host = a.hostPointer ? static_cast<const char*>(a.hostPointer) : static_cast<const char*>(p);
    *out = static_cast<char*>(a.devicePointer) + (static_cast<const char*>(p) - host);
    return true;
  }
  return false;
}

// Upper bound of max_query_len (keeps every row and grid count within int).
constexpr int kMaxQueryLen = 1 << 24;

bool multi_shape_ok(int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int max_query_len,
                    int max_context_len, int num_splits) {
  return decode_shape_ok(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, num_splits) &&
         max_query_len >= 1 && max_query_len <= kMaxQueryLen;
}

// Splits for several query tokens: the units are (sequence, KV head, row
// group), a row group being the row tiles one workgroup holds.
int resolve_multi_splits(int num_seqs, int h_q, int h_kv, int max_query_len, int max_context_len, int num_splits) {
  const int64_t max_tiles = ceil_div(std::max(max_context_len, 0), pkv::kTileTokens);
  const int row_tiles = pkv::multi_row_tiles(h_q, h_kv, max_query_len);
  const int64_t units = (int64_t)num_seqs * h_kv * pkv::multi_row_groups(row_tiles);
  int n = num_splits > 0 ? num_splits : choose_splits(units, max_tiles);
  return std::max(1, n);
}

// Decode (query_start == nullptr: one query token per sequence) and calls
// with several query tokens per sequence share validation and launch.
pkv_status run_attention(void* out, int out_dtype, const void* q, int q_dtype, const int32_t* query_start,
                         int num_query_tokens, int max_query_len, const void* new_k, const void* new_v,
                         int new_dtype, const void* k_cache, const void* v_cache, int kv_dtype, float k_scale,
                         float v_scale, const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                         int h_q, int h_kv, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                         int max_context_len, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, bool own_workspace = false) {
  const bool multi = query_start != nullptr;
  const bool append = new_k != nullptr;
  if (!decode_shape_ok(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, num_splits)) return PKV_EINVAL;
  if (num_blocks < 1 || max_blocks_per_seq < 1) return PKV_EINVAL;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PKV_EINVAL;
  if (!valid_dtype(out_dtype) || !valid_dtype(q_dtype) || !valid_dtype(kv_dtype)) return PKV_EINVAL;
  if (num_seqs == 0 || (multi && num_query_tokens == 0)) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_EINVAL;
  if (!own_workspace && !workspace) return PKV_EINVAL;
  if (!(std::isfinite(scale))) return PKV_EINVAL;
  if (kv_dtype == PKV_FP8_E4M3 && !(k_scale > 0.f && std::isfinite(k_scale) && v_scale > 0.f && std::isfinite(v_scale)))
    return PKV_EINVAL;

  if (h_q / h_kv > pkv::kMaxGroup) return PKV_EUNSUPPORTED;
  if (out_dtype == PKV_FP8_E4M3 || q_dtype == PKV_FP8_E4M3) return PKV_EUNSUPPORTED;
  const bool pair_ok = (q_dtype == kv_dtype) || (kv_dtype == PKV_FP8_E4M3 && q_dtype != PKV_F32);
  if (!pair_ok) return PKV_EUNSUPPORTED;

  // matrix-core path: 16-bit or FP8 caches whose blocks hold a power-of-two
  // number of 16-token tiles; everything else takes the vector path, which
  // serves one query token per sequence only
  const int tiles_per_block = block_size / pkv::kTileTokens;
  const bool matrix_core = kv_dtype != PKV_F32 && block_size % pkv::kTileTokens == 0 &&
                           (tiles_per_block & (tiles_per_block - 1)) == 0;
  if (multi && !matrix_core) return PKV_EUNSUPPORTED;
  if (append) {
    if (!matrix_core) return PKV_EUNSUPPORTED;
    if (!valid_dtype(new_dtype)) return PKV_EINVAL;
    const bool enc_ok = new_dtype == kv_dtype || (kv_dtype == PKV_FP8_E4M3 && new_dtype != PKV_FP8_E4M3);
    if (!enc_ok) return PKV_EUNSUPPORTED;
    // the kernel addresses new_k / new_v through 32-bit buffer offsets
    const int64_t new_bytes = (int64_t)num_seqs * h_kv * head_dim *
                              (new_dtype == PKV_F32 ? 4 : (new_dtype == PKV_FP8_E4M3 ? 1 : 2));
    if (new_bytes > INT32_MAX) return PKV_EUNSUPPORTED;
  }

  const int n = multi ? resolve_multi_splits(num_seqs, h_q, h_kv, max_query_len, max_context_len, num_splits)
                      : resolve_splits(num_seqs, h_kv, max_context_len, num_splits);
  const int row_tiles = multi ? pkv::multi_row_tiles(h_q, h_kv, max_query_len) : 1;
  const int row_groups = multi ? pkv::multi_row_groups(row_tiles) : 1;
  if ((int64_t)ceil_div((int64_t)num_seqs * h_kv, 8) * 8 * row_groups * n > INT32_MAX) return PKV_EUNSUPPORTED;
  // balanced ranges: decode, and several query tokens whose rows of a pair
  // fit one workgroup (one row group)
  int balanced = matrix_core && row_groups == 1 ? balanced_workgroups(num_seqs, h_kv, max_context_len, num_splits) : 0;
  // balanced ranges count every pair's tiles up to the table's capacity in an
  // int (a context may exceed max_context_len); otherwise one workgroup per
  // pair and split, whose layout the workspace size also covers
  if (balanced > 0 && (int64_t)num_seqs * h_kv *
                              ceil_div((int64_t)max_blocks_per_seq * block_size, pkv::kTileTokens) >= INT32_MAX)
    balanced = 0;
  // the library's own workspace (decode only) keeps a counters region of
  // fixed capacity, so that no call's partial states overlap another's counters
  const int counter_slots = own_workspace ? pkv::kStaticCounterSlots : 0;
  if (own_workspace && (multi || (int64_t)num_seqs * h_kv > counter_slots)) return PKV_EWORKSPACE;
  const pkv::WorkspaceLayout L =
      multi ? pkv::multi_workspace_layout(num_seqs, h_kv, head_dim, row_tiles, n, balanced)
            : pkv::decode_workspace_layout(num_seqs, h_q, h_kv, head_dim, n, balanced, counter_slots);
  if (own_workspace) {
    if (L.total > pkv::kStaticWorkspaceBytes) return PKV_EWORKSPACE;
    if (pkv::static_workspace(stream, &workspace) != hipSuccess) return PKV_EHIP;
  } else if (workspace_bytes < L.total) {
    return PKV_EWORKSPACE;
  }

  const double s = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)head_dim);
  const double log2e = 1.4426950408889634;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;

  pkv::DecodeLaunch a;
  a.out = out;
  a.out_dtype = out_dtype;
  a.q = q;
  a.q_dtype = q_dtype;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_dtype = kv_dtype;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_splits = n;
  a.tiles_per_split = (int)std::max<int64_t>(1, ceil_div(ceil_div(max_context_len, pkv::kTileTokens), n));
  a.scale_log2 = (float)(s * log2e * (fp8 ? (double)k_scale : 1.0));
  a.v_scale = fp8 ? v_scale : 1.f;
  a.workspace = workspace;
  a.matrix_core = matrix_core;
  a.query_start = query_start;
  a.num_query_tokens = multi ? num_query_tokens : 0;
  a.max_query_len = multi ? max_query_len : 1;
  a.new_k = new_k;
  a.new_v = new_v;
  a.new_dtype = new_dtype;
  a.k_scale_enc = k_scale;
  a.v_scale_enc = v_scale;
  a.balanced_workgroups = balanced;
  a.counter_slots = counter_slots;
  // resident workgroups per SIMD: 2 for the kernels holding two row tiles
  const int waves_per_simd =
      multi && pkv::multi_tiles_per_workgroup(row_tiles) == 2 ? 2 : pkv::kDecodeWavesPerSimd;
  a.lpt_shift = matrix_core && balanced == 0 ? longest_first_shift(num_seqs, h_kv, max_context_len, num_splits, n,
                                                                   row_groups, waves_per_simd)
                                             : -1;
  a.lds_ring = lds_ring_fits(matrix_core, balanced, kv_dtype, head_dim, multi, row_tiles) &&
               decode_grid(num_seqs, h_kv, row_groups, n) > (int64_t)pkv::kComputeUnits * pkv::kDecodeWavesPerSimd;
  a.pace = matrix_core && balanced == 0 && current_device_cus() == pkv::kComputeUnits;
  const hipError_t e = pkv::launch_decode(a, stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

// Workspace of a decode call with h_kv given and the split count forced
// (num_splits > 0) or chosen by the library: enough for either assignment
// (the balanced one is used on the matrix-core path only, which the shape
// alone does not tell).
size_t decode_workspace_bytes(int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int max_context_len,
                              int num_splits) {
  if (!decode_shape_ok(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, num_splits)) return 0;
  const int n = resolve_splits(num_seqs, h_kv, max_context_len, num_splits);
  const int balanced = balanced_workgroups(num_seqs, h_kv, max_context_len, num_splits);
  return std::max(pkv::decode_workspace_layout(num_seqs, h_q, h_kv, head_dim, n).total,
                  pkv::decode_workspace_layout(num_seqs, h_q, h_kv, head_dim, n, balanced).total);
}

}  // namespace

extern "C" {

const char* pkv_status_str(pkv_status status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_EINVAL: return "PKV_EINVAL: invalid argument";
    case PKV_EUNSUPPORTED: return "PKV_EUNSUPPORTED: combination not built";
    case PKV_ENOSPC: return "PKV_ENOSPC: not enough free blocks";
    case PKV_EWORKSPACE: return "PKV_EWORKSPACE: workspace too small";
    case PKV_EHIP: return "PKV_EHIP: HIP runtime error";
    default: return "unknown pkv status";
  }
}

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

int pkv_decode_num_splits(int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int max_context_len,
                          int num_splits) {
  if (!decode_shape_ok(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, num_splits)) return 0;
  const int balanced = balanced_workgroups(num_seqs, h_kv, max_context_len, num_splits);
  if (balanced > 0) return (int)ceil_div(balanced, (int64_t)num_seqs * h_kv);  // workgroups per pair, on average
  return resolve_splits(num_seqs, h_kv, max_context_len, num_splits);
}

size_t pkv_decode_workspace_bytes(int num_seqs, int h_q, int head_dim, int max_context_len, int block_size) {
  // the largest workspace over every KV-head count a call with these sizes
  // may pass (the divisors of h_q), each with the library's split choice
  size_t best = 0;
  for (int h_kv = 1; h_kv <= h_q; ++h_kv) {
    if (h_q % h_kv != 0) continue;
    best = std::max(best, decode_workspace_bytes(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, 0));
  }
  return best;
}

size_t pkv_decode_workspace_bytes_splits(int num_seqs, int h_q, int h_kv, int head_dim, int block_size,
                                         int max_context_len, int num_splits) {
  return decode_workspace_bytes(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, num_splits);
}

pkv_status pkv_paged_attention_decode(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                      const void* k_cache, const void* v_cache, pkv_dtype kv_dtype, float k_scale,
                                      float v_scale, const int32_t* block_tables, const int32_t* context_lens,
                                      int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int num_blocks,
                                      int max_blocks_per_seq, int max_context_len, float scale, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return run_attention(out, out_dtype, q, q_dtype, nullptr, 0, 1, nullptr, nullptr, 0, k_cache, v_cache, kv_dtype,
                       k_scale, v_scale, block_tables, context_lens, num_seqs, h_q, h_kv, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, 0, workspace, workspace_bytes,
                       stream);
}

pkv_status pkv_paged_attention_decode_splits(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                             const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                             float k_scale, float v_scale, const int32_t* block_tables,
                                             const int32_t* context_lens, int num_seqs, int h_q, int h_kv,
                                             int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                                             int max_context_len, float scale, int num_splits, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  return run_attention(out, out_dtype, q, q_dtype, nullptr, 0, 1, nullptr, nullptr, 0, k_cache, v_cache, kv_dtype,
                       k_scale, v_scale, block_tables, context_lens, num_seqs, h_q, h_kv, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, num_splits, workspace,
                       workspace_bytes, stream);
}

pkv_status pkv_paged_attention_decode_noalloc(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                              const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                              float k_scale, float v_scale, const int32_t* block_tables,
                                              const int32_t* context_lens, int num_seqs, int h_q, int h_kv,
                                              int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                                              int max_context_len, float scale, hipStream_t stream) {
  return run_attention(out, out_dtype, q, q_dtype, nullptr, 0, 1, nullptr, nullptr, 0, k_cache, v_cache, kv_dtype,
                       k_scale, v_scale, block_tables, context_lens, num_seqs, h_q, h_kv, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, 0, nullptr, 0, stream,
                       /*own_workspace=*/true);
}

namespace {
pkv_status decode_step(void* out, int out_dtype, const void* q, int q_dtype, const void* new_k, const void* new_v,
                       int new_dtype, void* k_cache, void* v_cache, int kv_dtype, float k_scale, float v_scale,
                       const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int h_q, int h_kv,
                       int head_dim, int block_size, int num_blocks, int max_blocks_per_seq, int max_context_len,
                       float scale, int num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (num_seqs > 0 && (!new_k || !new_v)) return PKV_EINVAL;
  return run_attention(out, out_dtype, q, q_dtype, nullptr, 0, 1, num_seqs > 0 ? new_k : nullptr, new_v, new_dtype,
                       k_cache, v_cache, kv_dtype, k_scale, v_scale, block_tables, context_lens, num_seqs, h_q,
                       h_kv, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                       num_splits, workspace, workspace_bytes, stream);
}
}  // namespace

pkv_status pkv_decode_step(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* new_k,
                           const void* new_v, pkv_dtype new_dtype, void* k_cache, void* v_cache, pkv_dtype kv_dtype,
                           float k_scale, float v_scale, const int32_t* block_tables, const int32_t* context_lens,
                           int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, int max_context_len, float scale, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return decode_step(out, out_dtype, q, q_dtype, new_k, new_v, new_dtype, k_cache, v_cache, kv_dtype, k_scale,
                     v_scale, block_tables, context_lens, num_seqs, h_q, h_kv, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, 0, workspace, workspace_bytes, stream);
}

pkv_status pkv_decode_step_splits(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                  const void* new_k, const void* new_v, pkv_dtype new_dtype, void* k_cache,
                                  void* v_cache, pkv_dtype kv_dtype, float k_scale, float v_scale,
                                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int h_q,
                                  int h_kv, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                                  int max_context_len, float scale, int num_splits, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return decode_step(out, out_dtype, q, q_dtype, new_k, new_v, new_dtype, k_cache, v_cache, kv_dtype, k_scale,
                     v_scale, block_tables, context_lens, num_seqs, h_q, h_kv, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, num_splits, workspace, workspace_bytes, stream);
}

int pkv_multi_num_splits(int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int max_query_len,
                         int max_context_len, int num_splits) {
  if (!multi_shape_ok(num_seqs, h_q, h_kv, head_dim, block_size, max_query_len, max_context_len, num_splits)) return 0;
  if (pkv::multi_row_groups(pkv::multi_row_tiles(h_q, h_kv, max_query_len)) == 1) {
    const int balanced = balanced_workgroups(num_seqs, h_kv, max_context_len, num_splits);
    if (balanced > 0) return (int)ceil_div(balanced, (int64_t)num_seqs * h_kv);  // workgroups per pair, on average
  }
  return resolve_multi_splits(num_seqs, h_q, h_kv, max_query_len, max_context_len, num_splits);
}

size_t pkv_multi_workspace_bytes(int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int max_query_len,
                                 int max_context_len, int num_splits) {
  if (!multi_shape_ok(num_seqs, h_q, h_kv, head_dim, block_size, max_query_len, max_context_len, num_splits)) return 0;
  const int n = resolve_multi_splits(num_seqs, h_q, h_kv, max_query_len, max_context_len, num_splits);
  const int row_tiles = pkv::multi_row_tiles(h_q, h_kv, max_query_len);
  // enough for either assignment (balanced ranges are taken on the
  // matrix-core path with one row group only)
  const int balanced =
      pkv::multi_row_groups(row_tiles) == 1 ? balanced_workgroups(num_seqs, h_kv, max_context_len, num_splits) : 0;
  return std::max(pkv::multi_workspace_layout(num_seqs, h_kv, head_dim, row_tiles, n).total,
                  pkv::multi_workspace_layout(num_seqs, h_kv, head_dim, row_tiles, n, balanced).total);
}

pkv_status pkv_paged_attention_multi(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                     const int32_t* query_start, int num_query_tokens, int max_query_len,
                                     const void* k_cache, const void* v_cache, pkv_dtype kv_dtype, float k_scale,
                                     float v_scale, const int32_t* block_tables, const int32_t* context_lens,
                                     int num_seqs, int h_q, int h_kv, int head_dim, int block_size, int num_blocks,
                                     int max_blocks_per_seq, int max_context_len, float scale, int num_splits,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!multi_shape_ok(num_seqs, h_q, h_kv, head_dim, block_size, max_query_len, max_context_len, num_splits))
    return PKV_EINVAL;
  if (num_query_tokens < 0) return PKV_EINVAL;
  if (num_seqs > 0 && !query_start) return PKV_EINVAL;
  return run_attention(out, out_dtype, q, q_dtype, query_start, num_query_tokens, max_query_len, nullptr, nullptr, 0,
                       k_cache, v_cache, kv_dtype, k_scale, v_scale, block_tables, context_lens, num_seqs, h_q, h_kv,
                       head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, num_splits,
                       workspace, workspace_bytes, stream);
}

pkv_status pkv_reshape_and_cache(const void* key, const void* value, pkv_dtype in_dtype, void* k_cache,
                                 void* v_cache, pkv_dtype kv_dtype, float k_scale, float v_scale,
                                 const int64_t* slot_mapping, int num_tokens, int h_kv, int head_dim, int block_size,
                                 int num_blocks, hipStream_t stream) {
  if (num_tokens < 0 || h_kv < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1) return PKV_EINVAL;
  if (!valid_dtype(in_dtype) || !valid_dtype(kv_dtype)) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_EINVAL;
  if (kv_dtype == PKV_FP8_E4M3 && in_dtype != PKV_FP8_E4M3 &&
      !(k_scale > 0.f && std::isfinite(k_scale) && v_scale > 0.f && std::isfinite(v_scale)))
    return PKV_EINVAL;
  if (head_dim % 8 != 0) return PKV_EUNSUPPORTED;
  if (in_dtype != kv_dtype && kv_dtype != PKV_FP8_E4M3) return PKV_EUNSUPPORTED;
  const hipError_t e =
      pkv::launch_reshape_and_cache(key, value, in_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, slot_mapping,
                                    num_tokens, h_kv, head_dim, block_size, num_blocks, stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, pkv_dtype kv_dtype, const int32_t* block_pairs,
                           int num_pairs, int h_kv, int head_dim, int block_size, int num_blocks, hipStream_t stream) {
  if (num_pairs < 0 || h_kv < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1) return PKV_EINVAL;
  if (!valid_dtype(kv_dtype)) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_pairs) return PKV_EINVAL;
  static const int kElementBytes[4] = {4, 2, 2, 1};
  const int64_t block_bytes = (int64_t)h_kv * block_size * head_dim * kElementBytes[kv_dtype];
  if (block_bytes % 16 != 0) return PKV_EUNSUPPORTED;
  const hipError_t e = pkv::launch_copy_blocks(k_cache, v_cache, k_cache, v_cache, block_pairs, num_pairs, block_bytes,
                                               num_blocks, num_blocks, stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, int dst_num_blocks, const void* src_k, const void* src_v,
                           int src_num_blocks, pkv_dtype kv_dtype, const int32_t* block_pairs, int num_pairs, int h_kv,
                           int head_dim, int block_size, hipStream_t stream) {
  if (num_pairs < 0 || h_kv < 1 || head_dim < 1 || block_size < 1 || dst_num_blocks < 1 || src_num_blocks < 1)
    return PKV_EINVAL;
  if (!valid_dtype(kv_dtype)) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !block_pairs) return PKV_EINVAL;
  static const int kElementBytes[4] = {4, 2, 2, 1};
  const int64_t block_bytes = (int64_t)h_kv * block_size * head_dim * kElementBytes[kv_dtype];
  if (block_bytes % 16 != 0) return PKV_EUNSUPPORTED;
  // every pointer the kernel follows must be memory of this device or pinned
  // host memory mapped into its address space; anything else is refused here
  void *dk, *dv, *sk, *sv, *pp;
  if (!device_address(dst_k, &dk) || !device_address(dst_v, &dv) || !device_address(src_k, &sk) ||
      !device_address(src_v, &sv) || !device_address(block_pairs, &pp))
    return PKV_EINVAL;
  const hipError_t e = pkv::launch_copy_blocks(dk, dv, sk, sv, static_cast<const int32_t*>(pp), num_pairs, block_bytes,
                                               src_num_blocks, dst_num_blocks, stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // extern "C"
