// Byte layouts of the attention workspaces (host code: the C ABI sizes
// workspaces with them, the launcher places the kernels' partial states).

#include "pkv_internal.h"

namespace pkv {

WorkspaceLayout decode_workspace_layout(int num_seqs, int h_q, int h_kv, int head_dim, int num_splits,
                                        int balanced_workgroups, int counter_slots) {
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t units = (size_t)num_seqs * h_kv;
  const size_t rows = balanced_workgroups > 0
                          ? (size_t)balanced_workgroups * 2 * (h_q / h_kv)  // two slots per workgroup, G rows each
                          : (size_t)num_seqs * h_q * num_splits;           // units * G * splits
  WorkspaceLayout L;
  L.counters = 0;
  L.ml = align((counter_slots > 0 ? (size_t)counter_slots : units) * sizeof(int32_t));
  L.acc = L.ml + align(rows * 2 * sizeof(float));
  L.total = L.acc + align(rows * head_dim * sizeof(float));
  return L;
}

WorkspaceLayout multi_workspace_layout(int num_seqs, int h_kv, int head_dim, int row_tiles, int num_splits,
                                       int balanced_workgroups) {
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  // one counter and 16 partial rows per split for every row tile the
  // workgroups hold (row groups x tiles per workgroup: one more than
  // row_tiles when an odd count is held two by two)
  const int per_wg = multi_tiles_per_workgroup(row_tiles);
  const size_t units = (((size_t)num_seqs * h_kv + 7) / 8) * 8 * multi_row_groups(row_tiles) * per_wg;
  const size_t rows = balanced_workgroups > 0 ? (size_t)balanced_workgroups * 2 * per_wg * 16  // two slots per range
                                              : units * num_splits * 16;
  WorkspaceLayout L;
  L.counters = 0;
  L.ml = align(units * sizeof(int32_t));
  L.acc = L.ml + align(rows * 2 * sizeof(float));
  L.total = L.acc + align(rows * head_dim * sizeof(float));
  return L;
}

}  // namespace pkv
