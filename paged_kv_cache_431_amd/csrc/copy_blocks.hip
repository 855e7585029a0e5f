// copy_blocks: the block copy of copy-on-write, for gfx950.
//
// Sequences share prefix blocks by reference; a sequence that appends into a
// shared, partly filled block moves onto a fresh block first ("Paged KV
// Cache" tutorial, section "Block Tables and Sharing"; "KV cache and
// PagedAttention in serving", section "The bonus: sharing via
// copy-on-write").  This kernel copies each reported (src, dst) block, all
// KV heads and slots, in the K pool and in the V pool.
//
// The same kernel moves blocks between two different pools for swapping
// (a preempted sequence's blocks go to host memory over PCIe and come back
// later: "KV cache and PagedAttention in serving", section "Beyond paging:
// radix trees and continuous batching"; "Paged KV Cache" tutorial, section
// "Offload").  One launch moves any number of scattered blocks; host pools
// are pinned host memory the GPU addresses directly, so the loads or the
// stores of a swap cross PCIe.
//
// A physical block is one contiguous run of h_kv * block_size * head_dim
// elements in each pool.  Workgroup (pair, pool, part) copies a 16 KiB part of
// one block: each thread moves four 16-byte pieces, all loads issued before
// the stores.  Block ids outside their pool are skipped.

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyPieces = 4;                                   // 16-byte pieces per thread
constexpr int64_t kCopyPart = (int64_t)kCopyThreads * kCopyPieces * 16;  // bytes per workgroup

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(uint8_t* dst_k, uint8_t* dst_v,
                                                                   const uint8_t* src_k, const uint8_t* src_v,
                                                                   const int32_t* pairs, int64_t block_bytes,
                                                                   int parts, int src_blocks, int dst_blocks) {
  const int part = blockIdx.x % parts;
  const int pool = (blockIdx.x / parts) & 1;
  const int pair = blockIdx.x / (2 * parts);
  const int src = pairs[2 * pair];
  const int dst = pairs[2 * pair + 1];
  if ((unsigned)src >= (unsigned)src_blocks || (unsigned)dst >= (unsigned)dst_blocks) return;
  const uint8_t* from = (pool ? src_v : src_k) + (int64_t)src * block_bytes;
  uint8_t* to = (pool ? dst_v : dst_k) + (int64_t)dst * block_bytes;
  u32x4 buf[kCopyPieces];
  int64_t off[kCopyPieces];
#pragma unroll
  for (int i = 0; i < kCopyPieces; ++i) {
    off[i] = (int64_t)part * kCopyPart + ((int64_t)i * kCopyThreads + threadIdx.x) * 16;
    if (off[i] < block_bytes) buf[i] = *reinterpret_cast<const u32x4*>(from + off[i]);
  }
#pragma unroll
  for (int i = 0; i < kCopyPieces; ++i)
    if (off[i] < block_bytes) *reinterpret_cast<u32x4*>(to + off[i]) = buf[i];
}

}  // namespace

hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int32_t* pairs,
                              int num_pairs, int64_t block_bytes, int src_blocks, int dst_blocks,
                              hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int parts = (int)((block_bytes + kCopyPart - 1) / kCopyPart);
  const int64_t grid = (int64_t)num_pairs * 2 * parts;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0, stream,
                     static_cast<uint8_t*>(dst_k), static_cast<uint8_t*>(dst_v), static_cast<const uint8_t*>(src_k),
                     static_cast<const uint8_t*>(src_v), pairs, block_bytes, parts, src_blocks, dst_blocks);
  return hipGetLastError();
}

}  // namespace pkv
