// reshape_and_cache: write each new token's K and V into its slot of the
// paged pool, for gfx950.
//
// A growing sequence takes free blocks one by one and its earlier blocks
// never move ("Paged KV Cache" tutorial, section "Answer Key", question 2),
// so the new
// token of a decode step writes exactly one slot: slot = block * B + offset,
// landing at cache[slot / B, head, slot % B, :].
//
// One thread moves 8 consecutive elements of one (token, head): 16-byte
// loads/stores for 16-bit data.  Into an FP8 pool each element is divided by
// the tensor scale (one correctly rounded binary32 division) and rounded to
// the nearest E4M3 code with saturation.

#include "device_common.h"
#include "kv_chunk.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kEsize[4] = {4, 2, 2, 1};

// The values' registers are needed here: keeps the compiler from sinking
// their loads below the slot test (they would then wait for the slot).
template <int DT>
__device__ __forceinline__ void issued(const Chunk8<DT>& c) {
  if constexpr (DT == kF32) {
    asm volatile("" ::"v"(c.w[0]), "v"(c.w[1]));
  } else {
    asm volatile("" ::"v"(c.w));
  }
}

template <int IN, int KV>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(const uint8_t* key, const uint8_t* value,
                                                                uint8_t* k_cache, uint8_t* v_cache,
                                                                const int64_t* slots, int num_tokens, int h_kv,
                                                                int head_dim, int block_size, int64_t num_slots,
                                                                float k_scale, float v_scale) {
  const int chunks = head_dim / 8;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;  // the host keeps the thread count below 2^31
  if (gid >= num_tokens * h_kv * chunks) return;
  const int c = gid % chunks;
  const int th = gid / chunks;
  const int h = th % h_kv;
  const int t = th / h_kv;
  // the token's K/V do not depend on its slot: their loads go out together
  // with the slot's, so the chain is two round trips (loads, then stores)
  const int64_t src = ((int64_t)th * head_dim + (int64_t)c * 8) * kEsize[IN];
  const Chunk8<IN> kin = load8<IN>(key + src);
  const Chunk8<IN> vin = load8<IN>(value + src);
  const int64_t slot = slots[t];
  issued<IN>(kin);
  issued<IN>(vin);
  if (slot < 0 || slot >= num_slots) return;  // padding or outside the pool
  int64_t blk, off;
  if (num_slots <= 0x7fffffff) {  // the common pool: 32-bit division
    const int s32 = (int)slot;
    blk = s32 / block_size;
    off = s32 - (int)blk * block_size;
  } else {
    blk = slot / block_size;
    off = slot - blk * block_size;
  }
  const int64_t dst = (((blk * h_kv + h) * block_size + off) * head_dim + (int64_t)c * 8) * kEsize[KV];
  if constexpr (IN == KV) {
    store8<KV>(k_cache + dst, kin);
    store8<KV>(v_cache + dst, vin);
  } else {
    store8<kFP8>(k_cache + dst, quantize8<IN>(kin, k_scale));
    store8<kFP8>(v_cache + dst, quantize8<IN>(vin, v_scale));
  }
}

template <int IN, int KV>
hipError_t launch(const void* key, const void* value, void* kc, void* vc, const int64_t* slots, int T, int h_kv,
                  int d, int bs, int nb, float ks, float vs, hipStream_t stream) {
  const int64_t threads = (int64_t)T * h_kv * (d / 8);
  if (threads == 0) return hipSuccess;
  if (threads > 0x7fffff00) return hipErrorInvalidValue;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((reshape_and_cache_kernel<IN, KV>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(key), static_cast<const uint8_t*>(value), static_cast<uint8_t*>(kc),
                     static_cast<uint8_t*>(vc), slots, T, h_kv, d, bs, (int64_t)nb * bs, ks, vs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, int in_dtype, void* k_cache, void* v_cache,
                                    int kv_dtype, float k_scale, float v_scale, const int64_t* slot_mapping,
                                    int num_tokens, int h_kv, int head_dim, int block_size, int num_blocks,
                                    hipStream_t stream) {
#define PKV_RC(IN, KV)                                                                                          \
  if (in_dtype == IN && kv_dtype == KV)                                                                         \
    return launch<IN, KV>(key, value, k_cache, v_cache, slot_mapping, num_tokens, h_kv, head_dim, block_size, \
                          num_blocks, k_scale, v_scale, stream);
  PKV_RC(kF32, kF32)
  PKV_RC(kF16, kF16)
  PKV_RC(kBF16, kBF16)
  PKV_RC(kFP8, kFP8)
  PKV_RC(kF32, kFP8)
  PKV_RC(kF16, kFP8)
  PKV_RC(kBF16, kFP8)
#undef PKV_RC
  return hipErrorInvalidValue;
}

}  // namespace pkv
