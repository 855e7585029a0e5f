// Paged attention for gfx950 (MI355X).
//
// The attention of a sequence's new query token(s) over that sequence's
// cached K/V, read block by block through the sequence's block table, never
// gathered into a contiguous copy ("KV cache and PagedAttention in serving",
// section "PagedAttention: virtual memory for GPUs"; "Paged KV Cache"
// tutorial, section "Block Tables and Sharing").  Query head g reads KV head
// g / G with G = h_q / h_kv, so one workgroup serves the whole query group of
// a KV head and reads each K/V byte once.
//
// Work decomposition
//   One workgroup (4 waves) per (sequence, KV head, split), and with several
//   query tokens per (sequence, KV head, row group, split).  The sequence's
//   16-token tiles are cut into `n` contiguous ranges (n <= num_splits, chosen
//   per sequence on the device from its own length); each wave takes a
//   contiguous quarter of its workgroup's range.  Each wave keeps an
//   online-softmax state (running max m, running sum l, unnormalised output
//   acc) per query row; the 4 waves merge through LDS; a sequence with several
//   ranges writes partial states to the workspace and the last workgroup to
//   finish (an atomic counter per (sequence, KV head, row tile)) merges them
//   and writes the output, so a call is a single kernel launch.
//   When the grid does not fit on the GPU at once, workgroups take the
//   sequences longest first (each workgroup ranks all context lengths in
//   LDS), so the workgroups that start last hold the shortest work.
//   Balanced ranges (few pairs with long contexts): every workgroup takes an
//   equal contiguous range of all pairs' tiles instead, laid out KV head by
//   KV head with one head block per XCD; a pair cut between ranges merges
//   through the workspace like splits.
//
// Memory pipeline (the kernel is bound by HBM bandwidth: each K/V byte is
// used by G query rows only)
//   A wave first loads the physical block ids of up to 64 of its tiles, one
//   per lane, then streams the tiles through a ring of NBUF register buffers:
//   while tile i is computed, the loads of the next NBUF-1 tiles are in
//   flight.  Loads are issued unconditionally, so the compiler can wait for
//   exactly the oldest tile instead of draining every outstanding load.  Each
//   tile's loads go through a buffer resource sized to the tile's rows
//   inside the context (the tail slots of a last block are not read), and a
//   ring step past the wave's last tile gets a resource of size 0, whose
//   loads return zeros without a memory access: it computes nothing.  When one
//   workgroup is the only reader of a (sequence, KV head)'s K/V (decode, and
//   several query tokens held by one row group) the loads are non-temporal:
//   nothing re-reads them.
//   LDS ring: over 16-bit caches with 256-byte rows and grids of more than
//   three workgroups per CU, the tiles come straight into a per-wave ring in
//   LDS (buffer loads to LDS, waits placed by the kernel) instead of through
//   registers.
//   Pacing: when a grid that fits on the GPU at once leaves some CUs with one
//   workgroup and others with two, the lone workgroups wait after each tile
//   (short sleeps on the real-time counter, for a share of the tile's step
//   time that grows with the number of shared CUs), so that the CUs holding
//   two get HBM sooner and all end together.
//
// Matrix-core path (16-bit or FP8 caches, block_size 16 x 2^k)
//   Scores: S^T[token][g] = K[token][:] . Q[g][:] with v_mfma_f32_16x16x32
//   (bf16 or f16): K is the A operand.  Each K load reads 1 KiB of the tile
//   contiguously (whole cache lines); the rows pass through a per-wave LDS
//   tile with rows padded by 16 bytes and come back in the operand layout
//   (lane = token, 16-byte chunks of the row).  Q (padded to 16 rows) is the
//   B operand and stays in registers for the whole walk.  The
//   accumulator layout puts scores for tokens 4*(lane/16)+r of query row
//   lane%16 in lane `lane`, which is exactly the B-operand layout the PV
//   product needs, so probabilities never move between lanes.
//   PV: O^T[d][g] += V^T[d][token] P^T[token][g].  The contraction index is
//   the token, so the A operand is V transposed: each wave stores its tile's
//   V rows, as loaded (4 token rows of a d-chunk per 16-byte load), into a
//   per-wave LDS tile in their natural [token][d] layout (16-byte chunks
//   XOR-swizzled by the row to spread banks), and one transposing LDS read
//   (ds_read_b64_tr_b16) per 16 rows of d returns the 4 tokens x 1 d cell
//   each lane needs.  The probabilities are split into a hi and a lo 16-bit
//   part (p = hi + lo + O(2^-16 p)) and applied by one v_mfma_f32_16x16x32
//   per 16 rows of d whose contraction takes each token twice, with its hi
//   and its lo part, so P keeps ~16 bits of precision at the MFMA count of a
//   single 16-bit P.
//   FP8 (OCP E4M3) K/V are converted in registers by the hardware converter
//   (exact into bf16/f16); k_scale folds into the logit scale and v_scale
//   into the final normalisation.
//   Tokens past the context (the tail of the last block) are masked by select
//   (V rows zeroed, scores set to -inf), never by multiplying, so whatever
//   those slots hold (NaN included) cannot leak into the result; tiles with
//   no such token branch around the selects.
//   The running max moves only when a score exceeds it by more than
//   kRescaleSlack (log2 units), so after the first tiles the accumulators are
//   rarely rescaled; probabilities relative to the stale max stay <= 2^8.
//
// Cross-split merge
//   Partial states are written and read with device-scope (agent) relaxed
//   atomic stores and loads, which the gfx950 memory system keeps coherent
//   across the XCDs' separate L2 caches without writing back or invalidating
//   whole caches; a vmcnt(0) wait orders them before the counter increment.
//
// Several new query tokens per sequence (MT)
//   The 16 MFMA columns hold (query token, query head) rows of a 16-row tile
//   instead of the group's heads; each lane masks scores past its row's
//   causal limit.  A workgroup holds up to two row tiles (RT), so one walk
//   of the K/V serves 32 rows; when a (sequence, KV head) has more row groups
//   than one, they run on one XCD so that their walks share that XCD's L2.
//
// Decode step (AP): the new tokens' scatter inside the launch
//   The one wave that reads a sequence's last position writes the new token
//   there, and computes that tile with the rows it wrote (staged in LDS)
//   instead of the loaded ones, so nothing waits for the write.
//
// Vector path (fp32 caches, any block size): the same decomposition, one
// token at a time, lanes owning head dimensions, fp32 FMAs and wave
// reductions.

#include "device_common.h"
#include "kv_chunk.h"
#include "pkv_internal.h"


namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;

struct Params {
  void* out;
  const void* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t* counters;
  float* ws_ml;   // [rows][2]: running max, running sum
  float* ws_acc;  // [rows][D]
  int h_q, h_kv, group, block_size, num_blocks, max_blocks_per_seq;
  int num_splits, tiles_per_split, units;
  int tile_shift;  // log2(block_size / 16) on the matrix-core path
  float scale_log2, v_scale;
  int out_dtype;
  // Several query tokens per sequence (null for decode): the query rows of
  // sequence s are [query_start[s], query_start[s + 1]) of q and out.
  const int32_t* query_start;
  int num_query_tokens, max_query_len;
  int lpt_shift;   // decode: >= 0 takes sequences longest first (tile counts >> lpt_shift), -1 in order
  int pace_lo, pace_hi;  // workgroups [pace_lo, pace_hi) pace their tiles (a CU each); empty: none
  int pace_share32;      // a paced wave waits this many 32nds of each tile's step time
  int balanced;    // decode: tiles of all (sequence, KV head) pairs cut into gridDim.x equal ranges
  int row_tiles;   // 16-row tiles of (query token, head) rows per (sequence, KV head)
  int row_groups;  // workgroups per (sequence, KV head, split): row_tiles / RT, rounded up
  // Decode step that appends each sequence's new token itself (null
  // otherwise): new_k, new_v [S, h_kv, D] in new_dtype go to position ctx - 1
  // (its slot from the block table), converted as the scatter converts.
  const uint8_t* new_k;
  const uint8_t* new_v;
  uint8_t* k_store;
  uint8_t* v_store;
  int new_dtype;
  float k_scale_enc, v_scale_enc;
};

struct Item {
  int s, kvh, unit, split, ctx, n_tiles, n_splits_seq, t_begin, t_end;
  // decode step: the sequence's context length, before clamping, lies in
  // [1, table capacity], so position ctx - 1 is the new token's own slot (a
  // longer one is attended over the table's tokens and writes nothing)
  bool append;
  int rt, m, q0;  // several query tokens: first row tile, query tokens of the sequence, first query row
  // balanced ranges (bal_r > 0): range length, first workgroup holding a
  // piece of this pair, first tile of the pair in the flattened order
  int bal_r, bal_w0, bal_p;
};

// Workgroup id -> work item.  Consecutive workgroup ids go to the 8 XCDs in
// turn, so every split of one (sequence, KV head) gets an id with the same
// residue mod 8: their partial results meet in one XCD's L2.  With several
// query tokens (MT) the row groups of one (sequence, KV head) share that
// residue too, so they read its K/V through the same L2.
//
// Query token i of the m new tokens of a sequence with ctx cached tokens
// (its own K/V included) sits at position ctx - m + i and attends to the
// positions up to and including its own.
// Workgroup id -> unit index (decode: the (sequence, KV head) index; with
// several query tokens the (sequence, KV head, row group) index).
__device__ __forceinline__ int decode_unit(const Params& p) {
  const int wg = blockIdx.x;
  return ((wg >> 3) / p.num_splits) * 8 + (wg & 7);
}

// Exclusive prefix sum of x over the workgroup's threads in thread order;
// part holds kDecodeWaves ints.  Every thread calls this; part may be reused
// after the next barrier.
__device__ int block_exclusive_scan(int x, int* part) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) part[w] = incl;
  __syncthreads();
  int base = 0;
  for (int j = 0; j < w; ++j) base += part[j];
  return base + incl - x;
}

// Longest pairs first.  Workgroups start in id order as resident ones
// finish, so when the grid does not fit at once, handing the pairs out in
// decreasing order of work lets the long ones start first and the short ones
// fill the end (the longest-processing-time-first rule of list scheduling):
// the launch no longer waits on a long pair that started late.  Rank r of
// the sequences ordered by tile count (>> p.lpt_shift), longest first, ties
// in index order; *ctx_out receives its context length as stored (items
// clamp it).  Every thread of the workgroup calls this (at most kLptMaxSeqs
// sequences); lds holds kLptBins + 8 ints.
__device__ int lpt_sequence(const Params& p, int r, int* lds, int* ctx_out) {
  constexpr int PER = kLptMaxSeqs / kDecodeThreads;  // consecutive sequences per thread
  constexpr int BPT = kLptBins / kDecodeThreads;     // bins per thread
  int* hist = lds;              // sequences per bin
  int* part = lds + kLptBins;   // [0, 4): scan partials; 4, 5: the rank's bin and its first rank; 6, 7: result
  const int S = p.units / p.h_kv;
  const int t = threadIdx.x;
  const int cap = p.max_blocks_per_seq * p.block_size;
  int bin[PER], ctx[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = t * PER + i;
    const int raw = s < S ? p.context_lens[s] : 0;
    const int c = raw < 0 ? 0 : (raw > cap ? cap : raw);
    ctx[i] = raw;
    bin[i] = s < S ? min(((c + kTileTokens - 1) / kTileTokens) >> p.lpt_shift, kLptBins - 1) : -1;
  }
  for (int b = t; b < kLptBins; b += kDecodeThreads) hist[b] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (bin[i] >= 0) atomicAdd(&hist[bin[i]], 1);
  __syncthreads();
  // thread t holds the bins [top - BPT, top), walked downwards: the
  // sequences in higher bins than these come first
  const int top = kLptBins - BPT * t;
  int local = 0;
#pragma unroll
  for (int j = 1; j <= BPT; ++j) local += hist[top - j];
  int run = block_exclusive_scan(local, part);
#pragma unroll
  for (int j = 1; j <= BPT; ++j) {
    const int h = hist[top - j];
    if (run <= r && r < run + h) {
      part[4] = top - j;
      part[5] = run;
    }
    run += h;
  }
  __syncthreads();
  const int bstar = part[4];
  const int k = r - part[5];  // rank r is the k-th sequence of bin bstar in index order
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) cnt += bin[i] == bstar;
  int before = block_exclusive_scan(cnt, part);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (bin[i] == bstar) {
      if (before == k) {
        part[6] = t * PER + i;
        part[7] = ctx[i];
      }
      ++before;
    }
  }
  __syncthreads();
  const int seq = part[6];
  *ctx_out = part[7];
  __syncthreads();  // the LDS is the walk's next
  return seq;
}

template <bool MT, int RT, bool LPT = false>
__device__ __forceinline__ bool get_item(const Params& p, Item& it, int* lds) {
  const int wg = blockIdx.x;
  const int j = wg >> 3;
  it.unit = decode_unit(p);
  it.split = j % p.num_splits;
  int base = it.unit;  // (sequence, KV head) index
  it.rt = 0;
  if constexpr (MT) {
    const int y = it.unit >> 3;
    it.rt = (y % p.row_groups) * RT;
    base = (y / p.row_groups) * 8 + (it.unit & 7);
  }
  if (base >= p.units) return false;
  int ctx;
  const int cap = p.max_blocks_per_seq * p.block_size;
  if constexpr (LPT) {
    // the unit's KV head (and row group) stay; its sequence is the one of
    // that rank.  All splits and row groups of a unit take the same one.
    const int kvh = base % p.h_kv;
    it.s = lpt_sequence(p, base / p.h_kv, lds, &ctx);
    base = it.s * p.h_kv + kvh;
    if constexpr (MT) it.unit = ((base >> 3) * p.row_groups + it.rt / RT) * 8 + (base & 7);
    else it.unit = base;
  } else {
    it.s = base / p.h_kv;
    ctx = p.context_lens[it.s];
  }
  it.append = ctx >= 1 && ctx <= cap;
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  it.kvh = base - it.s * p.h_kv;
  it.ctx = ctx;
  int n_tok = ctx;  // positions any row of the item attends to: [0, n_tok)
  if constexpr (MT) {
    // rows beyond the query table are clamped away, never read or written
    int q0 = p.query_start[it.s], q1 = p.query_start[it.s + 1];
    q0 = min(max(q0, 0), p.num_query_tokens);
    q1 = min(max(q1, q0), p.num_query_tokens);
    it.q0 = q0;
    it.m = min(q1 - q0, p.max_query_len);
    const int first_row = it.rt * 16;
    if (first_row >= it.m * p.group) return false;  // no query row in these tiles
    const int i_last = min(it.m - 1, (first_row + 16 * RT - 1) / p.group);
    n_tok = min(ctx, max(0, ctx - it.m + i_last + 1));
  }
  it.n_tiles = (n_tok + kTileTokens - 1) / kTileTokens;
  int ns = (it.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  it.n_splits_seq = ns > p.num_splits ? p.num_splits : ns;
  const int per = it.n_splits_seq > 0 ? (it.n_tiles + it.n_splits_seq - 1) / it.n_splits_seq : 0;
  it.t_begin = it.split * per;
  it.t_end = min(it.n_tiles, it.t_begin + per);
  it.bal_r = 0;
  return true;
}

template <int D>
struct MergeSmem {
  float acc[kDecodeWaves][kMaxGroup][D + 4];  // +4 floats: rows start on different banks
  float m[kDecodeWaves][kMaxGroup];
  float l[kDecodeWaves][kMaxGroup];
  int flag;
};

__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every store this wave issued has completed.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Store the DW = D/16 outputs (times `mul`) a thread holds of one output
// row: a[4 h + q] is element 64 h + 4 chunk + q, so that the 16 threads of a
// row store 64 contiguous elements per instruction (and read their states
// from LDS the same way, without bank conflicts).  NT: non-temporal stores,
// for the outputs of several query tokens (4 tokens: 6.2 MB per launch of
// the 70B shape; 1-3 % faster launches), not for decode's (slower there).
template <int D, bool NT = false>
__device__ __forceinline__ void store_out(const Params& p, size_t row, int chunk, const float* a, float mul) {
  constexpr int DW = D / 16;
  const size_t off = row * D + (size_t)chunk * 4;
  if (p.out_dtype == kF32) {
    float* o = static_cast<float*>(p.out) + off;
#pragma unroll
    for (int h = 0; h < DW / 4; ++h) {
      const float* x = a + 4 * h;
      if constexpr (NT) __builtin_nontemporal_store(f32x4{x[0] * mul, x[1] * mul, x[2] * mul, x[3] * mul}, reinterpret_cast<f32x4*>(o + 64 * h));
      else *reinterpret_cast<float4*>(o + 64 * h) = make_float4(x[0] * mul, x[1] * mul, x[2] * mul, x[3] * mul);
    }
  } else {
    uint16_t* o = static_cast<uint16_t*>(p.out) + off;
#pragma unroll
    for (int h = 0; h < DW / 4; ++h) {
      uint32_t packed[2];
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        // A 16-bit output is the fp32 output rounded to nearest-even: the
        // products stay rounded fp32 values (the compiler would otherwise fuse
        // the multiply into a mixed-precision instruction that rounds once).
        float y0 = a[4 * h + e] * mul, y1 = a[4 * h + e + 1] * mul;
        asm volatile("" : "+v"(y0), "+v"(y1));
        uint32_t lo, hi;
        if (p.out_dtype == kBF16) {
          lo = f32_to_bf16_rne(y0);
          hi = f32_to_bf16_rne(y1);
        } else {
          lo = f32_to_f16_bits(y0);
          hi = f32_to_f16_bits(y1);
        }
        packed[e / 2] = lo | (hi << 16);
      }
      if constexpr (NT) __builtin_nontemporal_store(u32x2{packed[0], packed[1]}, reinterpret_cast<u32x2*>(o + 64 * h));
      else *reinterpret_cast<u32x2*>(o + 64 * h) = u32x2{packed[0], packed[1]};
    }
  }
}

// Store DW = D/16 consecutive outputs (times `mul`) of one output row,
// elements chunk * DW + e (the balanced-range kernels' merge).  Rounding as
// in store_out.
template <int D>
__device__ __forceinline__ void store_out_contig(const Params& p, size_t row, int chunk, const float* a, float mul) {
  constexpr int DW = D / 16;
  const size_t off = row * D + (size_t)chunk * DW;
  if (p.out_dtype == kF32) {
    float* o = static_cast<float*>(p.out) + off;
#pragma unroll
    for (int e = 0; e < DW; e += 4) {
      float4 v = make_float4(a[e] * mul, a[e + 1] * mul, a[e + 2] * mul, a[e + 3] * mul);
      *reinterpret_cast<float4*>(o + e) = v;
    }
  } else {
    uint16_t* o = static_cast<uint16_t*>(p.out) + off;
    uint32_t packed[DW / 2];
#pragma unroll
    for (int e = 0; e < DW; e += 2) {
      float y0 = a[e] * mul, y1 = a[e + 1] * mul;
      asm volatile("" : "+v"(y0), "+v"(y1));
      uint32_t lo, hi;
      if (p.out_dtype == kBF16) {
        lo = f32_to_bf16_rne(y0);
        hi = f32_to_bf16_rne(y1);
      } else {
        lo = f32_to_f16_bits(y0);
        hi = f32_to_f16_bits(y1);
      }
      packed[e / 2] = lo | (hi << 16);
    }
    if constexpr (DW == 8) {
      *reinterpret_cast<u32x4*>(o) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    } else {
      *reinterpret_cast<u32x2*>(o) = u32x2{packed[0], packed[1]};
    }
  }
}

// Store DW outputs of one output row, elements c + 16 e (times `mul`): the
// layout the cross-range merge works in, where each store instruction of a
// row's 16 threads covers contiguous bytes.  Rounding as in store_out.
template <int D>
__device__ __forceinline__ void store_out_spread(const Params& p, size_t row, int c, const float* a, float mul) {
  constexpr int DW = D / 16;
  const size_t off = row * D + c;
  if (p.out_dtype == kF32) {
    float* o = static_cast<float*>(p.out) + off;
#pragma unroll
    for (int e = 0; e < DW; ++e) o[16 * e] = a[e] * mul;
  } else {
    uint16_t* o = static_cast<uint16_t*>(p.out) + off;
#pragma unroll
    for (int e = 0; e < DW; ++e) {
      float y = a[e] * mul;
      asm volatile("" : "+v"(y));
      o[16 * e] = (uint16_t)(p.out_dtype == kBF16 ? f32_to_bf16_rne(y) : f32_to_f16_bits(y));
    }
  }
}

// Output row of row r (0..15) of row tile k of an item, false if the row
// holds no query: decode rows are the group's query heads; with several query
// tokens row r of tile k is (query token, head) = divmod(16 (rt + k) + r, group).
template <bool MT>
__device__ __forceinline__ bool out_row(const Params& p, const Item& it, int k, int r, size_t& row) {
  const int G = p.group;
  if constexpr (MT) {
    const int gr = (it.rt + k) * 16 + r;
    const int i = gr / G;
    row = (size_t)(it.q0 + i) * p.h_q + it.kvh * G + (gr - i * G);
    return i < it.m;
  } else {
    row = (size_t)it.s * p.h_q + it.kvh * G + r;
    return r < G;
  }
}

// Rows of row tile k that attend over nothing (an empty context) get 0.
template <int D, bool MT>
__device__ void write_zeros(const Params& p, const Item& it, int k) {
  constexpr int DW = D / 16;
  const int g = threadIdx.x >> 4, chunk = threadIdx.x & 15;
  size_t row;
  if (!out_row<MT>(p, it, k, g, row)) return;
  float z[DW];
#pragma unroll
  for (int e = 0; e < DW; ++e) z[e] = 0.f;
  store_out<D>(p, row, chunk, z, 1.f);
}

// Merge the 4 waves' states of row tile k (already in `sm`, after a
// barrier), then either write the output (one range) or publish this range's
// partial state and let the last range of the (sequence, KV head, row tile)
// combine all of them.  Row tile k of a workgroup of RT row tiles has its
// own counter and partial rows: index unit * RT + k.
template <int D, bool MT, int RT, bool QUAD = true>
__device__ void finish(const Params& p, const Item& it, int k, MergeSmem<D>& sm) {
  constexpr int DW = D / 16;
  const int t = threadIdx.x;
  const int g = t >> 4, chunk = t & 15;
  const int R = MT ? 16 : p.group;  // rows of a row tile (partial-state rows per split)
  const int cidx = it.unit * RT + k;
  size_t row;
  const bool row_ok = out_row<MT>(p, it, k, g, row);
  // This thread's elements of the row: with one range 64 h + 4 chunk + q
  // (16-byte LDS reads and output stores, the 16 threads of a row on
  // consecutive bytes), for partial states chunk + 16 e, so that every store
  // and load instruction of the merge covers 64 contiguous bytes of a row
  // instead of scattering 4-byte accesses 32 bytes apart.  The kernels with
  // balanced ranges (QUAD false) keep chunk * DW + e for one range: at their
  // register limit the wider reads made the two-row-tile kernel spill 16
  // bytes more per lane (bf16 4-token batch of 32 long contexts 435 -> 440 us).
  const bool whole = it.n_splits_seq == 1;
  float a[DW];
  float mstar = kNegInf, lstar = 0.f;
#pragma unroll
  for (int e = 0; e < DW; ++e) a[e] = 0.f;
  if (row_ok) {
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) mstar = fmaxf(mstar, sm.m[w][g]);
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = mstar == kNegInf ? 0.f : fast_exp2(sm.m[w][g] - mstar);
      lstar += f * sm.l[w][g];
      if (QUAD && whole) {
#pragma unroll
        for (int h = 0; h < DW / 4; ++h) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&sm.acc[w][g][64 * h + 4 * chunk]);
#pragma unroll
          for (int q = 0; q < 4; ++q) a[4 * h + q] += f * v[q];
        }
      } else {
        const int e0 = whole ? chunk * DW : chunk;
        const int es = whole ? 1 : 16;
#pragma unroll
        for (int e = 0; e < DW; ++e) a[e] += f * sm.acc[w][g][e0 + es * e];
      }
    }
  }
  // a row that sees no position (only with several query tokens, when a
  // sequence has more new tokens than cached ones) gets 0
  if (whole) {
    if (row_ok) {
      if constexpr (QUAD) store_out<D, MT>(p, row, chunk, a, lstar > 0.f ? p.v_scale / lstar : 0.f);
      else store_out_contig<D>(p, row, chunk, a, lstar > 0.f ? p.v_scale / lstar : 0.f);
    }
    return;
  }
  const size_t base = (size_t)cidx * p.num_splits * R + g;  // partial row of split 0
  // partial row of piece sp: split sp of the pair, or with balanced ranges
  // slot 0 (first item) or 1 (last item) of range bal_w0 + sp, row tile k:
  // the pair is the first item of every range after bal_w0, and of bal_w0
  // only if it starts where that range starts
  auto prow_of = [&](int sp) -> size_t {
    if (it.bal_r > 0) {
      const int w = it.bal_w0 + sp;
      const int slot = (sp > 0 || it.bal_p == w * it.bal_r) ? 0 : 1;
      return (((size_t)w * 2 + slot) * RT + k) * R + g;
    }
    return base + (size_t)sp * R;
  };
  if (row_ok) {
    const size_t prow = prow_of(it.split);
    float* dst = p.ws_acc + prow * D + chunk;
#pragma unroll
    for (int e = 0; e < DW; ++e) store_agent(dst + 16 * e, a[e]);
    if (chunk == 0) {
      store_agent(p.ws_ml + 2 * prow, mstar);
      store_agent(p.ws_ml + 2 * prow + 1, lstar);
    }
  }
  wait_vm();  // this range's partial state is complete device-wide before it is counted
  __syncthreads();
  if (t == 0) {
    const int prev = __hip_atomic_fetch_add(p.counters + cidx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == it.n_splits_seq - 1;
    if (last) __hip_atomic_store(p.counters + cidx, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.flag = last;
  }
  __syncthreads();
  if (!sm.flag) return;
  if (!row_ok) return;
  float mm = kNegInf;
  for (int sp = 0; sp < it.n_splits_seq; ++sp) mm = fmaxf(mm, load_agent(p.ws_ml + 2 * prow_of(sp)));
  float ll = 0.f;
  float o[DW];
#pragma unroll
  for (int e = 0; e < DW; ++e) o[e] = 0.f;
  for (int sp = 0; sp < it.n_splits_seq; ++sp) {
    const size_t prow = prow_of(sp);
    const float m_i = load_agent(p.ws_ml + 2 * prow);
    const float l_i = load_agent(p.ws_ml + 2 * prow + 1);
    const float f = mm == kNegInf ? 0.f : fast_exp2(m_i - mm);
    ll += f * l_i;
    const float* src = p.ws_acc + prow * D + chunk;
#pragma unroll
    for (int e = 0; e < DW; ++e) o[e] += f * load_agent(src + 16 * e);
  }
  store_out_spread<D>(p, row, chunk, o, ll > 0.f ? p.v_scale / ll : 0.f);
}

// Balanced ranges (decode with long contexts over few (sequence, KV head)
// pairs, where one workgroup per pair and split leaves the work uneven): the
// tiles of all pairs are cut into equal contiguous ranges, one per
// workgroup, so every workgroup reads the same number of bytes whatever the
// mix of context lengths.  A range may hold the end of one pair, whole pairs
// and the start of another: each is an item of its own, run one after the
// other; the pieces of a pair split over several workgroups meet through the
// workspace as splits do.
//
// The pairs are laid out KV head by KV head (all sequences of head 0, then
// of head 1, ...), and with a grid of 8k workgroups, range j of head block x
// goes to a workgroup id with residue x mod 8: one XCD walks all pairs of
// "its" heads.  Sequences that share prefix blocks (copy-on-write sharing)
// then read them through one L2.  A range runs its items from the last to
// the first, so the piece that starts a pair (its prefix) comes first:
// every range walks its prefix at the start of the launch, and the sharers
// of a prefix walk it at about the same time.
// The query rows of sequence s for balanced ranges: one query token (decode),
// or with several query tokens its rows [q0, q0 + m) of q and out, clamped
// as get_item clamps them; every row of a pair is in one workgroup (its
// tiles are the context's: the last row sees them all).
__device__ __forceinline__ void query_rows(const Params& p, int s, Item& it) {
  it.rt = 0;
  it.m = 1;
  it.q0 = 0;
  if (p.query_start != nullptr) {
    int q0 = p.query_start[s], q1 = p.query_start[s + 1];
    q0 = min(max(q0, 0), p.num_query_tokens);
    q1 = min(max(q1, q0), p.num_query_tokens);
    it.q0 = q0;
    it.m = min(q1 - q0, p.max_query_len);
  }
}

struct Balanced {
  int S, H, cap;  // sequences, KV heads, context lengths taken at most this
  int T_head;     // tiles of one KV head's pairs (every head has the same)
  int r;          // tiles per range (0: this workgroup has none)
  int w;          // this workgroup's range
  int pos, end;   // its range [pos, end) still to run, items taken from the end
};

// pre (LDS, S + 1 entries) receives the prefix sums of the sequences' tile
// counts; every thread of the workgroup calls this.
__device__ void balanced_setup(const Params& p, int* pre, Balanced& b) {
  b.S = p.units / p.h_kv;
  b.H = p.h_kv;
  // contexts are clamped to the table's capacity, as items clamp them; the
  // host keeps all pairs' tiles at that capacity within an int
  b.cap = p.max_blocks_per_seq * p.block_size;
  const int S = b.S, cap = b.cap;
  auto seq_tiles = [&](int s) {
    int c = p.context_lens[s];
    c = c < 0 ? 0 : (c > cap ? cap : c);
    return (c + kTileTokens - 1) / kTileTokens;
  };
  if (threadIdx.x < 64) {  // wave 0: pre[s] = tiles of sequences 0 .. s-1
    const int lane = threadIdx.x;
    const int per = (S + 63) / 64;  // consecutive sequences per lane
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      const int s = lane * per + i;
      if (s < S) sum += seq_tiles(s);
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int run = incl - sum;
    for (int i = 0; i < per; ++i) {
      const int s = lane * per + i;
      if (s < S) {
        run += seq_tiles(s);
        pre[s + 1] = run;
      }
    }
    if (lane == 0) pre[0] = 0;
  }
  __syncthreads();
  b.T_head = pre[S];
  const int T = b.H * b.T_head;  // every pair's tiles
  // ranges of at least kBalancedMinRange tiles: with short contexts the
  // later ranges get nothing
  const int W = (int)gridDim.x;
  const int w_eff = T > 0 ? min(W, (T + kBalancedMinRange - 1) / kBalancedMinRange) : 0;
  b.r = w_eff > 0 ? (T + w_eff - 1) / w_eff : 0;
  // range of this workgroup: consecutive ranges (one head's pairs) on one XCD
  b.w = (W & 7) == 0 ? (int)(blockIdx.x & 7) * (W >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  b.pos = b.w < w_eff ? b.w * b.r : 0;
  b.end = b.w < w_eff ? min(T, b.pos + b.r) : 0;
}

// The next item of this workgroup's range, taken from the range's end:
// false when the range is done.
__device__ bool balanced_next(const Params& p, const int* pre, Balanced& b, Item& it) {
  if (b.end <= b.pos) return false;
  const int last = b.end - 1;          // the item holds this flattened tile
  const int h = last / b.T_head;       // its KV head
  const int q = last - h * b.T_head;   // its tile among that head's pairs
  // the sequence whose pair holds tile q: the last s with pre[s] <= q
  // (sequences without tiles hold none)
  int lo = 0, hi = b.S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= q) lo = mid;
    else hi = mid - 1;
  }
  const int ts = pre[lo + 1] - pre[lo];  // > 0: q lies in it
  const int first = h * b.T_head + pre[lo];  // the pair's first flattened tile
  const int begin = max(first, b.pos);
  it.s = lo;
  it.kvh = h;
  it.unit = lo * b.H + h;
  const int ctx = p.context_lens[lo];
  it.append = ctx >= 1 && ctx <= b.cap;
  it.ctx = ctx < 0 ? 0 : (ctx > b.cap ? b.cap : ctx);
  it.n_tiles = ts;
  it.t_begin = begin - first;
  it.t_end = b.end - first;
  it.bal_r = b.r;
  it.bal_w0 = first / b.r;
  it.bal_p = first;
  it.n_splits_seq = (first + ts - 1) / b.r - it.bal_w0 + 1;
  it.split = b.w - it.bal_w0;
  query_rows(p, lo, it);
  b.end = begin;
  return true;
}

// Pairs of sequences without tiles (context 0) get zeros.
template <int D, bool MT, int RT>
__device__ void balanced_zeros(const Params& p, const int* pre, const Balanced& b) {
  for (int u = blockIdx.x; u < p.units; u += gridDim.x) {
    const int s = u / b.H;
    if (pre[s + 1] == pre[s]) {
      Item z;
      z.s = s;
      z.kvh = u - s * b.H;
      query_rows(p, s, z);
#pragma unroll
      for (int k = 0; k < RT; ++k) write_zeros<D, MT>(p, z, k);
    }
  }
}

// ---------------------------------------------------------------- matrix-core path

template <int CT>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (CT == kBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
}

// Issue spacing after a group of MFMAs.  With the toolchain in use, vector
// instructions that overwrote a source register of a v_mfma_f32_16x16x32 (its
// A operand or its accumulator input; 8 passes on gfx950) a few instructions
// after issue gave wrong results.  Each group is therefore issued with no
// other instruction in between (the scheduler is kept out) and followed by 16
// wait states, which cover every read of the operands of its last MFMA.
__device__ __forceinline__ void mfma_guard() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Two E4M3 bytes of w (bytes 0-1, or 2-3 when HI) -> the packed CT pair
// holding them, lower byte in the low half.  Every E4M3 value is exact in
// bf16 and in f16, and one gfx950 conversion (scale 1) produces the pair.
// Only the whole 32-bit result is used: with the toolchain in use, reading
// element 1 of the builtin's two-element result compiled to a copy of
// element 0, while the register itself holds both conversions (checked for
// all 256 codes on the GPU).
template <int CT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_pair(uint32_t w) {
  if constexpr (CT == kBF16) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
}

// K/V loads go through a buffer resource per tile: its base is the tile's
// address (wave-uniform), its size the bytes of the tile's rows inside the
// context, or 0 for a ring step past the wave's last tile or a block id
// outside the pool, whose loads then return zeros without touching memory
// (the hardware's range check), so the ring issues every load
// unconditionally and reads no byte twice.  When one
// workgroup is the only reader of a (sequence, KV head)'s K/V, as in decode,
// the loads are non-temporal (the caches do not keep the lines for a reuse
// that never comes); when several workgroups (row groups of several query
// tokens) walk the same K/V, they share it through one L2 and the loads keep
// the normal policy.  In a buffer load the per-lane part of the offset is a
// vector register, the part common to the wave a scalar one.
constexpr int kBufferWord3 = 0x00020000;  // raw (untyped) 32-bit data format

template <bool STREAM>
__device__ __forceinline__ u32x4 kv_load16(__amdgpu_buffer_rsrc_t r, int lane_off, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, off, STREAM ? 2 : 0));
}
template <bool STREAM>
__device__ __forceinline__ u32x2 kv_load8(__amdgpu_buffer_rsrc_t r, int lane_off, int off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, lane_off, off, STREAM ? 2 : 0));
}
template <bool STREAM>
__device__ __forceinline__ uint32_t kv_load4(__amdgpu_buffer_rsrc_t r, int lane_off, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, lane_off, off, STREAM ? 2 : 0);
}

// Pacing of a workgroup alone on its CU: after each tile it waits
// Params::pace_share32 / 32 of the tile's step time, when the workgroup holds
// at least kPaceMinTiles tiles (8 per wave).  The share grows with the number
// of CUs holding two workgroups (S = grid - kComputeUnits): the lone
// workgroups should end with the shared CUs, and the more CUs share, the
// slower each of them reads.  Measured best shares (in eighths, 16-bit
// caches, 8 KiB tiles) were 8, 9-10, 10-11 and 12 for S = 16-24, 64, 96 and
// 120-128 with one row tile, and 1.5-2 eighths less with two row tiles (their
// tiles take longer); past the best share the lone workgroups end last, and
// the time grows fast, so the line below stays at or under it.
constexpr int kPaceMinTiles = 8 * kDecodeWaves;
// A step counts for at most this many ticks of the 100 MHz counter (10 us,
// about 7 times a step of the 70B-style layer), so that a wave held up for
// long (preempted, say) does not sleep in proportion.
constexpr uint64_t kPaceMaxStepTicks = 1000;
__host__ __device__ constexpr int pace_share32(int shared_cus, int row_tiles) {
  return (row_tiles == 2 ? 26 : 32) + (shared_cus > 16 ? (shared_cus - 16) / 7 : 0);
}

// One 16-byte-per-lane buffer load straight into LDS: lane l's 16 bytes land
// at LDS byte address lds + 16 l; bytes past the resource's size arrive as
// zeros.  Written as assembly, so that the compiler, which does not model
// which LDS bytes such a load writes, adds no wait of its own: the kernel
// waits for these loads itself (s_waitcnt vmcnt) before reading their LDS.
// The instruction has no register results.
template <bool NT>
__device__ __forceinline__ void lds_load16(i32x4 rsrc, uint32_t lds, int lane_off, int off) {
  if constexpr (NT) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "s"(lds), "v"(lane_off), "s"(rsrc), "s"(off) : "memory", "m0");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(lane_off), "s"(rsrc), "s"(off) : "memory", "m0");
  }
}

// A raw buffer resource over [base, base + bytes) as four words (for assembly).
__device__ __forceinline__ i32x4 raw_rsrc(const uint8_t* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), bytes, kBufferWord3};
}

template <int KV, int D>
struct MfmaTile {
  static constexpr int ES = KV == kFP8 ? 1 : 2;  // bytes per cached element
  static constexpr int ROW = D * ES;              // bytes of one token's row (one head)
  static constexpr int KCH = ROW / 64;            // 16-byte K chunks per lane
  // K is loaded 1 KiB at a time (lane l: bytes 16 l .. 16 l + 15 of the
  // tile's 1 KiB piece c, so every load covers whole cache lines); the rows go
  // to a per-wave LDS tile and come back in the MFMA operand layout.  LDS rows
  // are padded by 16 bytes (KLDS = ROW + 16): the 16 rows an operand read
  // touches then fall on different banks for ROW = 64, 128 and 256.
  static constexpr int LPR = ROW / 16;  // 16-byte chunks (lanes) per row
  static constexpr int RPK = 64 / LPR;  // rows per 1 KiB load
  static constexpr int KLDS = ROW + 16; // LDS bytes per K row
  static constexpr int VB = D * ES / 16;          // V bytes per lane per token row
  static constexpr int VDW = VB / 4;              // ... in dwords (1, 2 or 4)
  // Bytes of K and V one 16-token tile brings in.
  static constexpr int TILE_BYTES = 2 * kTileTokens * ROW;
  // Register buffers in the load ring (tile i + NBUF - 1 is loaded while
  // tile i is computed): two for 8 KiB tiles, three for smaller ones, which
  // keeps the kernel within the register budget of 3 waves per SIMD.
  static constexpr int NBUF = TILE_BYTES >= 8192 ? 2 : 3;
  u32x4 k[KCH];
  uint32_t v[4][VDW];
  int lim;   // valid tokens in the tile (0..16)
  int tok0;  // position of its first token
};

// RT: 16-row tiles of query rows per workgroup (several query tokens only):
// with two, one walk of the K/V serves 32 rows, at 2 waves per SIMD for the
// registers of both tiles' states.  STREAM: K/V loads are non-temporal (the
// only walk of each (sequence, KV head)); false when several workgroups walk
// the same K/V and share it through L2.  BAL: balanced ranges (decode only;
// at most two workgroups per CU, so 2 waves per SIMD and their registers).
// DMA: K/V tiles (16-bit, 256-byte rows, one row tile) come straight into an
// LDS ring instead of through registers; its 64 KiB per workgroup leave room
// for two workgroups per CU.
template <int KV, int CT, int D, bool MT, bool AP, int RT, bool STREAM, bool BAL, bool LPT, bool DMA, bool PACE = false>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(
    RT == 1 && !BAL && !DMA ? kDecodeWavesPerSimd : 2))) void
decode_mfma_kernel(Params p) {
  static_assert(!DMA || (KV != kFP8 && D == 128 && RT == 1), "the LDS ring serves 16-bit rows of 256 bytes");
  using Tile = MfmaTile<KV, D>;
  constexpr int ROW = Tile::ROW;
  constexpr int KCH = Tile::KCH;
  constexpr int VDW = Tile::VDW;
  constexpr int NBUF = Tile::NBUF;
  constexpr int NK = D / 32;  // MFMA k-steps for the scores
  constexpr int NT = D / 16;  // 16-row output tiles of the PV product
  constexpr int VCH = D / 8;  // 16-byte chunks in a 16-bit V row

  __shared__ union {
    struct {
      // per-wave V tile of 16 tokens in its natural [token][d] layout, 16-bit
      // elements, 16-byte chunks of each row XOR-swizzled by the row
      u32x4 vtile[kDecodeWaves][DMA ? 1 : kTileTokens * VCH];
      // decode step: the new token's K and V rows as stored in the pools, one
      // copy per wave (each wave stages its own: no barrier)
      uint8_t newrow[kDecodeWaves][2][ROW];
      // per-wave K tile: row t, 16-byte chunk c at byte t * KLDS + 16 c
      u32x4 ktile[kDecodeWaves][DMA ? 1 : kTileTokens * Tile::KLDS / 16];
      // LDS ring of the direct loads: per wave and ring stage, the K tile
      // (row t, chunk c at chunk c ^ (t & 7) of row t) and the V tile (the
      // layout of vtile)
      u32x4 dk[kDecodeWaves][DMA ? NBUF : 1][DMA ? kTileTokens * VCH : 1];
      u32x4 dv[kDecodeWaves][DMA ? NBUF : 1][DMA ? kTileTokens * VCH : 1];
      // decode step with direct loads: the new token's K and V rows as given
      // (16 bytes per lane land in lane order)
      u32x4 nraw[kDecodeWaves][2][DMA && AP ? 64 : 1];
    } t;
    MergeSmem<D> merge;
    int lpt[kLptBins + 8];  // longest pairs first: bins and scan partials (before the walk)
  } sm;

  // balanced ranges: prefix sums of the sequences' tile counts
  __shared__ int sm_pre[BAL ? kBalancedMaxSeqs + 1 : 1];

  constexpr int CH = D / 8;  // 8-element chunks of a row
  // decode step: the new token's rows as loaded, 8 bytes at a time, from
  // new_k (kx) and new_v (vx); a lane's chunk is the OR of the two
  u32x2 kx[4] = {}, vx[4] = {};

  // One work item: a (sequence, KV head[, row group]) and a range of its
  // tiles; every early return below leaves the item, not the kernel.
  auto run_item = [&](Item& it) {
    if (it.n_tiles == 0) {
      if (it.split == 0) {
#pragma unroll
        for (int k = 0; k < RT; ++k) write_zeros<D, MT>(p, it, k);
      }
      return;
    }
    if (it.split >= it.n_splits_seq) return;

    const int lane = threadIdx.x & 63;
    // wave-uniform (the compiler cannot tell on its own), so every per-wave
    // quantity below lives in scalar registers and the tile loop is uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lo16 = lane & 15;
    const int q4 = lane >> 4;
    const int G = p.group;

    // Q as the B operand: column lo16 of row tile k is row lo16 of that tile (a
    // query head; with several query tokens a (query token, head) pair), same
    // d order as the K chunks.  Padding rows hold zeros and never form an
    // address outside the item's rows.  row_lim: positions [0, row_lim) the
    // row attends to.
    u32x4 qop[RT][NK];
    int row_lim[RT];
    // several query tokens: every row attends to at least the positions
    // [0, first_row_lim) (those of the first new token, ctx - m + 1)
    const int first_row_lim = MT ? it.ctx - it.m + 1 : it.ctx;
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      bool row_ok;
      size_t qr;
      row_lim[k] = it.ctx;
      if constexpr (MT) {
        const int gr = (it.rt + k) * 16 + lo16;
        const int i = gr / G;
        row_ok = i < it.m;
        const int ic = row_ok ? i : it.m - 1;  // it.m >= 1 for an item with rows
        qr = (size_t)(it.q0 + ic) * p.h_q + it.kvh * G + (row_ok ? gr - i * G : 0);
        row_lim[k] = min(it.ctx, max(0, it.ctx - it.m + ic + 1));
      } else {
        row_ok = lo16 < G;
        qr = (size_t)it.s * p.h_q + it.kvh * G + (row_ok ? lo16 : G - 1);
      }
      const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + qr * D;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int d0 = KV == kFP8 ? 64 * (kk >> 1) + 16 * q4 + 8 * (kk & 1) : 32 * kk + 8 * q4;
        qop[k][kk] = row_ok ? *reinterpret_cast<const u32x4*>(qrow + d0) : u32x4{0u, 0u, 0u, 0u};
      }
    }

    // the new token's rows converted to the pool's element type, into the
    // owner wave's LDS copy (K row, then V row)
    auto stage_new_token = [&]() {
      c8_u32x4 nraw0, nraw1;
      if constexpr (DMA) {
        // called at an owner's tile after its wait, when only the next
        // tile's loads are in flight: the rows' direct loads, issued before
        // those, have landed
        const int es = p.new_dtype == kF32 ? 4 : (p.new_dtype == kFP8 ? 1 : 2);
        const bool is_v = lane >= CH;
        const uint8_t* src = reinterpret_cast<const uint8_t*>(sm.t.nraw[wave][is_v ? 1 : 0]) +
                             (is_v ? lane - CH : lane) * 8 * es;
        const bool mine = lane < 2 * CH;
        nraw0 = mine ? *reinterpret_cast<const c8_u32x4*>(src) : c8_u32x4{0u, 0u, 0u, 0u};
        nraw1 = mine && es == 4 ? *reinterpret_cast<const c8_u32x4*>(src + 16) : c8_u32x4{0u, 0u, 0u, 0u};
      } else {
        nraw0 = c8_u32x4{kx[0][0] | vx[0][0], kx[0][1] | vx[0][1], kx[1][0] | vx[1][0], kx[1][1] | vx[1][1]};
        nraw1 = c8_u32x4{kx[2][0] | vx[2][0], kx[2][1] | vx[2][1], kx[3][0] | vx[3][0], kx[3][1] | vx[3][1]};
      }
      if (lane < 2 * CH) {
        const bool is_v = lane >= CH;
        uint8_t* stage = &sm.t.newrow[wave][is_v ? 1 : 0][(is_v ? lane - CH : lane) * 8 * Tile::ES];
        if constexpr (KV == kFP8) {
          const float enc = is_v ? p.v_scale_enc : p.k_scale_enc;
          Chunk8<kFP8> x;
          if (p.new_dtype == kF32) {
            Chunk8<kF32> c;
            c.w[0] = nraw0;
            c.w[1] = nraw1;
            x = quantize8<kF32>(c, enc);
          } else if (p.new_dtype == kF16) {
            Chunk8<kF16> c;
            c.w = nraw0;
            x = quantize8<kF16>(c, enc);
          } else if (p.new_dtype == kBF16) {
            Chunk8<kBF16> c;
            c.w = nraw0;
            x = quantize8<kBF16>(c, enc);
          } else {
            x.w = c8_u32x2{nraw0[0], nraw0[1]};
          }
          store8<kFP8>(stage, x);
        } else {
          Chunk8<KV> x;
          x.w = nraw0;
          store8<KV>(stage, x);
        }
      }
    };

    f32x4 acc[RT][NT];
    float m_run[RT], l_run[RT];
#pragma unroll
    for (int k = 0; k < RT; ++k) {
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[k][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run[k] = kNegInf;
      l_run[k] = 0.f;
    }

    // This wave's tiles: wb, wb + ws, ..., n_my of them.  With one workgroup
    // per pair and split, a contiguous slice of the range (ws = 1).  With
    // balanced ranges every 4th tile from t_begin + wave (ws = 4): the 4 waves
    // walk an item together, front to back, so a shared prefix at the start
    // of a pair is read in a quarter of the time, and the sequences sharing
    // it (whose workgroups start it together on one XCD) stay close enough
    // to find each other's lines in L2 (32K FP8 batch, 8 sequences per
    // prefix: fetch 1.049 -> 1.017 x the unique K/V bytes, decode 216 -> 211
    // us).  One workgroup per pair measured no faster this way.
    const int span = it.t_end - it.t_begin;
    constexpr int ws = BAL ? kDecodeWaves : 1;
    int wb, n_my;
    if constexpr (ws == 1) {
      const int per_w = span > 0 ? (span + kDecodeWaves - 1) / kDecodeWaves : 0;
      wb = it.t_begin + wave * per_w;
      n_my = max(0, min(it.t_end, wb + per_w) - wb);
    } else {
      wb = it.t_begin + wave;
      n_my = span > wave ? (span - wave + ws - 1) / ws : 0;
    }

    const int32_t* bt_row = p.block_tables + (size_t)it.s * p.max_blocks_per_seq;
    const size_t head_bytes = (size_t)p.block_size * ROW;
    const size_t block_bytes = head_bytes * p.h_kv;
    const uint8_t* k_head = p.k_cache + it.kvh * head_bytes;
    const uint8_t* v_head = p.v_cache + it.kvh * head_bytes;
    const int k_lane = lane * 16;                           // K: 16 bytes of each 1 KiB piece
    const int v_lane = (4 * q4) * ROW + lo16 * Tile::VB;    // V: row 4 q4 + rr, chunk lo16
    // Direct loads: 1 KiB piece j of a tile (rows 4 j .. 4 j + 3) lands in
    // LDS in lane order, lane (q4, lo16) at chunk lo16 of row 4 j + q4, so a
    // lane reads the memory chunk whose swizzled place that is: K chunk
    // lo16 ^ (row & 7), V chunk lo16 ^ ((row & 7) << 1); row & 7 is
    // 4 (j & 1) + q4, so pieces 0, 2 and 1, 3 share an offset.
    const int dk_even = q4 * ROW + ((lo16 ^ q4) << 4);
    const int dk_odd = q4 * ROW + ((lo16 ^ q4 ^ 4) << 4);
    const int dv_even = q4 * ROW + ((lo16 ^ (q4 << 1)) << 4);
    const int dv_odd = q4 * ROW + ((lo16 ^ (q4 << 1) ^ 8) << 4);

    // Decode step: the wave whose tiles include the sequence's last position
    // (the last tile of the last split) appends the new token: it computes
    // that tile with the new rows (staged in LDS at the start) in place of the
    // loaded ones, and writes them to the pool after its last tile.  No other
    // wave or workgroup reads that position, so nothing waits for the write.
    const bool owner = AP && it.append && it.t_end == it.n_tiles && n_my > 0 && wb + ws * (n_my - 1) == it.n_tiles - 1;
    const int last_tok0 = (it.n_tiles - 1) * kTileTokens;
    const int stage_tok0 = (n_my >= 2 ? wb + ws : wb) * kTileTokens;  // direct loads: where the owner stages
    int last_phys = -1;  // physical block of the last position (owner wave)

    auto compute_tile = [&](Tile& r, bool valid, int stage) {
      const int lim = valid ? r.lim : 0;
      uint8_t* kt = reinterpret_cast<uint8_t*>(sm.t.ktile[wave]);
      u32x4* dks = sm.t.dk[wave][DMA ? stage : 0];
      u32x4* dvs = sm.t.dv[wave][DMA ? stage : 0];
      if constexpr (DMA) {
        // this tile's direct loads are done when only the next tile's 8
        // (issued after them) are in flight
        static_assert(KCH == 4 && VDW == 4 && NBUF == 2, "direct loads: 4 K and 4 V loads per tile, one tile ahead");
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      } else {
        // 0) K rows into the wave's LDS tile (lane l of load c holds chunk
        //    l % LPR of row RPK c + l / LPR)
#pragma unroll
        for (int c = 0; c < KCH; ++c)
          *reinterpret_cast<u32x4*>(kt + (Tile::RPK * c + lane / Tile::LPR) * Tile::KLDS + (lane % Tile::LPR) * 16) =
              r.k[c];
      }
      if constexpr (AP && DMA) {
        // the owner converts the new rows (loaded in its first chunk) into the
        // pools' element type at its second tile, or its only one: the rows'
        // loads came before that tile's, so they have landed, and the LDS
        // work overlaps the ring instead of lengthening the last tile
        if (owner && valid && r.tok0 == stage_tok0) stage_new_token();
      }
      if constexpr (AP) {
        if (owner && valid && r.tok0 == last_tok0) {  // the tile holding the new token (wave-uniform)
          const int row = it.ctx - 1 - r.tok0;
          if constexpr (DMA) {
            if (lane < 16) {
              dks[16 * row + (lane ^ (row & 7))] = *reinterpret_cast<const u32x4*>(&sm.t.newrow[wave][0][lane * 16]);
              dvs[16 * row + (lane ^ ((row & 7) << 1))] =
                  *reinterpret_cast<const u32x4*>(&sm.t.newrow[wave][1][lane * 16]);
            }
          } else if (lane < Tile::LPR) {
            *reinterpret_cast<u32x4*>(kt + row * Tile::KLDS + lane * 16) =
                *reinterpret_cast<const u32x4*>(&sm.t.newrow[wave][0][lane * 16]);
          }
          if constexpr (!DMA) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              if (4 * q4 + rr == row) {
#pragma unroll
                for (int w = 0; w < VDW; ++w)
                  r.v[rr][w] = *reinterpret_cast<const uint32_t*>(&sm.t.newrow[wave][1][lo16 * Tile::VB + 4 * w]);
              }
            }
          }
        }
      }
      // K in the operand layout: lane (lo16, q4) holds chunk q4 + 4 c of row lo16
      u32x4 kr[KCH];
      if constexpr (DMA) {
#pragma unroll
        for (int c = 0; c < KCH; ++c) kr[c] = dks[16 * lo16 + ((q4 + 4 * c) ^ (lo16 & 7))];
      } else {
#pragma unroll
        for (int c = 0; c < KCH; ++c)
          kr[c] = *reinterpret_cast<const u32x4*>(kt + lo16 * Tile::KLDS + (q4 + 4 * c) * 16);
      }
      // 1) scores for the 16 tokens of the tile against each (padded) row tile
      f32x4 sc[RT];
#pragma unroll
      for (int k = 0; k < RT; ++k) sc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        u32x4 a;
        if constexpr (KV == kFP8) {
          const uint32_t w0 = kr[kk >> 1][2 * (kk & 1)], w1 = kr[kk >> 1][2 * (kk & 1) + 1];
          a = u32x4{fp8x2_to_pair<CT, false>(w0), fp8x2_to_pair<CT, true>(w0), fp8x2_to_pair<CT, false>(w1),
                    fp8x2_to_pair<CT, true>(w1)};
        } else {
          a = kr[kk];
        }
#pragma unroll
        for (int k = 0; k < RT; ++k) sc[k] = mfma_16x16x32<CT>(a, qop[k][kk], sc[k]);
      }
      mfma_guard();

      // 2) V -> LDS in its natural layout; masked rows are zeroed first (the
      //    direct loads put V there themselves, rows past the context as
      //    zeros from the range check)
      const bool partial = lim < kTileTokens;
      if (!DMA && partial) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (4 * q4 + rr >= lim) {
#pragma unroll
            for (int w = 0; w < VDW; ++w) r.v[rr][w] = 0u;
          }
      }
      // Row t of the tile, 16-byte chunk c sits at chunk c ^ swz(t) of row t:
      // the transposed reads below then touch all banks evenly.
      auto vt_chunk = [&](int t, int c) { return t * VCH + (c ^ ((t & (VCH / 2 - 1)) << 1)); };
      u32x4* vt = DMA ? dvs : sm.t.vtile[wave];
#pragma unroll
      for (int rr = 0; rr < (DMA ? 0 : 4); ++rr) {
        const int t = 4 * q4 + rr;  // this lane holds d = lo16 * D/16 ... of row t
        uint32_t w16[D / 32];       // those D/16 elements as 16-bit pairs
        if constexpr (KV == kFP8) {
#pragma unroll
          for (int w = 0; w < VDW; ++w) {  // FP8 V as f16 (exact), the PV product's type
            w16[2 * w] = fp8x2_to_pair<kF16, false>(r.v[rr][w]);
            w16[2 * w + 1] = fp8x2_to_pair<kF16, true>(r.v[rr][w]);
          }
        } else {
#pragma unroll
          for (int w = 0; w < VDW; ++w) w16[w] = r.v[rr][w];
        }
        if constexpr (D == 128) {
          vt[vt_chunk(t, lo16)] = u32x4{w16[0], w16[1], w16[2], w16[3]};
        } else {
          reinterpret_cast<u32x2*>(vt + vt_chunk(t, lo16 >> 1))[lo16 & 1] = u32x2{w16[0], w16[1]};
        }
      }
      compiler_fence();

      // 3) online softmax (log2 domain), per row tile; row g = lo16, tokens
      //    4*q4 + rr; probabilities of those tokens as hi + lo 16-bit parts
      //    (p = hi + lo + O(2^-16 p)), the B operands of the PV products
      u32x2 p_hi[RT], p_lo[RT];
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        float s[4];
        // causal limit of this lane's row within the tile (several query tokens)
        const int row_cut = MT ? min(lim, row_lim[k] - r.tok0) : lim;
        if constexpr (MT) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) s[rr] = sc[k][rr] * p.scale_log2;
          // wave-uniform: a whole tile before the first new token's position
          // is seen by every row, so it skips the selects
          if (partial || r.tok0 + kTileTokens > first_row_lim) {
            asm volatile("");  // keeps this a branch instead of selects on every tile
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              if (4 * q4 + rr >= row_cut) s[rr] = kNegInf;
          }
        } else {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) s[rr] = sc[k][rr] * p.scale_log2;
          if (partial) {       // wave-uniform: full decode tiles skip the selects
            asm volatile("");  // keeps this a branch instead of selects on every tile
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              if (4 * q4 + rr >= row_cut) s[rr] = kNegInf;
          }
        }
        // Each lane tests its own 4 scores against its row's running max.  Only
        // when a lane of the wave exceeds it by more than the slack (always for
        // the first tile with a finite score) are the row maxima formed across
        // the 4 lanes of each row and the state rescaled; otherwise the tile
        // needs no cross-lane step at all.
        const float mx_lane = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        if (__builtin_amdgcn_ballot_w64(mx_lane > m_run[k] + kRescaleSlack) != 0) {
          float mx = fmaxf(mx_lane, shfl_xor_f32(mx_lane, 16));
          mx = fmaxf(mx, shfl_xor_f32(mx, 32));
          const bool grow = mx > m_run[k] + kRescaleSlack;  // the same on the 4 lanes of a row
          const float m_new = grow ? mx : m_run[k];
          const float alpha = grow ? fast_exp2(m_run[k] - m_new) : 1.f;  // 0 when m_run is -inf
          l_run[k] *= alpha;
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[k][n] *= alpha;
          m_run[k] = m_new;
        }
        const float m_use = m_run[k] == kNegInf ? 0.f : m_run[k];
        float pr[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) pr[rr] = fast_exp2(s[rr] - m_use);
        l_run[k] += (pr[0] + pr[1]) + (pr[2] + pr[3]);

        if constexpr (KV == kFP8) {
          // FP8 V carries 4 significant bits; P rounded once to f16 (11 bits,
          // round to nearest even) costs about 2e-4 rel-L2 of the output
          // against the float64 oracle, and one f16 MFMA per 16 rows of d
          // replaces the hi + lo contraction (fewer VALU and MFMA cycles: the
          // FP8 4-token step 245 -> 235 us, decode 212 -> 210 us)
          typedef _Float16 h2v __attribute__((ext_vector_type(2)));
          const h2v p01 = {(_Float16)pr[0], (_Float16)pr[1]}, p23 = {(_Float16)pr[2], (_Float16)pr[3]};
          p_hi[k] = u32x2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
          p_lo[k] = u32x2{0u, 0u};
        } else if constexpr (CT == kBF16) {
          float lo_part[4];
          uint32_t hb[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            hb[rr] = __float_as_uint(pr[rr]) & 0xffff0000u;
            lo_part[rr] = pr[rr] - __uint_as_float(hb[rr]);
          }
          p_hi[k] = u32x2{__builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u),
                          __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u)};
          p_lo[k] = u32x2{__builtin_amdgcn_perm(__float_as_uint(lo_part[1]), __float_as_uint(lo_part[0]), 0x07060302u),
                          __builtin_amdgcn_perm(__float_as_uint(lo_part[3]), __float_as_uint(lo_part[2]), 0x07060302u)};
        } else {
          const auto h01 = __builtin_amdgcn_cvt_pkrtz(pr[0], pr[1]);
          const auto h23 = __builtin_amdgcn_cvt_pkrtz(pr[2], pr[3]);
          const auto l01 = __builtin_amdgcn_cvt_pkrtz(pr[0] - (float)h01[0], pr[1] - (float)h01[1]);
          const auto l23 = __builtin_amdgcn_cvt_pkrtz(pr[2] - (float)h23[0], pr[3] - (float)h23[1]);
          p_hi[k] = u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
          p_lo[k] = u32x2{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)};
        }
      }

      // 4) O^T += V^T P^T: per 16 rows of d, one 16x16x32 MFMA whose
      //    contraction runs over the tile's 16 tokens twice, once with the hi
      //    and once with the lo part of P: the 8 contraction slots of lane
      //    group q4 are (tokens 4 q4 .. 4 q4 + 3, hi) then (the same tokens,
      //    lo), so its A operand is the 8-byte V^T cell of those 4 tokens
      //    twice and its B operand the hi cell followed by the lo cell (FP8
      //    caches: one 16x16x16 f16 MFMA, the cell and the f16 P cell)
      // A operands by transposing reads: lane (4k + m) of each 16-lane group
      // points at 4 elements d = 16n + 4m .. +3 of token 4*q4 + k, and lane j
      // receives element j of those 4 tokens' rows, i.e. V^T[16n + j][4*q4 .. +3]
      u32x2 cell[NT];
      {
        const int t = 4 * q4 + (lo16 >> 2);
        const int m = lo16 & 3;
        typedef __attribute__((address_space(3))) char lds_char;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          lds_char* a = (lds_char*)(vt + vt_chunk(t, 2 * n + (m >> 1))) + 8 * (m & 1);
          cell[n] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                  (__attribute__((address_space(3))) v4i16*)a));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        const u32x4 pb = u32x4{p_hi[k][0], p_hi[k][1], p_lo[k][0], p_lo[k][1]};
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          if constexpr (KV == kFP8) {  // f16 V^T cell x f16 P, contraction over the 4 tokens
            typedef _Float16 h4v __attribute__((ext_vector_type(4)));
            acc[k][n] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4v, cell[n]),
                                                              __builtin_bit_cast(h4v, p_hi[k]), acc[k][n], 0, 0, 0);
          } else {
            acc[k][n] = mfma_16x16x32<CT>(u32x4{cell[n][0], cell[n][1], cell[n][0], cell[n][1]}, pb, acc[k][n]);
          }
        }
      }
      mfma_guard();
      compiler_fence();
    };

    for (int c0 = 0; c0 < n_my; c0 += 64) {
      const int cn = min(64, n_my - c0);  // tiles in this chunk (>= 1)
      const int t0 = wb + ws * c0;        // its first tile
      // Lane j holds the physical block of tile t0 + j (clamped into the chunk,
      // so only table entries of blocks the context covers are read).
      const int ids = bt_row[(t0 + ws * min(lane, cn - 1)) >> p.tile_shift];
      // Decode step: every wave loads its (sequence, KV head)'s new K and V rows
      // right after the chunk's block ids, so waiting for the ids (L2-resident)
      // never waits for these (cold) rows, and before the chunk's first tile,
      // whose loads they arrive with; only the wave that owns the last
      // position reads them, in its first chunk (the others' loads read nothing).
      // Lane l < CH holds 8 elements of K, lane CH + l those of V (the rest
      // none).  The loads are unconditional, whatever the element type (a
      // branch here would make the compiler drain every load in flight, and so
      // would loads placed before the loop): each lane reads 32
      // bytes at its chunk, 8 at a time, through buffer resources over new_k and
      // new_v, whose range check returns zeros past the arrays' end and for the
      // lanes a resource does not serve (chunks and arrays are multiples of 8
      // bytes, so no 8-byte read straddles the end); 8 elements take the first
      // 8, 16 or 32 bytes.
      int nr_off = 0, nr_avail = 0;  // direct loads of the new rows: lane offset, bytes readable
      if constexpr (AP) {
        // wave-uniform (kept in scalar registers: a resource built from vector
        // registers would need a loop over the distinct values)
        const int es = __builtin_amdgcn_readfirstlane(p.new_dtype == kF32 ? 4 : (p.new_dtype == kFP8 ? 1 : 2));
        const int bytes = __builtin_amdgcn_readfirstlane(p.units * D * es);  // [S, h_kv, D]
        const int row = __builtin_amdgcn_readfirstlane((it.s * p.h_kv + it.kvh) * D * es);
        const int off_k = lane < CH ? row + lane * 8 * es : bytes;
        const int off_v = lane >= CH && lane < 2 * CH ? row + (lane - CH) * 8 * es : bytes;
        // only the owner uses the rows, staging them during its first chunk:
        // every other wave and chunk issues the same loads over resources of
        // size 0, which read nothing (the same instructions keep the same waits)
        const int avail = owner && c0 == 0 ? bytes : 0;
        if constexpr (DMA) {
          // the whole rows go straight into this wave's LDS staging, 16 bytes
          // per lane (lanes past the row read nothing), after the first ring
          // tile's loads (below): the block ids' wait never waits for them
          nr_off = lane * 16 < D * es ? row + lane * 16 : bytes;
          nr_avail = avail;
        } else {
          const __amdgpu_buffer_rsrc_t rk =
              __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.new_k), (short)0, avail, kBufferWord3);
          const __amdgpu_buffer_rsrc_t rv =
              __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.new_v), (short)0, avail, kBufferWord3);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            kx[w] = kv_load8<false>(rk, off_k, 8 * w);
            vx[w] = kv_load8<false>(rv, off_v, 8 * w);
          }
        }
      }

      // jr: the ring step's tile of the chunk (wave-uniform); jr >= cn past the
      // end, where the loads return zeros without a memory access
      auto load_tile = [&](Tile& r, int jr, int stage) {
        const int j = min(jr, cn - 1);
        const int tok0 = (t0 + ws * j) * kTileTokens;
        int phys = __builtin_amdgcn_readlane(ids, j);
        const bool ok = (unsigned)phys < (unsigned)p.num_blocks;
        phys = ok ? phys : 0;
        const int rem = it.ctx - tok0;
        r.lim = ok ? (rem < kTileTokens ? rem : kTileTokens) : 0;
        r.tok0 = tok0;
        const int sub = (t0 + ws * j) & ((1 << p.tile_shift) - 1);  // 16-token tile within the block
        const size_t off = (size_t)phys * block_bytes + (size_t)sub * (kTileTokens * ROW);
        // the rows inside the context only: the unused tail slots of a
        // sequence's last block come back as zeros without being read
        const int bytes = ok && jr < cn ? r.lim * ROW : 0;
        const __amdgpu_buffer_rsrc_t kr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(k_head + off), (short)0, bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t vr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(v_head + off), (short)0, bytes, kBufferWord3);
        if constexpr (DMA) {
          typedef __attribute__((address_space(3))) void lds_void;
          const i32x4 kd = raw_rsrc(k_head + off, bytes);
          const i32x4 vd = raw_rsrc(v_head + off, bytes);
          const uint32_t kl = (uint32_t)(uintptr_t)(lds_void*)sm.t.dk[wave][stage];
          const uint32_t vl = (uint32_t)(uintptr_t)(lds_void*)sm.t.dv[wave][stage];
          // every LDS read of this stage (the tile two steps back) is done
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            lds_load16<STREAM>(kd, kl + 1024 * j, (j & 1) ? dk_odd : dk_even, 1024 * j);
            lds_load16<STREAM>(vd, vl + 1024 * j, (j & 1) ? dv_odd : dv_even, 1024 * j);
          }
          return;
        }
#pragma unroll
        for (int c = 0; c < KCH; ++c) r.k[c] = kv_load16<STREAM>(kr, k_lane, c * 1024);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          if constexpr (VDW == 4) {
            const u32x4 x = kv_load16<STREAM>(vr, v_lane, rr * ROW);
            r.v[rr][0] = x[0];
            r.v[rr][1] = x[1];
            r.v[rr][2] = x[2];
            r.v[rr][3] = x[3];
          } else if constexpr (VDW == 2) {
            const u32x2 x = kv_load8<STREAM>(vr, v_lane, rr * ROW);
            r.v[rr][0] = x[0];
            r.v[rr][1] = x[1];
          } else {
            r.v[rr][0] = kv_load4<STREAM>(vr, v_lane, rr * ROW);
          }
        }
      };

      // Ring of NBUF buffers: tile i + NBUF - 1 is loaded while tile i is computed.
      Tile buf[NBUF];
#pragma unroll
      for (int b = 0; b < NBUF - 1; ++b) {
        load_tile(buf[b], b, b);
        // keep the tiles' loads in ring order, so that waiting for the oldest
        // tile never waits for a younger one
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (AP) {
        if (owner && c0 + cn == n_my) last_phys = __builtin_amdgcn_readlane(ids, cn - 1);
        if constexpr (DMA) {
          // first chunk only: the staging then holds the rows until the owner
          // converts them at its second tile (or its only one)
          if (c0 == 0) {
            typedef __attribute__((address_space(3))) void lds_void;
            lds_load16<false>(raw_rsrc(p.new_k, nr_avail), (uint32_t)(uintptr_t)(lds_void*)sm.t.nraw[wave][0], nr_off, 0);
            lds_load16<false>(raw_rsrc(p.new_v, nr_avail), (uint32_t)(uintptr_t)(lds_void*)sm.t.nraw[wave][1], nr_off, 0);
          }
        } else {
          // the owner stages the new token once its first tile is in flight
          if (c0 == 0 && owner) stage_new_token();
        }
      }
      // Pacing (PACE, launched only when some CUs hold one workgroup and
      // others two): a workgroup alone on its CU waits after each tile but
      // its last, in short sleeps on the real-time counter (100 MHz), for a
      // share of the time the tile's step took (from the second step on: the
      // first includes the start's dependent reads).  Wave-uniform; its loads
      // of the next tiles are in flight meanwhile.
      static_assert(!PACE || (!DMA && !BAL && NBUF == 2), "pacing: the register ring of 8 KiB tiles");
      const bool pace = PACE && (int)blockIdx.x >= p.pace_lo && (int)blockIdx.x < p.pace_hi &&
                        it.t_end - it.t_begin >= kPaceMinTiles;
      uint64_t t_step = 0;
      for (int i = 0; i < cn; i += NBUF) {
#pragma unroll
        for (int b = 0; b < NBUF; ++b) {
          load_tile(buf[(b + NBUF - 1) % NBUF], i + b + NBUF - 1, (b + NBUF - 1) % NBUF);
          // a ring step past the wave's last tile computes nothing (its
          // loads read nothing); the kernels holding two row tiles measured
          // faster computing it on zeros than branching around it
          if (RT == 2 || i + b < cn) compute_tile(buf[b], i + b < cn, b);
          if (PACE && __builtin_expect(pace, 0)) {
            const uint64_t now = __builtin_amdgcn_s_memrealtime();
            // no wait after the wave's last tile: only its merge is left
            if (t_step != 0 && c0 + i + b + 1 < n_my) {
              const uint64_t step = now - t_step < kPaceMaxStepTicks ? now - t_step : kPaceMaxStepTicks;
              const uint64_t until = now + step * (uint64_t)p.pace_share32 / 32;
              uint64_t t = now;
              while (t < until) {
                __builtin_amdgcn_s_sleep(2);
                t = __builtin_amdgcn_s_memrealtime();
              }
              t_step = t;
            } else {
              t_step = now;
            }
          }
        }
      }
    }
    if constexpr (DMA) {
      // the ring's last direct loads (zeros past the wave's tiles) land in
      // LDS that the merge below reuses
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // The new token's slot and rows (the owner's lanes of its rows): the rows
    // leave the LDS, which the merge reuses, for registers, and are stored
    // after the merge, whose barriers would otherwise wait for the store.
    [[maybe_unused]] uint8_t* new_dst = nullptr;
    [[maybe_unused]] Chunk8<KV> new_rows{};
    if constexpr (AP) {
      if (owner && (unsigned)last_phys < (unsigned)p.num_blocks && lane < 2 * CH) {
        const bool is_v = lane >= CH;
        const int c = is_v ? lane - CH : lane;
        const int pos = it.ctx - 1;
        const int off = pos - (pos / p.block_size) * p.block_size;
        const size_t dst = (((size_t)last_phys * p.h_kv + it.kvh) * p.block_size + off) * ROW + c * 8 * Tile::ES;
        new_rows = load8<KV>(&sm.t.newrow[wave][is_v ? 1 : 0][c * 8 * Tile::ES]);
        new_dst = (is_v ? p.v_store : p.k_store) + dst;
      }
    }

#pragma unroll
    for (int k = 0; k < RT; ++k) {
      float l_row = l_run[k] + shfl_xor_f32(l_run[k], 16);
      l_row += shfl_xor_f32(l_row, 32);
      // every wave is done with its tiles (first row tile) or the previous
      // row tile's merge has read the LDS: reuse it
      __syncthreads();
#pragma unroll
      for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(&sm.merge.acc[wave][lo16][16 * n + 4 * q4]) = acc[k][n];
      if (q4 == 0) {
        sm.merge.m[wave][lo16] = m_run[k];
        sm.merge.l[wave][lo16] = l_row;
      }
      __syncthreads();
      finish<D, MT, RT, !BAL>(p, it, k, sm.merge);
    }
    if constexpr (AP) {
      if (new_dst != nullptr) store8<KV>(new_dst, new_rows);
    }
  };

  Item it;
  if constexpr (!BAL) {  // one item: a pair (row group) and split
    if (!get_item<MT, RT, LPT>(p, it, sm.lpt)) return;
    run_item(it);
  } else {  // the items of this workgroup's range, one after the other
    Balanced bal;
    balanced_setup(p, sm_pre, bal);
    while (balanced_next(p, sm_pre, bal, it)) {
      run_item(it);
      __syncthreads();  // this item's merge is done with the LDS
    }
    balanced_zeros<D, MT, RT>(p, sm_pre, bal);
  }
}

// ---------------------------------------------------------------- vector path

template <int DT>
__device__ __forceinline__ float load_elem(const void* base, size_t i) {
  if constexpr (DT == kF32) return static_cast<const float*>(base)[i];
  else if constexpr (DT == kFP8) return elem_to_f32<kFP8>(static_cast<const uint8_t*>(base)[i]);
  else return elem_to_f32<DT>(static_cast<const uint16_t*>(base)[i]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f32(v, m);
  return v;
}

template <int KV, int QT, int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_vector_kernel(Params p) {
  constexpr int J = D / 64;
  __shared__ MergeSmem<D> sm;

  Item it;
  if (!get_item<false, 1>(p, it, nullptr)) return;
  if (it.n_tiles == 0) {
    if (it.split == 0) write_zeros<D, false>(p, it, 0);
    return;
  }
  if (it.split >= it.n_splits_seq) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = p.group;

  float qv[kMaxGroup][J], acc[kMaxGroup][J], m[kMaxGroup], l[kMaxGroup];
  const size_t qrow0 = ((size_t)it.s * p.h_q + it.kvh * G) * D;
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float x = load_elem<QT>(p.q, qrow0 + (size_t)(g < G ? g : G - 1) * D + lane + 64 * j);
      qv[g][j] = g < G ? x : 0.f;
      acc[g][j] = 0.f;
    }
    m[g] = kNegInf;
    l[g] = 0.f;
  }

  const int32_t* bt_row = p.block_tables + (size_t)it.s * p.max_blocks_per_seq;
  for (int ti = it.t_begin + wave; ti < it.t_end; ti += kDecodeWaves) {
    const int t0 = ti * kTileTokens;
    const int t1 = min(t0 + kTileTokens, it.ctx);
    for (int t = t0; t < t1; ++t) {
      const int phys = bt_row[t / p.block_size];
      if ((unsigned)phys >= (unsigned)p.num_blocks) continue;
      const size_t row = (((size_t)phys * p.h_kv + it.kvh) * p.block_size + t % p.block_size) * D;
      float kd[J], vd[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        kd[j] = load_elem<KV>(p.k_cache, row + lane + 64 * j);
        vd[j] = load_elem<KV>(p.v_cache, row + lane + 64 * j);
      }
#pragma unroll
      for (int g = 0; g < kMaxGroup; ++g) {
        if (g < G) {
          float part = 0.f;
#pragma unroll
          for (int j = 0; j < J; ++j) part += qv[g][j] * kd[j];
          const float s = wave_sum(part) * p.scale_log2;
          const float m_new = fmaxf(m[g], s);
          const float alpha = fast_exp2(m[g] - m_new);
          const float pe = fast_exp2(s - m_new);
          l[g] = l[g] * alpha + pe;
#pragma unroll
          for (int j = 0; j < J; ++j) acc[g][j] = acc[g][j] * alpha + pe * vd[j];
          m[g] = m_new;
        }
      }
    }
  }

#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
#pragma unroll
    for (int j = 0; j < J; ++j) sm.acc[wave][g][lane + 64 * j] = acc[g][j];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
      sm.m[wave][g] = m[g];
      sm.l[wave][g] = l[g];
    }
  }
  __syncthreads();
  finish<D, false, 1>(p, it, 0, sm);
}

template <typename K>
hipError_t launch(K kernel, int grid, const Params& p, hipStream_t stream) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kDecodeThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool MT, bool AP, int RT, bool ST, bool BAL, bool LPT, bool DMA>
hipError_t dispatch_mfma_types(const DecodeLaunch& a, int grid, const Params& p, hipStream_t s) {
  if (a.kv_dtype == kBF16 && a.q_dtype == kBF16)
    return launch(decode_mfma_kernel<kBF16, kBF16, D, MT, AP, RT, ST, BAL, LPT, DMA>, grid, p, s);
  if (a.kv_dtype == kF16 && a.q_dtype == kF16)
    return launch(decode_mfma_kernel<kF16, kF16, D, MT, AP, RT, ST, BAL, LPT, DMA>, grid, p, s);
  if constexpr (!DMA) {
    if (a.kv_dtype == kFP8 && a.q_dtype == kBF16)
      return launch(decode_mfma_kernel<kFP8, kBF16, D, MT, AP, RT, ST, BAL, LPT, false>, grid, p, s);
    if (a.kv_dtype == kFP8 && a.q_dtype == kF16)
      return launch(decode_mfma_kernel<kFP8, kF16, D, MT, AP, RT, ST, BAL, LPT, false>, grid, p, s);
  }
  return hipErrorInvalidValue;
}

// Kernels with balanced ranges have no order to choose; the others are built
// with and without the longest-first ranking, so that a launch that does not
// rank runs no trace of it.  The LDS ring is built for the one-row-tile
// kernels over 16-bit caches with 256-byte rows, and taken when the host asks
// for it.
template <int D, bool MT, bool AP, int RT, bool ST, bool BAL = false>
hipError_t dispatch_mfma(const DecodeLaunch& a, int grid, const Params& p, hipStream_t s) {
  if constexpr (D == 128 && RT == 1 && !BAL) {
    if (a.lds_ring && a.kv_dtype != kFP8) {
      if (p.lpt_shift >= 0) return dispatch_mfma_types<D, MT, AP, RT, ST, false, true, true>(a, grid, p, s);
      return dispatch_mfma_types<D, MT, AP, RT, ST, false, false, true>(a, grid, p, s);
    }
  }
  if constexpr (!BAL) {
    if (p.lpt_shift >= 0) return dispatch_mfma_types<D, MT, AP, RT, ST, false, true, false>(a, grid, p, s);
  }
  if constexpr (D == 128 && !BAL && ((!MT && RT == 1) || (MT && RT == 2 && ST))) {
    // pacing of the workgroups alone on their CUs: the register ring over
    // 16-bit caches (FP8 tiles measured slower paced), for one token per
    // sequence, and for several whose two row tiles one workgroup holds as
    // the only reader of its K/V
    if (p.pace_hi > p.pace_lo) {
      if (a.kv_dtype == kBF16 && a.q_dtype == kBF16)
        return launch(decode_mfma_kernel<kBF16, kBF16, D, MT, AP, RT, ST, false, false, false, true>, grid, p, s);
      if (a.kv_dtype == kF16 && a.q_dtype == kF16)
        return launch(decode_mfma_kernel<kF16, kF16, D, MT, AP, RT, ST, false, false, false, true>, grid, p, s);
    }
  }
  return dispatch_mfma_types<D, MT, AP, RT, ST, BAL, false, false>(a, grid, p, s);
}

template <int D>
hipError_t dispatch(const DecodeLaunch& a, int grid, const Params& p, hipStream_t s) {
  if (a.query_start != nullptr) {
    if (!a.matrix_core || a.new_k != nullptr) return hipErrorInvalidValue;
    // one row group: this workgroup is the K/V's only reader
    const bool only_reader = p.row_groups == 1;
    if (p.balanced) {  // balanced ranges hold every row of a pair: one row group
      if (!only_reader) return hipErrorInvalidValue;
      return multi_tiles_per_workgroup(p.row_tiles) == 2 ? dispatch_mfma<D, true, false, 2, true, true>(a, grid, p, s)
                                                         : dispatch_mfma<D, true, false, 1, true, true>(a, grid, p, s);
    }
    if (multi_tiles_per_workgroup(p.row_tiles) == 2) {
      return only_reader ? dispatch_mfma<D, true, false, 2, true>(a, grid, p, s)
                         : dispatch_mfma<D, true, false, 2, false>(a, grid, p, s);
    }
    return only_reader ? dispatch_mfma<D, true, false, 1, true>(a, grid, p, s)
                       : dispatch_mfma<D, true, false, 1, false>(a, grid, p, s);
  }
  if (a.new_k != nullptr) {
    if (!a.matrix_core) return hipErrorInvalidValue;
    return p.balanced ? dispatch_mfma<D, false, true, 1, true, true>(a, grid, p, s)
                      : dispatch_mfma<D, false, true, 1, true>(a, grid, p, s);
  }
  if (a.matrix_core) {
    return p.balanced ? dispatch_mfma<D, false, false, 1, true, true>(a, grid, p, s)
                      : dispatch_mfma<D, false, false, 1, true>(a, grid, p, s);
  } else {
    if (a.kv_dtype == kF32 && a.q_dtype == kF32) return launch(decode_vector_kernel<kF32, kF32, D>, grid, p, s);
    if (a.kv_dtype == kBF16 && a.q_dtype == kBF16) return launch(decode_vector_kernel<kBF16, kBF16, D>, grid, p, s);
    if (a.kv_dtype == kF16 && a.q_dtype == kF16) return launch(decode_vector_kernel<kF16, kF16, D>, grid, p, s);
    if (a.kv_dtype == kFP8 && a.q_dtype == kBF16) return launch(decode_vector_kernel<kFP8, kBF16, D>, grid, p, s);
    if (a.kv_dtype == kFP8 && a.q_dtype == kF16) return launch(decode_vector_kernel<kFP8, kF16, D>, grid, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream) {
  const bool multi = a.query_start != nullptr;
  const int row_tiles = multi ? multi_row_tiles(a.h_q, a.h_kv, a.max_query_len) : 1;
  const WorkspaceLayout L =
      multi ? multi_workspace_layout(a.num_seqs, a.h_kv, a.head_dim, row_tiles, a.num_splits, a.balanced_workgroups)
            : decode_workspace_layout(a.num_seqs, a.h_q, a.h_kv, a.head_dim, a.num_splits, a.balanced_workgroups,
                                      a.counter_slots);
  Params p;
  p.out = a.out;
  p.q = a.q;
  p.k_cache = static_cast<const uint8_t*>(a.k_cache);
  p.v_cache = static_cast<const uint8_t*>(a.v_cache);
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  char* ws = static_cast<char*>(a.workspace);
  p.counters = reinterpret_cast<int32_t*>(ws + L.counters);
  p.ws_ml = reinterpret_cast<float*>(ws + L.ml);
  p.ws_acc = reinterpret_cast<float*>(ws + L.acc);
  p.h_q = a.h_q;
  p.h_kv = a.h_kv;
  p.group = a.h_q / a.h_kv;
  p.block_size = a.block_size;
  p.num_blocks = a.num_blocks;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_splits = a.num_splits;
  p.tiles_per_split = a.tiles_per_split;
  p.tile_shift = 0;
  while ((kTileTokens << p.tile_shift) < a.block_size) ++p.tile_shift;
  p.units = a.num_seqs * a.h_kv;
  p.scale_log2 = a.scale_log2;
  p.v_scale = a.v_scale;
  p.out_dtype = a.out_dtype;
  p.query_start = a.query_start;
  p.num_query_tokens = a.num_query_tokens;
  p.max_query_len = a.max_query_len;
  p.row_tiles = row_tiles;
  p.row_groups = multi ? multi_row_groups(row_tiles) : 1;
  p.balanced = a.balanced_workgroups > 0 ? 1 : 0;
  p.lpt_shift = a.lpt_shift;
  p.new_k = static_cast<const uint8_t*>(a.new_k);
  p.new_v = static_cast<const uint8_t*>(a.new_v);
  p.k_store = static_cast<uint8_t*>(const_cast<void*>(a.k_cache));
  p.v_store = static_cast<uint8_t*>(const_cast<void*>(a.v_cache));
  p.new_dtype = a.new_dtype;
  p.k_scale_enc = a.k_scale_enc;
  p.v_scale_enc = a.v_scale_enc;
  const int grid = p.balanced ? a.balanced_workgroups : ((p.units + 7) / 8) * 8 * p.row_groups * a.num_splits;
  if (grid == 0) return hipSuccess;
  p.pace_lo = p.pace_hi = p.pace_share32 = 0;
  if (a.pace && !p.balanced && grid > kComputeUnits && 2 * grid <= 3 * kComputeUnits &&
      a.tiles_per_split >= kPaceMinTiles) {
    p.pace_lo = grid - kComputeUnits;
    p.pace_hi = kComputeUnits;
    p.pace_share32 = pace_share32(grid - kComputeUnits, multi_tiles_per_workgroup(p.row_tiles));
  }
  if (a.head_dim == 128) return dispatch<128>(a, grid, p, stream);
  if (a.head_dim == 64) return dispatch<64>(a, grid, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
