// Host block manager: on-demand block allocation over a FIFO free list, with
// reference counts, fork and copy-on-write of a shared tail block.
//
// Follows "AI Engineering Visualised: KV cache" (intro: blocks are handed out
// only as a sequence grows), the "Paged KV Cache" tutorial (sections "Block
// Tables and Sharing": a block returns to the free list once nothing
// references it, prefix blocks shared by reference count, and a block of
// its own for a sequence that appends into a shared, partly filled last
// block; "Internal Fragmentation": only the last block is partly empty;
// "Answer Key" question 2: a growing sequence takes free blocks one by one
// and its earlier blocks never move) and "KV cache and PagedAttention in
// serving" ("The bonus: sharing via copy-on-write").
//
// The FIFO order, the all-or-nothing append and the (src, dst) report of a
// copy-on-write are this library's policy; the declarations in pkv.h state it.

#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

struct pkv_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> refcount;
  struct Seq {
    std::vector<int32_t> table;
    int64_t tokens = 0;
  };
  std::unordered_map<int32_t, Seq> seqs;
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t block_size) { return (tokens + block_size - 1) / block_size; }

}  // namespace

extern "C" {

pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pkv_bm** out) {
  if (out == nullptr || num_blocks <= 0 || block_size <= 0) return PKV_EINVAL;
  *out = nullptr;
  pkv_bm* bm = new (std::nothrow) pkv_bm();
  if (bm == nullptr) return PKV_EINVAL;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcount.assign(num_blocks, 0);
  if (free_order != nullptr) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return PKV_EINVAL;
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(b);
  }
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

pkv_status pkv_bm_append(pkv_bm* bm, int32_t seq, int32_t n_tokens, int64_t* slots_out, int32_t* cow_src,
                         int32_t* cow_dst) {
  if (bm == nullptr || seq < 0 || n_tokens < 0) return PKV_EINVAL;
  if (cow_src) *cow_src = -1;
  if (cow_dst) *cow_dst = -1;
  auto it = bm->seqs.find(seq);
  const int64_t held = it == bm->seqs.end() ? 0 : it->second.tokens;
  const int64_t have_blocks = it == bm->seqs.end() ? 0 : (int64_t)it->second.table.size();
  const int32_t bs = bm->block_size;
  // A partly filled last block that another sequence also references must be
  // replaced by a private copy before this sequence writes into it.
  const bool cow = n_tokens > 0 && held % bs != 0 && bm->refcount[it->second.table.back()] > 1;
  const int64_t needed = blocks_for(held + n_tokens, bs) - have_blocks + (cow ? 1 : 0);
  if (needed > (int64_t)bm->free_list.size()) return PKV_ENOSPC;

  pkv_bm::Seq& s = bm->seqs[seq];  // creates an empty sequence if new
  if (cow) {
    const int32_t src = s.table.back();
    const int32_t dst = bm->free_list.front();
    bm->free_list.pop_front();
    bm->refcount[src] -= 1;
    bm->refcount[dst] = 1;
    s.table.back() = dst;
    if (cow_src) *cow_src = src;
    if (cow_dst) *cow_dst = dst;
  }
  for (int32_t i = 0; i < n_tokens; ++i) {
    if (s.tokens % bs == 0) {  // the token starts a new block
      const int32_t fresh = bm->free_list.front();
      bm->free_list.pop_front();
      bm->refcount[fresh] = 1;
      s.table.push_back(fresh);
    }
    if (slots_out) slots_out[i] = (int64_t)s.table[s.tokens / bs] * bs + s.tokens % bs;
    s.tokens += 1;
  }
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_bm* bm, int32_t parent, int32_t child) {
  if (bm == nullptr || child < 0) return PKV_EINVAL;
  auto p = bm->seqs.find(parent);
  if (p == bm->seqs.end() || bm->seqs.count(child)) return PKV_EINVAL;
  pkv_bm::Seq copy = p->second;
  for (int32_t b : copy.table) bm->refcount[b] += 1;
  bm->seqs.emplace(child, std::move(copy));
  return PKV_OK;
}

pkv_status pkv_bm_free(pkv_bm* bm, int32_t seq) {
  if (bm == nullptr) return PKV_EINVAL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_EINVAL;
  for (int32_t b : it->second.table) {
    if (--bm->refcount[b] == 0) bm->free_list.push_back(b);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_bm_block_table(const pkv_bm* bm, int32_t seq, int32_t* out, int32_t cap, int32_t* n_blocks,
                       int32_t* n_tokens) {
  if (bm == nullptr) return PKV_EINVAL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_EINVAL;
  const auto& t = it->second.table;
  if (n_blocks) *n_blocks = (int32_t)t.size();
  if (n_tokens) *n_tokens = (int32_t)it->second.tokens;
  if (out != nullptr) {
    if ((int64_t)t.size() > cap) return PKV_EINVAL;
    std::copy(t.begin(), t.end(), out);
  }
  return PKV_OK;
}

pkv_status pkv_bm_export(const pkv_bm* bm, const int32_t* seqs, int32_t num_seqs, int32_t* tables, int32_t max_blocks,
                  int32_t* context_lens) {
  if (bm == nullptr || num_seqs < 0 || max_blocks < 0 || (num_seqs > 0 && (seqs == nullptr || tables == nullptr)))
    return PKV_EINVAL;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end() || (int64_t)it->second.table.size() > max_blocks) return PKV_EINVAL;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables + (int64_t)i * max_blocks;
    std::fill(row, row + max_blocks, -1);
    std::copy(s.table.begin(), s.table.end(), row);
    if (context_lens) context_lens[i] = (int32_t)s.tokens;
  }
  return PKV_OK;
}

int32_t pkv_bm_num_free(const pkv_bm* bm) { return bm ? (int32_t)bm->free_list.size() : -1; }

int32_t pkv_bm_refcount(const pkv_bm* bm, int32_t block) {
  if (bm == nullptr || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refcount[block];
}

pkv_status pkv_bm_free_list(const pkv_bm* bm, int32_t* out, int32_t cap, int32_t* n) {
  if (bm == nullptr) return PKV_EINVAL;
  if (n) *n = (int32_t)bm->free_list.size();
  if (out != nullptr) {
    if ((int64_t)bm->free_list.size() > cap) return PKV_EINVAL;
    std::copy(bm->free_list.begin(), bm->free_list.end(), out);
  }
  return PKV_OK;
}

}  // extern "C"
