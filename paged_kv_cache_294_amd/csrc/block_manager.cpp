// Host block manager: which pool blocks each sequence holds, who shares them, and the
// slots and copies a step needs. Plain C++ on the host; its outputs (block tables,
// slot_mapping, copy pairs) are what the device calls of this library consume.
//
// Rules (page "vLLM 部署深度指南", section "PagedAttention 原理", KV-cache listing: a
// FIFO free list starting as 0 .. num_blocks-1, ceil(n / block_size) blocks per sequence,
// an out-of-memory error when the list is empty; page "vLLM GitHub 项目 …", section 二,
// item 1: a new block only when the last one is full; item 4: sequences that share a
// prefix point at the same blocks):
//   allocate  a new sequence takes ceil(n / bs) blocks from the front of the free list,
//             all or none
//   append    the next token goes to the last block if it has room and no other
//             sequence references it; a full last block gets a fresh block appended; a
//             shared, partly filled last block is replaced by a fresh block and reported
//             as a (source, destination) copy that must run on the device first
//             (copy-on-write)
//   fork      the child shares every block of the parent (reference counts + 1)
//   free      every block of the sequence loses a reference, in table order; blocks left
//             with none go to the back of the free list
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

struct pa_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };
  // The free list is a FIFO of at most num_blocks entries, kept in a ring allocated once,
  // so taking and returning blocks never allocates.
  struct FreeList {
    std::vector<int32_t> ring;
    int64_t head = 0, count = 0;
    int64_t size() const { return count; }
    bool empty() const { return count == 0; }
    int32_t pop_front() {
      const int32_t b = ring[(size_t)head];
      head = head + 1 == (int64_t)ring.size() ? 0 : head + 1;
      --count;
      return b;
    }
    void push_back(int32_t b) {
      int64_t at = head + count;
      if (at >= (int64_t)ring.size()) at -= (int64_t)ring.size();
      ring[(size_t)at] = b;
      ++count;
    }
    int32_t at(int64_t i) const {
      int64_t k = head + i;
      if (k >= (int64_t)ring.size()) k -= (int64_t)ring.size();
      return ring[(size_t)k];
    }
  };
  int64_t num_blocks = 0;
  int32_t block_size = 16;
  FreeList free_list;
  std::vector<int32_t> refs;
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.pop_front();
    refs[(size_t)b] = 1;
    return b;
  }
};

namespace {

int64_t blocks_for(int64_t len, int32_t bs) { return (len + bs - 1) / bs; }

}  // namespace

PA_EXPORT pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, pa_block_manager** out) {
  if (out == nullptr) return PA_ERR_INVALID;
  *out = nullptr;
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0) return PA_ERR_INVALID;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (bm == nullptr) return PA_ERR_INVALID;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->refs.assign((size_t)num_blocks, 0);
    bm->free_list.ring.resize((size_t)num_blocks);
    for (int64_t b = 0; b < num_blocks; ++b) bm->free_list.push_back((int32_t)b);
  } catch (...) {
    delete bm;
    return PA_ERR_INVALID;
  }
  *out = bm;
  return PA_OK;
}

PA_EXPORT void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

PA_EXPORT pa_status pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, int64_t num_tokens) {
  if (bm == nullptr || num_tokens < 0 || bm->seqs.count(seq_id)) return PA_ERR_INVALID;
  const int64_t need = blocks_for(num_tokens, bm->block_size);
  if (need > (int64_t)bm->free_list.size()) return PA_ERR_EXHAUSTED;
  try {
    pa_block_manager::Seq s;
    s.blocks.reserve((size_t)need);
    bm->seqs.reserve(bm->seqs.size() + 1);
    for (int64_t j = 0; j < need; ++j) s.blocks.push_back(bm->take());  // cannot throw now
    s.len = num_tokens;
    bm->seqs.emplace(seq_id, std::move(s));
  } catch (...) {  // host memory: nothing was taken (the reserves come first)
    return PA_ERR_INVALID;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_append_slot(pa_block_manager* bm, int64_t seq_id, int64_t* slot,
                                      int64_t* copy_src, int64_t* copy_dst) {
  if (bm == nullptr || slot == nullptr || copy_src == nullptr || copy_dst == nullptr)
    return PA_ERR_INVALID;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID;
  pa_block_manager::Seq& s = it->second;
  *copy_src = *copy_dst = -1;
  const int64_t pos = s.len;
  const int64_t bs = bm->block_size;
  if (pos == (int64_t)s.blocks.size() * bs) {
    if (bm->free_list.empty()) return PA_ERR_EXHAUSTED;
    try {
      s.blocks.reserve(s.blocks.size() + 1);
    } catch (...) {
      return PA_ERR_INVALID;
    }
    s.blocks.push_back(bm->take());
  } else if (bm->refs[s.blocks.back()] > 1) {
    if (bm->free_list.empty()) return PA_ERR_EXHAUSTED;
    const int32_t old = s.blocks.back();
    const int32_t fresh = bm->take();
    bm->refs[old] -= 1;
    s.blocks.back() = fresh;
    *copy_src = old;
    *copy_dst = fresh;
  }
  s.len = pos + 1;
  *slot = (int64_t)s.blocks[(size_t)(pos / bs)] * bs + pos % bs;
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                                       int64_t* slot_mapping, int64_t* copies,
                                       int32_t* num_copies, int32_t* num_done) {
  if (bm == nullptr || n < 0 || num_copies == nullptr || num_done == nullptr) return PA_ERR_INVALID;
  if (n > 0 && (seq_ids == nullptr || slot_mapping == nullptr || copies == nullptr))
    return PA_ERR_INVALID;
  *num_copies = 0;
  *num_done = 0;
  for (int32_t i = 0; i < n; ++i) slot_mapping[i] = -1;
  for (int32_t i = 0; i < n; ++i) {
    int64_t src, dst;
    const pa_status st = pa_bm_append_slot(bm, seq_ids[i], &slot_mapping[i], &src, &dst);
    if (st != PA_OK) {
      slot_mapping[i] = -1;
      return st;
    }
    if (src >= 0) {
      copies[2 * *num_copies] = src;
      copies[2 * *num_copies + 1] = dst;
      *num_copies += 1;
    }
    *num_done = i + 1;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (bm == nullptr || bm->seqs.count(child)) return PA_ERR_INVALID;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return PA_ERR_INVALID;
  try {
    pa_block_manager::Seq s = it->second;
    bm->seqs.reserve(bm->seqs.size() + 1);
    for (int32_t b : s.blocks) bm->refs[(size_t)b] += 1;
    bm->seqs.emplace(child, std::move(s));
  } catch (...) {  // host memory: the copy or the reserve failed before any count moved
    return PA_ERR_INVALID;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_bm_free(pa_block_manager* bm, int64_t seq_id) {
  if (bm == nullptr) return PA_ERR_INVALID;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID;
  for (int32_t b : it->second.blocks)
    if (--bm->refs[(size_t)b] == 0) bm->free_list.push_back(b);
  bm->seqs.erase(it);
  return PA_OK;
}

PA_EXPORT int64_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq_id) {
  if (bm == nullptr) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

PA_EXPORT int64_t pa_bm_seq_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out,
                                  int64_t cap) {
  if (bm == nullptr) return -1;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return -1;
  const std::vector<int32_t>& t = it->second.blocks;
  for (int64_t j = 0; j < (int64_t)t.size() && j < cap && out != nullptr; ++j) out[j] = t[(size_t)j];
  return (int64_t)t.size();
}

PA_EXPORT int64_t pa_bm_num_free(const pa_block_manager* bm) {
  return bm == nullptr ? -1 : (int64_t)bm->free_list.size();
}

PA_EXPORT int64_t pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int64_t cap) {
  if (bm == nullptr) return -1;
  for (int64_t j = 0; j < bm->free_list.size() && j < cap && out != nullptr; ++j)
    out[j] = bm->free_list.at(j);
  return bm->free_list.size();
}

PA_EXPORT int32_t pa_bm_refcount(const pa_block_manager* bm, int64_t block) {
  if (bm == nullptr || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refs[(size_t)block];
}

PA_EXPORT double pa_bm_usage(const pa_block_manager* bm) {
  if (bm == nullptr) return -1.0;
  return 1.0 - (double)bm->free_list.size() / (double)bm->num_blocks;
}

PA_EXPORT double pa_bm_slot_utilisation(const pa_block_manager* bm) {
  if (bm == nullptr) return -1.0;
  const int64_t used = bm->num_blocks - (int64_t)bm->free_list.size();
  if (used == 0) return 0.0;
  // tokens held by a block: the most any table that references it has written there
  std::unordered_map<int32_t, int64_t> filled;
  try {
    filled.reserve((size_t)used);
  } catch (...) {
    return -1.0;
  }
  const int64_t bs = bm->block_size;
  for (const auto& kv : bm->seqs) {
    const auto& s = kv.second;
    for (size_t j = 0; j < s.blocks.size(); ++j) {
      const int64_t n = s.len - (int64_t)j * bs;
      const int64_t f = n < bs ? n : bs;
      int64_t& cur = filled[s.blocks[j]];
      if (f > cur) cur = f;
    }
  }
  int64_t total = 0;
  for (const auto& kv : filled) total += kv.second;
  return (double)total / (double)(used * bs);
}

PA_EXPORT pa_status pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids,
                                       int32_t n, int32_t max_blocks, int32_t pad,
                                       int32_t* tables, int32_t* lens) {
  if (bm == nullptr || n < 0 || max_blocks < 0) return PA_ERR_INVALID;
  if (n > 0 && (seq_ids == nullptr || tables == nullptr || lens == nullptr)) return PA_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PA_ERR_INVALID;
    const auto& s = it->second;
    if ((int64_t)s.blocks.size() > max_blocks || s.len > INT32_MAX) return PA_ERR_INVALID;
    int32_t* row = tables + (int64_t)i * max_blocks;
    size_t j = 0;
    for (; j < s.blocks.size(); ++j) row[j] = s.blocks[j];
    for (; j < (size_t)max_blocks; ++j) row[j] = pad;
    lens[i] = (int32_t)s.len;
  }
  return PA_OK;
}
