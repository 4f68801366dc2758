// Random traces through the host block manager's C ABI (pa_bm_*), built together with
// block_manager.cpp under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_block_manager_sanitized.py. After every operation the manager's state is
// checked against what its own queries must satisfy:
//   - every sequence's table holds ceil(len / block_size) blocks;
//   - a block's reference count equals the number of table entries naming it;
//   - the free list holds exactly the blocks with no reference, each once;
//   - usage = 1 - free / num_blocks;
//   - an appended token's slot is table[pos / bs] * bs + pos % bs of the table after the
//     append, and a copy is reported exactly when the last block was shared;
//   - a refused operation (bad id, exhausted pool) leaves the state as it was.
// Exits 0 when every check held; a failed check prints it and exits 1, and a memory or
// UB error makes the sanitizers abort.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "../include/pagedkv.h"

namespace {

int failures = 0;

#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      std::fprintf(stderr, "check failed: %s: ", #cond); \
      std::fprintf(stderr, __VA_ARGS__);                  \
      std::fprintf(stderr, "\n");                         \
      ++failures;                                         \
      return;                                             \
    }                                                     \
  } while (0)

struct Snapshot {
  std::map<int64_t, std::vector<int32_t>> tables;
  std::map<int64_t, int64_t> lens;
  std::vector<int32_t> free_list;
  bool operator==(const Snapshot& o) const {
    return tables == o.tables && lens == o.lens && free_list == o.free_list;
  }
};

Snapshot snapshot(const pa_block_manager* bm, const std::vector<int64_t>& ids, int64_t nb) {
  Snapshot s;
  for (int64_t id : ids) {
    const int64_t n = pa_bm_seq_table(bm, id, nullptr, 0);
    std::vector<int32_t> t((size_t)(n > 0 ? n : 0));
    if (n > 0) pa_bm_seq_table(bm, id, t.data(), n);
    s.tables[id] = t;
    s.lens[id] = pa_bm_seq_len(bm, id);
  }
  const int64_t nf = pa_bm_free_list(bm, nullptr, 0);
  s.free_list.resize((size_t)(nf > 0 ? nf : 0));
  if (nf > 0) pa_bm_free_list(bm, s.free_list.data(), nf);
  (void)nb;
  return s;
}

void check_state(const pa_block_manager* bm, const std::vector<int64_t>& ids, int64_t nb,
                 int32_t bs) {
  const Snapshot s = snapshot(bm, ids, nb);
  std::vector<int32_t> refs((size_t)nb, 0);
  for (const auto& kv : s.tables) {
    const int64_t len = s.lens.at(kv.first);
    CHECK(len >= 0, "sequence %lld has no length", (long long)kv.first);
    CHECK((int64_t)kv.second.size() == (len + bs - 1) / bs, "sequence %lld: %zu blocks for %lld tokens",
          (long long)kv.first, kv.second.size(), (long long)len);
    for (int32_t b : kv.second) {
      CHECK(b >= 0 && b < nb, "block %d outside the pool", b);
      refs[(size_t)b] += 1;
    }
  }
  std::vector<int32_t> seen((size_t)nb, 0);
  for (int32_t b : s.free_list) {
    CHECK(b >= 0 && b < nb, "free block %d outside the pool", b);
    CHECK(seen[(size_t)b] == 0, "block %d twice in the free list", b);
    seen[(size_t)b] = 1;
  }
  int64_t free_count = 0;
  for (int64_t b = 0; b < nb; ++b) {
    CHECK(pa_bm_refcount(bm, b) == refs[(size_t)b], "block %lld: count %d, table entries %d",
          (long long)b, pa_bm_refcount(bm, b), refs[(size_t)b]);
    CHECK((refs[(size_t)b] == 0) == (seen[(size_t)b] == 1), "block %lld: free list and references disagree",
          (long long)b);
    free_count += refs[(size_t)b] == 0;
  }
  CHECK(pa_bm_num_free(bm) == free_count, "num_free %lld, expected %lld", (long long)pa_bm_num_free(bm),
        (long long)free_count);
  const double usage = pa_bm_usage(bm);
  CHECK(usage == 1.0 - (double)free_count / (double)nb, "usage %f", usage);
  const double util = pa_bm_slot_utilisation(bm);
  CHECK(util >= 0.0 && util <= 1.0, "slot utilisation %f", util);
}

void run_trace(uint64_t seed) {
  std::mt19937_64 rng(seed);
  auto pick = [&](int64_t lo, int64_t hi) {  // inclusive
    return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1));
  };
  const int64_t nb = pick(1, 48);
  static const int32_t kSizes[] = {1, 2, 4, 16};
  const int32_t bs = kSizes[pick(0, 3)];
  pa_block_manager* bm = nullptr;
  if (pa_bm_create(nb, bs, &bm) != PA_OK || bm == nullptr) {
    std::fprintf(stderr, "create failed\n");
    ++failures;
    return;
  }
  std::vector<int64_t> ids;  // live sequences
  int64_t next_id = 0;
  for (int step = 0; step < 600 && failures == 0; ++step) {
    const int op = (int)pick(0, 9);
    if (op <= 1) {  // allocate a new sequence
      const int64_t tokens = pick(0, 3 * bs);
      const Snapshot before = snapshot(bm, ids, nb);
      const pa_status st = pa_bm_allocate(bm, next_id, tokens);
      if (st == PA_OK) {
        ids.push_back(next_id);
      } else {
        CHECK(st == PA_ERR_EXHAUSTED, "allocate returned %d", (int)st);
        CHECK(snapshot(bm, ids, nb) == before, "a refused allocate changed the state");
      }
      ++next_id;
    } else if (op <= 5 && !ids.empty()) {  // append tokens to a few sequences at once
      const int32_t n = (int32_t)pick(1, 6);
      std::vector<int64_t> seqs((size_t)n), slots((size_t)n), copies((size_t)(2 * n));
      for (auto& x : seqs) x = ids[(size_t)pick(0, (int64_t)ids.size() - 1)];
      int32_t ncopies = -1, done = -1;
      const pa_status st =
          pa_bm_append_slots(bm, seqs.data(), n, slots.data(), copies.data(), &ncopies, &done);
      CHECK(st == PA_OK || st == PA_ERR_EXHAUSTED, "append_slots returned %d", (int)st);
      CHECK(done >= 0 && done <= n && (st != PA_OK || done == n), "done %d of %d", done, n);
      for (int32_t i = 0; i < done; ++i) CHECK(slots[(size_t)i] >= 0, "token %d has no slot", i);
      for (int32_t i = done; i < n; ++i) CHECK(slots[(size_t)i] == -1, "token %d past the refusal has a slot", i);
      for (int32_t c = 0; c < ncopies; ++c) {
        const int64_t src = copies[(size_t)(2 * c)], dst = copies[(size_t)(2 * c + 1)];
        CHECK(src >= 0 && src < nb && dst >= 0 && dst < nb && src != dst, "copy %lld -> %lld",
              (long long)src, (long long)dst);
      }
    } else if (op == 6 && !ids.empty()) {  // one append, checked slot by slot
      const int64_t id = ids[(size_t)pick(0, (int64_t)ids.size() - 1)];
      const int64_t pos = pa_bm_seq_len(bm, id);
      const int64_t nblk = pa_bm_seq_table(bm, id, nullptr, 0);
      std::vector<int32_t> t((size_t)nblk + 1);
      if (nblk > 0) pa_bm_seq_table(bm, id, t.data(), nblk);
      const bool shared_last = pos % bs != 0 && nblk > 0 && pa_bm_refcount(bm, t[(size_t)nblk - 1]) > 1;
      const Snapshot before = snapshot(bm, ids, nb);
      int64_t slot = -1, src = -1, dst = -1;
      const pa_status st = pa_bm_append_slot(bm, id, &slot, &src, &dst);
      if (st == PA_OK) {
        const int64_t n2 = pa_bm_seq_table(bm, id, t.data(), (int64_t)t.size());
        CHECK(pa_bm_seq_len(bm, id) == pos + 1, "length after append");
        CHECK(n2 == (pos + bs) / bs, "table after append");
        CHECK(slot == (int64_t)t[(size_t)(pos / bs)] * bs + pos % bs, "slot %lld", (long long)slot);
        CHECK((src >= 0) == shared_last, "copy reported %d, shared last block %d", src >= 0, shared_last);
        if (src >= 0) CHECK(dst == t[(size_t)(pos / bs)], "copy destination is not the new last block");
      } else {
        CHECK(st == PA_ERR_EXHAUSTED, "append returned %d", (int)st);
        CHECK(snapshot(bm, ids, nb) == before, "a refused append changed the state");
      }
    } else if (op == 7 && !ids.empty()) {  // fork
      const int64_t parent = ids[(size_t)pick(0, (int64_t)ids.size() - 1)];
      CHECK(pa_bm_fork(bm, parent, next_id) == PA_OK, "fork");
      CHECK(pa_bm_fork(bm, parent, next_id) == PA_ERR_INVALID, "fork onto a live id");
      ids.push_back(next_id++);
    } else if (op == 8 && !ids.empty()) {  // free
      const size_t k = (size_t)pick(0, (int64_t)ids.size() - 1);
      CHECK(pa_bm_free(bm, ids[k]) == PA_OK, "free");
      CHECK(pa_bm_free(bm, ids[k]) == PA_ERR_INVALID, "second free");
      ids.erase(ids.begin() + (long)k);
    } else {  // refused calls on unknown ids, and the padded tables of every sequence
      int64_t slot, src, dst;
      CHECK(pa_bm_append_slot(bm, next_id + 7, &slot, &src, &dst) == PA_ERR_INVALID, "append unknown");
      CHECK(pa_bm_seq_len(bm, next_id + 7) == -1, "length of unknown");
      if (!ids.empty()) CHECK(pa_bm_allocate(bm, ids[0], 1) == PA_ERR_INVALID, "allocate live id");
      const int32_t maxb = (int32_t)(3 * nb + 4);
      std::vector<int32_t> tables(ids.size() * (size_t)maxb + 1), lens(ids.size() + 1);
      const pa_status st = pa_bm_block_tables(bm, ids.data(), (int32_t)ids.size(), maxb, -9,
                                              tables.data(), lens.data());
      CHECK(st == PA_OK, "block_tables returned %d", (int)st);
      for (size_t i = 0; i < ids.size(); ++i) {
        const int64_t n = pa_bm_seq_table(bm, ids[i], nullptr, 0);
        CHECK(lens[i] == pa_bm_seq_len(bm, ids[i]), "padded table length");
        for (int64_t j = n; j < maxb; ++j) CHECK(tables[i * (size_t)maxb + (size_t)j] == -9, "padding");
      }
    }
    if (failures == 0) check_state(bm, ids, nb, bs);
  }
  while (!ids.empty() && failures == 0) {  // everything freed: every block is free again
    CHECK(pa_bm_free(bm, ids.back()) == PA_OK, "final free");
    ids.pop_back();
  }
  if (failures == 0) CHECK(pa_bm_num_free(bm) == nb, "blocks lost: %lld free of %lld",
                           (long long)pa_bm_num_free(bm), (long long)nb);
  pa_bm_destroy(bm);
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t first = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 0;
  const int count = argc > 2 ? std::atoi(argv[2]) : 50;
  for (int i = 0; i < count && failures == 0; ++i) run_trace(first + (uint64_t)i);
  if (failures) return 1;
  std::printf("%d traces ok\n", count);
  return 0;
}
