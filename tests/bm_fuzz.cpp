// Host-only stress driver for the block manager (csrc/block_manager.cpp),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_block_manager_sanitized.py.  A seeded stream of calls --
// valid ones and deliberately invalid ones -- runs against the C ABI, and
// after every call the program checks, through the query entry points only:
//   * every block's count equals the number of tables holding it;
//   * the free list holds exactly the blocks with count 0, each once;
//   * a failing call changed nothing (state snapshot before and after);
//   * a decode step's metadata matches the tables and lengths.
// Exit status 0 when every check held.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <random>
#include <vector>

#include "pkv_block_manager.h"

// The library's last-error helper lives with the GPU entry points; this
// host-only build supplies its own.
namespace pkv {
pkv_status fail(pkv_status st, const char*, ...) { return st; }
const char* last_error() { return ""; }
}  // namespace pkv

namespace {

int g_failures = 0;
#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);         \
      if (++g_failures > 10) exit(1);                                         \
    }                                                                         \
  } while (0)

struct Snapshot {
  std::vector<int32_t> free_list;
  std::vector<int64_t> blocks;  // count, hash, ntok per block
  std::map<int64_t, std::vector<int32_t>> tables;
  std::map<int64_t, std::vector<int32_t>> seq_info;
  bool operator==(const Snapshot& o) const {
    return free_list == o.free_list && blocks == o.blocks && tables == o.tables &&
           seq_info == o.seq_info;
  }
};

Snapshot snapshot(pkv_block_manager* bm, int nb, const std::vector<int64_t>& ids) {
  Snapshot s;
  s.free_list.resize(pkv_bm_num_free_blocks(bm));
  CHECK(pkv_bm_free_blocks(bm, s.free_list.data(), (int32_t)s.free_list.size()) == PKV_OK);
  for (int b = 0; b < nb; ++b) {
    int32_t rc, nt;
    int64_t h;
    CHECK(pkv_bm_block(bm, b, &rc, &h, &nt) == PKV_OK);
    s.blocks.push_back(rc);
    s.blocks.push_back(h);
    s.blocks.push_back(nt);
  }
  for (int64_t id : ids) {
    int32_t n, c, t;
    CHECK(pkv_bm_sequence(bm, id, &n, &c, &t) == PKV_OK);
    s.seq_info[id] = {n, c, t};
    std::vector<int32_t> tab(t);
    CHECK(pkv_bm_block_table(bm, id, tab.data(), t) == PKV_OK);
    s.tables[id] = tab;
  }
  return s;
}

void check_invariants(const Snapshot& s, int nb) {
  std::vector<int> held(nb, 0), in_free(nb, 0);
  for (auto& kv : s.tables)
    for (int32_t b : kv.second) {
      CHECK(b >= 0 && b < nb);
      if (b >= 0 && b < nb) ++held[b];
    }
  for (int32_t b : s.free_list) {
    CHECK(b >= 0 && b < nb);
    if (b >= 0 && b < nb) ++in_free[b];
  }
  for (int b = 0; b < nb; ++b) {
    CHECK(s.blocks[3 * b] == held[b]);
    CHECK(in_free[b] == (held[b] == 0 ? 1 : 0));
  }
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? strtoull(argv[1], nullptr, 10) : 1;
  const int steps = argc > 2 ? atoi(argv[2]) : 20000;
  std::mt19937_64 rng(seed);
  auto uni = [&](int lo, int hi) { return (int)(lo + rng() % (uint64_t)(hi - lo + 1)); };
  const int B = std::vector<int>{2, 4, 16}[seed % 3];
  const int nb = uni(4, 24);
  pkv_block_manager* bm = nullptr;
  CHECK(pkv_bm_create(nb, B, &bm) == PKV_OK);
  std::vector<int64_t> live, placed;  // all sequences; those holding blocks
  int64_t next_id = 100;
  // a few shared prefixes so that sharing and reuse of freed blocks happen
  std::vector<std::vector<int32_t>> prefixes;
  for (int i = 0; i < 3; ++i) {
    std::vector<int32_t> p(B * uni(1, 2));
    for (auto& t : p) t = uni(0, 2);
    prefixes.push_back(p);
  }
  for (int step = 0; step < steps; ++step) {
    const int op = uni(0, 9);
    const Snapshot before = snapshot(bm, nb, live);
    pkv_status st = PKV_OK;
    bool expect_change = true;
    if (op <= 2 && live.size() < 12) {  // add a sequence
      std::vector<int32_t> toks = uni(0, 1) ? prefixes[uni(0, 2)] : std::vector<int32_t>{};
      const int extra = uni(1, 3 * B);
      for (int i = 0; i < extra; ++i) toks.push_back(uni(0, 2));
      st = pkv_bm_add_sequence(bm, next_id, toks.data(), (int32_t)toks.size());
      CHECK(st == PKV_OK);
      live.push_back(next_id++);
    } else if (op == 3 && !live.empty()) {  // allocate (may fail: held or no blocks)
      const int64_t id = live[uni(0, (int)live.size() - 1)];
      int32_t can = 0;
      CHECK(pkv_bm_can_allocate(bm, id, &can) == PKV_OK);
      st = pkv_bm_allocate(bm, id);
      const bool held = before.tables.at(id).size() > 0;
      if (held) CHECK(st == PKV_ERR_INVALID);
      else CHECK((st == PKV_OK) == (can == 1));
      if (st == PKV_OK) placed.push_back(id);
    } else if (op <= 6 && !placed.empty()) {  // one decode step for a placed sequence
      const int64_t id = placed[uni(0, (int)placed.size() - 1)];
      CHECK(pkv_bm_append_token(bm, id, uni(0, 2)) == PKV_OK);
      int32_t can = 0;
      CHECK(pkv_bm_can_append(bm, id, &can) == PKV_OK);
      const Snapshot mid = snapshot(bm, nb, live);
      st = pkv_bm_may_append(bm, id);
      CHECK((st == PKV_OK) == (can == 1));
      if (st != PKV_OK) {
        CHECK(st == PKV_ERR_NO_BLOCKS);
        CHECK(snapshot(bm, nb, live) == mid);
        // preempt it, as a scheduler would
        CHECK(pkv_bm_deallocate(bm, id) == PKV_OK);
        for (size_t i = 0; i < placed.size(); ++i)
          if (placed[i] == id) placed.erase(placed.begin() + i);
      } else {
        // metadata of a decode step over every placed, grown sequence
        const int n = (int)placed.size();
        int32_t width = 0;
        for (int64_t p : placed) width = std::max<int32_t>(width, (int32_t)snapshot(bm, nb, {p}).tables[p].size());
        std::vector<int32_t> slot(n), ctx(n), tab((size_t)n * width);
        int32_t mk = 0;
        st = pkv_bm_build_decode(bm, placed.data(), n, width, nullptr, nullptr, slot.data(),
                                 ctx.data(), tab.data(), &mk);
        // a sequence whose append is pending (only this one was grown) may
        // be a block short: then the builder refuses, changing nothing
        if (st == PKV_OK) {
          const Snapshot now = snapshot(bm, nb, live);
          for (int i = 0; i < n; ++i) {
            const auto& t = now.tables.at(placed[i]);
            const int32_t len = now.seq_info.at(placed[i])[0];
            CHECK(ctx[i] == len);
            CHECK(slot[i] == t.back() * B + (len - 1) % B);
            for (int j = 0; j < width; ++j)
              CHECK(tab[(size_t)i * width + j] == (j < (int)t.size() ? t[j] : -1));
          }
        } else {
          CHECK(st == PKV_ERR_INVALID);
        }
        expect_change = true;
      }
    } else if (op == 7 && !placed.empty()) {  // finish or preempt
      const size_t k = (size_t)uni(0, (int)placed.size() - 1);
      CHECK(pkv_bm_deallocate(bm, placed[k]) == PKV_OK);
      placed.erase(placed.begin() + k);
    } else if (op == 8 && !live.empty()) {  // remove a sequence (fails while placed)
      const size_t k = (size_t)uni(0, (int)live.size() - 1);
      const bool held = before.tables.at(live[k]).size() > 0;
      st = pkv_bm_remove_sequence(bm, live[k]);
      CHECK((st == PKV_OK) == !held);
      if (st == PKV_OK) live.erase(live.begin() + k);
    } else {  // invalid calls: must fail and change nothing
      expect_change = false;
      int32_t out = 0;
      CHECK(pkv_bm_allocate(bm, 999999) == PKV_ERR_INVALID);
      CHECK(pkv_bm_can_append(bm, 999999, &out) == PKV_ERR_INVALID);
      CHECK(pkv_bm_add_sequence(bm, 5, nullptr, 3) == PKV_ERR_INVALID);
      CHECK(pkv_bm_block(bm, nb, &out, nullptr, nullptr) == PKV_ERR_INVALID);
      int32_t tiny[1];
      if (pkv_bm_num_free_blocks(bm) > 1)
        CHECK(pkv_bm_free_blocks(bm, tiny, 1) == PKV_ERR_INVALID);
      if (!placed.empty()) {
        std::vector<int64_t> dup = {placed[0], placed[0]};
        std::vector<int32_t> s(2), c(2), t(2 * 64);
        CHECK(pkv_bm_decode_step(bm, dup.data(), 2, 64, nullptr, nullptr, s.data(), c.data(),
                                 t.data(), nullptr) == PKV_ERR_INVALID);
      }
    }
    const Snapshot after = snapshot(bm, nb, live);
    check_invariants(after, nb);
    if (!expect_change) CHECK(after == before);
  }
  pkv_bm_destroy(bm);
  printf("seed %llu: %d steps, block size %d, %d blocks, %d check failures\n",
         (unsigned long long)seed, steps, B, nb, g_failures);
  return g_failures ? 1 : 0;
}
