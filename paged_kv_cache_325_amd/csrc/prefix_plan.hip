// Host planner of the shared-prefix decode: which sequences of a decode batch
// hold their leading splits in the same physical blocks, so that the decode
// kernel attends each such split once for all of them.
//
// Why equal block ids mean equal K/V: nano-vllm architecture page,
// "Hash-basiertes Prefix Caching" and "Kern-Designentscheidungen" item 2 --
// a full block of prompt tokens whose chained hash is already cached is
// given the cached block's id, so sequences with a common prompt prefix
// share those physical blocks.  The grouping rule below is this library's
// own (the pages describe no such plan):
//   1. only whole decode splits (S keys, split s = keys sS .. (s+1)S - 1) are
//      shared, and only before a sequence's last position (ctx - 1, the row
//      a decode step stores): a sequence is eligible if ctx - 1 >= S;
//   2. eligible sequences are classed by their first block id (classes in
//      order of their first member);
//   3. a class is ordered by its members' table rows over the blocks holding
//      keys 0 .. ctx - 2, lexicographically (a prefix first), ties by batch
//      index;
//   4. the order is cut into runs of 16 / G members (their query heads of
//      one kv head fill one 16-column MFMA tile); runs of one are dropped;
//   5. a run shares k = min(lcp * B, min(ctx) - 1) / S splits, lcp being the
//      number of leading table entries common to all its members (k = 0:
//      dropped).
#include <algorithm>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace pkv {

int64_t prefix_plan_words_bound(int batch, int max_context_len, int split_tokens) {
  if (batch < 0 || split_tokens <= 0) return -1;
  const int64_t groups = batch / 2;
  const int64_t splits = std::max(max_context_len - 1, 0) / split_tokens;
  return kPlanHeader + batch + kPlanGroupWords * groups + 2 * groups * splits;
}

int64_t build_prefix_plan(const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                          int batch, int block_size, int group, int split_tokens, int32_t* plan,
                          int64_t capacity, int32_t* items_out) {
  const int run_len = kPlanMembers / group;
  std::vector<int32_t> skip(batch, 0);
  std::vector<std::vector<int>> subgroups;
  std::vector<int32_t> items;  // (subgroup, split) pairs
  // entries of the blocks that hold keys 0 .. ctx - 2
  auto used = [&](int b) -> int {
    const int n = context_lens[b];
    return n > 1 ? (n - 2) / block_size + 1 : 0;
  };
  auto row = [&](int b) { return block_tables + (int64_t)b * max_blocks; };

  if (run_len >= 2) {
    std::unordered_map<int32_t, int> class_of;
    std::vector<std::vector<int>> classes;
    for (int b = 0; b < batch; ++b) {
      if ((int64_t)context_lens[b] - 1 < split_tokens) continue;
      const int32_t first = row(b)[0];
      auto f = class_of.find(first);
      if (f == class_of.end()) {
        class_of.emplace(first, (int)classes.size());
        classes.push_back({b});
      } else {
        classes[f->second].push_back(b);
      }
    }
    for (std::vector<int>& m : classes) {
      if (m.size() < 2) continue;
      std::sort(m.begin(), m.end(), [&](int x, int y) {
        const int32_t *rx = row(x), *ry = row(y);
        const int ux = used(x), uy = used(y);
        if (std::lexicographical_compare(rx, rx + ux, ry, ry + uy)) return true;
        if (std::lexicographical_compare(ry, ry + uy, rx, rx + ux)) return false;
        return x < y;
      });
      for (size_t i = 0; i < m.size(); i += run_len) {
        const size_t e = std::min(m.size(), i + (size_t)run_len);
        if (e - i < 2) continue;
        int lcp = used(m[i]);
        int64_t last = (int64_t)context_lens[m[i]] - 1;
        for (size_t t = i + 1; t < e; ++t) {
          lcp = std::min(lcp, used(m[t]));
          last = std::min(last, (int64_t)context_lens[m[t]] - 1);
        }
        for (int c = 0; c < lcp; ++c) {
          bool same = true;
          for (size_t t = i + 1; t < e && same; ++t) same = row(m[t])[c] == row(m[i])[c];
          if (!same) {
            lcp = c;
            break;
          }
        }
        const int64_t shared = std::min((int64_t)lcp * block_size, last);
        const int64_t k = shared / split_tokens;
        if (k < 1) continue;
        const int p = (int)subgroups.size();
        subgroups.emplace_back(m.begin() + i, m.begin() + e);
        for (size_t t = i; t < e; ++t) skip[m[t]] = (int32_t)k;
        for (int64_t s = 0; s < k; ++s) {
          items.push_back(p);
          items.push_back((int32_t)s);
        }
      }
    }
  }
  const int64_t n_items = (int64_t)items.size() / 2;
  const int64_t words =
      kPlanHeader + batch + (int64_t)kPlanGroupWords * subgroups.size() + 2 * n_items;
  if (words > capacity) return -1;
  int32_t* w = plan;
  *w++ = split_tokens;
  *w++ = (int32_t)n_items;
  *w++ = batch;
  *w++ = group;
  *w++ = (int32_t)subgroups.size();
  for (int b = 0; b < batch; ++b) *w++ = skip[b];
  for (const std::vector<int>& sgm : subgroups) {
    *w++ = (int32_t)sgm.size();
    for (int t = 0; t < kPlanMembers; ++t) *w++ = t < (int)sgm.size() ? sgm[t] : -1;
  }
  for (int32_t v : items) *w++ = v;
  *items_out = (int32_t)n_items;
  return words;
}

}  // namespace pkv
