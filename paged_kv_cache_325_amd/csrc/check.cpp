// Host-side range check of one step's metadata (pkv_check_metadata in
// pkv.h).  The attention entry points do not read device arrays on the host,
// so out-of-range slots, block ids or lengths are undefined behaviour there;
// a caller that wants them caught copies the arrays to the host and calls
// this first.  Host code only.
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "pkv.h"
#include "pkv_error.h"

using pkv::fail;

extern "C" {

pkv_status pkv_check_metadata(const int32_t* slot_mapping, int32_t num_tokens,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, const int32_t* cu_seqlens_q,
                              int32_t batch, int32_t max_context_len, int32_t max_seqlen_q,
                              int32_t total_q, int32_t block_size, int64_t num_blocks) {
  if (num_tokens < 0 || batch < 0 || max_blocks_per_seq < 0 || max_context_len < 0 ||
      max_seqlen_q < 0 || num_blocks < 0)
    return fail(PKV_ERR_INVALID, "check_metadata: counts and sizes must be >= 0");
  if (block_size <= 0) return fail(PKV_ERR_INVALID, "check_metadata: block_size must be > 0");
  const int64_t num_slots = num_blocks * (int64_t)block_size;

  // slots: -1 (no store) or a slot of the pool, each used at most once
  if (slot_mapping && num_tokens > 0) {
    std::vector<int32_t> used;
    used.reserve((size_t)num_tokens);
    for (int32_t t = 0; t < num_tokens; ++t) {
      const int32_t s = slot_mapping[t];
      if (s == -1) continue;
      if (s < 0 || (int64_t)s >= num_slots)
        return fail(PKV_ERR_INVALID, "slot_mapping[%d] = %d outside [-1, %lld)", t, s,
                    (long long)num_slots);
      used.push_back(s);
    }
    std::sort(used.begin(), used.end());
    const auto dup = std::adjacent_find(used.begin(), used.end());
    if (dup != used.end())
      return fail(PKV_ERR_INVALID, "slot_mapping holds slot %d more than once", *dup);
  }

  // context lengths within the bound and the table width
  if (context_lens) {
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t n = context_lens[b];
      if (n < 0 || n > max_context_len)
        return fail(PKV_ERR_INVALID, "context_lens[%d] = %d outside [0, max_context_len = %d]",
                    b, n, max_context_len);
      if ((int64_t)n > cap)
        return fail(PKV_ERR_INVALID,
                    "context_lens[%d] = %d needs more than max_blocks_per_seq (%d) blocks", b, n,
                    max_blocks_per_seq);
    }
  }

  // every table column a context uses names a block of the pool
  if (block_tables && context_lens) {
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t used_cols = (int32_t)(((int64_t)context_lens[b] + block_size - 1) / block_size);
      const int32_t* row = block_tables + (int64_t)b * max_blocks_per_seq;
      for (int32_t j = 0; j < used_cols; ++j)
        if (row[j] < 0 || (int64_t)row[j] >= num_blocks)
          return fail(PKV_ERR_INVALID, "block_tables[%d][%d] = %d outside [0, %lld)", b, j, row[j],
                      (long long)num_blocks);
    }
  }

  // query offsets: non-decreasing from >= 0, no sequence above max_seqlen_q,
  // all rows inside q
  if (cu_seqlens_q && batch > 0) {
    if (cu_seqlens_q[0] < 0)
      return fail(PKV_ERR_INVALID, "cu_seqlens_q[0] = %d < 0", cu_seqlens_q[0]);
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t n = (int64_t)cu_seqlens_q[b + 1] - cu_seqlens_q[b];
      if (n < 0)
        return fail(PKV_ERR_INVALID, "cu_seqlens_q decreases at %d (%d -> %d)", b,
                    cu_seqlens_q[b], cu_seqlens_q[b + 1]);
      if (n > max_seqlen_q)
        return fail(PKV_ERR_INVALID, "sequence %d has %lld query rows > max_seqlen_q = %d", b,
                    (long long)n, max_seqlen_q);
    }
    if (total_q >= 0 && cu_seqlens_q[batch] > total_q)
      return fail(PKV_ERR_INVALID, "cu_seqlens_q[%d] = %d > total_q = %d", batch,
                  cu_seqlens_q[batch], total_q);
  }
  return PKV_OK;
}

}  // extern "C"
