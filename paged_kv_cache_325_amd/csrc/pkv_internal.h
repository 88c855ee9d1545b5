// Host-side interface between the C ABI (api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kHeadDim = 128;      // head_dim supported by the kernels
constexpr int kBlockSize = 256;    // the pages' tokens per KV block
constexpr int kMaxBlockSize = 4096;

// Block sizes the kernels take: 16 and 32 (a 64-token tile spans several
// blocks; each 16-row quarter lies in one) and every multiple of 64 up to
// kMaxBlockSize (a 64-token tile lies in one block), which includes all
// multiples of 256.
inline bool block_size_supported(int b) {
  return b == 16 || b == 32 || (b > 0 && b % 64 == 0 && b <= kMaxBlockSize);
}

// Division of n in [0, 2^32) by a divisor fixed at launch, by multiplication
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994, the unsigned round-up method): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0), t = mulhi(m, n).
struct FastDiv {
  uint32_t d = 1, m = 1, s1 = 0, s2 = 0;
  FastDiv() = default;
  explicit FastDiv(uint32_t div) : d(div) {
    uint32_t l = 0;
    while (l < 32 && (1ull << l) < div) ++l;
    m = (uint32_t)(((1ull << 32) * ((1ull << l) - div)) / div + 1);
    s1 = l < 1 ? l : 1;
    s2 = l > 1 ? l - 1 : 0;
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
    const uint32_t t = (uint32_t)(((uint64_t)m * n) >> 32);
    return (t + ((n - t) >> s1)) >> s2;
  }
};

// ---- slot scatter -------------------------------------------------------
hipError_t launch_kv_store(int elem_bytes, const void* k, int64_t k_stride, const void* v,
                           int64_t v_stride, void* k_cache, void* v_cache, const int32_t* slots,
                           int num_tokens, int num_kv_heads, int block_size,
                           hipStream_t stream);

// ---- paged decode -------------------------------------------------------
// Query heads of one GQA group handled by one decode workgroup.
int decode_heads_per_wg(int group);

struct DecodePlan {
  int group;         // Hq / Hkv
  int heads_per_wg;  // 1, 2, 4 or 8
  int head_chunks;   // ceil(group / heads_per_wg)
  int split_tokens;  // keys per split, multiple of 64
  int nsplit;        // ceil(max_context_len / split_tokens), >= 1
  size_t workspace_bytes;
};

// Returns false if the group size is not supported.
bool plan_decode(int batch, int num_q_heads, int num_kv_heads, int max_context_len,
                 int num_splits, int block_size, DecodePlan* plan);

struct DecodeLaunch {
  const void* q;
  int64_t q_stride;  // elements between sequences' query rows
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* context_lens;
  int32_t batch, num_q_heads, num_kv_heads;
  int32_t block_size = kBlockSize;  // block_size_supported()
  float scale;
  void* out;
  float* workspace;
  // fused store of this step's rows (decode step); k_new == nullptr: none
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  int64_t k_new_stride = 0, v_new_stride = 0;  // elements between sequences
  const int32_t* slot_mapping = nullptr;
  // shared-prefix plan (device words, see below); nullptr: none
  const int32_t* prefix_plan = nullptr;
  int32_t prefix_items = 0;
};

// ---- shared-prefix decode plan ---------------------------------------------
// Sequences whose block tables begin with the same physical blocks hold the
// same K/V there; the plan names runs of such sequences ("subgroups") and the
// leading splits they share, so that each shared split is attended once for
// all members of its subgroup (one MFMA tile: up to 16 query columns, the
// members' query heads of one kv head) and merged per sequence with its
// private splits.  Device words (int32):
//   [0] split length S the plan was built for, [1] items, [2] batch,
//   [3] GQA group size G, [4] subgroups P;
//   skip[batch]: leading splits of sequence b computed by its subgroup;
//   P records of kPlanGroupWords: member count, kPlanMembers member ids;
//   items x 2: subgroup, split.
constexpr int kPlanHeader = 5;
constexpr int kPlanMembers = 16;
constexpr int kPlanGroupWords = 1 + kPlanMembers;

int64_t prefix_plan_words_bound(int batch, int max_context_len, int split_tokens);
// Builds the plan on the host; returns the number of words written, or -1
// if `capacity` is too small.  *items receives the number of items.
int64_t build_prefix_plan(const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                          int batch, int block_size, int group, int split_tokens, int32_t* plan,
                          int64_t capacity, int32_t* items);

// The split kernel (partials, and outputs of single-split sequences) and the
// merge kernel (outputs of split sequences).  Only q, caches, tables and
// scale are used by the split launch; the merge uses context_lens, batch,
// head counts, out and workspace.
hipError_t launch_decode_split(int elem_bytes, const DecodePlan& plan, const DecodeLaunch& a,
                               hipStream_t stream);
hipError_t launch_decode_merge(int elem_bytes, const DecodePlan& plan, const DecodeLaunch& a,
                               hipStream_t stream);

// ---- varlen causal prefill ----------------------------------------------
bool prefill_supported_group(int group);

struct PrefillLaunch {
  const void* q;
  int64_t q_stride;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_seqlens_q;
  int32_t max_seqlen_q;
  const int32_t* context_lens;
  const int32_t* block_tables;
  int32_t max_blocks;
  int32_t batch, num_q_heads, num_kv_heads;
  int32_t block_size = kBlockSize;  // block_size_supported()
  float scale;
  void* out;
  void* workspace;  // prefill_workspace_bytes(), zero on entry, zero on exit
  // contiguous keys (no cache): cu_seqlens_k != nullptr
  const int32_t* cu_seqlens_k = nullptr;
  const void* k_rows = nullptr;
  const void* v_rows = nullptr;
  int64_t k_row_stride = 0, v_row_stride = 0;  // elements
};

size_t prefill_workspace_bytes();
hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream);

}  // namespace pkv
