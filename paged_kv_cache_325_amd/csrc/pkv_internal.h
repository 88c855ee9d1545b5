// Host-side interface between the C ABI (api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kHeadDim = 128;    // head_dim supported by the kernels
constexpr int kBlockSize = 256;  // tokens per KV block

// ---- slot scatter -------------------------------------------------------
hipError_t launch_kv_store(int elem_bytes, const void* k, int64_t k_stride, const void* v,
                           int64_t v_stride, void* k_cache, void* v_cache, const int32_t* slots,
                           int num_tokens, int num_kv_heads, hipStream_t stream);

// ---- paged decode -------------------------------------------------------
// Query heads of one GQA group handled by one decode workgroup.
int decode_heads_per_wg(int group);

struct DecodePlan {
  int group;         // Hq / Hkv
  int heads_per_wg;  // 1, 2, 4 or 8
  int head_chunks;   // group / heads_per_wg
  int split_tokens;  // keys per split, multiple of 64
  int nsplit;        // ceil(max_context_len / split_tokens), >= 1
  size_t workspace_bytes;
};

// Returns false if the group size is not supported.
bool plan_decode(int batch, int num_q_heads, int num_kv_heads, int max_context_len,
                 int num_splits, DecodePlan* plan);

struct DecodeLaunch {
  const void* q;
  int64_t q_stride;  // elements between sequences' query rows
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* context_lens;
  int32_t batch, num_q_heads, num_kv_heads;
  float scale;
  void* out;
  float* workspace;
  // fused store of this step's rows (decode step); k_new == nullptr: none
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  int64_t k_new_stride = 0, v_new_stride = 0;  // elements between sequences
  const int32_t* slot_mapping = nullptr;
};

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
