// C ABI of libpkv: argument checks, split planning and kernel launches.
// Every check on host scalars and pointers happens before the first HIP call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "pkv.h"
#include "pkv_error.h"
#include "pkv_internal.h"

namespace pkv {

namespace {
thread_local std::string g_last_error;
}  // namespace

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

const char* last_error() { return g_last_error.c_str(); }

}  // namespace pkv

namespace {

using pkv::fail;

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pkv_dtype dt) { return dt == PKV_BF16 ? 2 : dt == PKV_FP32 ? 4 : 0; }

// Checks shared by the three attention-side entry points.
pkv_status check_geometry(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size) {
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID, "num_q_heads (%d) and num_kv_heads (%d) must be positive",
                num_q_heads, num_kv_heads);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  if (head_dim <= 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID, "head_dim (%d) and block_size (%d) must be positive", head_dim,
                block_size);
  if (head_dim != pkv::kHeadDim)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d is not supported (only 128)", head_dim);
  if (!pkv::block_size_supported(block_size))
    return fail(PKV_ERR_UNSUPPORTED,
                "block_size %d is not supported (16, 32, or a multiple of 64 up to %d)",
                block_size, pkv::kMaxBlockSize);
  return PKV_OK;
}

pkv_status check_stride(const char* name, int64_t stride, int64_t min_elems, int eb) {
  if (stride < min_elems)
    return fail(PKV_ERR_INVALID, "%s (%lld) is smaller than a row (%lld elements)", name,
                (long long)stride, (long long)min_elems);
  if ((stride * eb) % 16 != 0)
    return fail(PKV_ERR_INVALID, "%s (%lld elements) does not keep rows 16-byte aligned", name,
                (long long)stride);
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return pkv::last_error(); }

int64_t pkv_kv_block_bytes(pkv_dtype dtype, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size) {
  const int eb = elem_bytes(dtype);
  if (eb == 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0) return -1;
  return (int64_t)block_size * num_kv_heads * head_dim * eb;
}

pkv_status pkv_kv_store(pkv_dtype dtype, const void* k, int64_t k_token_stride, const void* v,
                        int64_t v_token_stride, void* k_cache, void* v_cache,
                        const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int64_t num_blocks, void* stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PKV_ERR_INVALID, "unknown dtype %d", (int)dtype);
  if (num_tokens < 0) return fail(PKV_ERR_INVALID, "num_tokens (%d) < 0", num_tokens);
  if (num_blocks < 0) return fail(PKV_ERR_INVALID, "num_blocks (%lld) < 0", (long long)num_blocks);
  pkv_status st = check_geometry(num_kv_heads, num_kv_heads, head_dim, block_size);
  if (st != PKV_OK) return st;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID, "null pointer argument with num_tokens = %d", num_tokens);
  if (num_blocks == 0)
    return fail(PKV_ERR_INVALID, "num_blocks is 0 but %d tokens are to be stored", num_tokens);
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID, "k, v, k_cache and v_cache must be 16-byte aligned");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if ((st = check_stride("k_token_stride", k_token_stride, row, eb)) != PKV_OK) return st;
  if ((st = check_stride("v_token_stride", v_token_stride, row, eb)) != PKV_OK) return st;
  if (num_blocks * block_size > (int64_t)INT32_MAX + 1)
    return fail(PKV_ERR_UNSUPPORTED, "num_blocks * block_size exceeds the int32 slot range");
  return hip_status(pkv::launch_kv_store(eb, k, k_token_stride, v, v_token_stride, k_cache,
                                         v_cache, slot_mapping, num_tokens, num_kv_heads,
                                         block_size, (hipStream_t)stream),
                    "kv_store launch");
}

static bool decode_plan_for(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_context_len, int32_t block_size,
                            int32_t num_splits, pkv::DecodePlan* plan) {
  if (batch < 0 || max_context_len < 0 || num_splits < 0) return false;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return false;
  if (head_dim != pkv::kHeadDim || !pkv::block_size_supported(block_size)) return false;
  return pkv::plan_decode(batch, num_q_heads, num_kv_heads, max_context_len, num_splits,
                          block_size, plan);
}

size_t pkv_paged_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_context_len,
                                        int32_t block_size, int32_t num_splits) {
  pkv::DecodePlan plan;
  if (!decode_plan_for(batch, num_q_heads, num_kv_heads, head_dim, max_context_len, block_size,
                       num_splits, &plan))
    return 0;
  return plan.workspace_bytes;
}

int32_t pkv_paged_decode_split_tokens(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_context_len,
                                      int32_t block_size, int32_t num_splits) {
  pkv::DecodePlan plan;
  if (!decode_plan_for(batch, num_q_heads, num_kv_heads, head_dim, max_context_len, block_size,
                       num_splits, &plan))
    return 0;
  return plan.split_tokens;
}

}  // extern "C"

namespace {

enum DecodeParts { kSplitOnly = 1, kMergeOnly = 2, kSplitAndMerge = 3 };

// ---- fixed scratch of pkv_paged_decode_step_noalloc ------------------------
// For callers that cannot allocate device memory, the split-K partials of the
// no-allocation decode step live in this array, one copy per GPU, allocated
// with the library's code object and held until the process ends.  In host
// code `scratch` names a host-side stand-in, not the device array: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever handed to a kernel.  Every call on a
// GPU shares its copy, so calls that overlap on one GPU race.  The partials
// need no initialisation (each is written before the merge reads it).
static __device__ __align__(256) float scratch[PKV_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

pkv_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_UNSUPPORTED, "device %d: the fixed scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
      if (!p || ((uintptr_t)p & 255u) != 0)
        return fail(PKV_ERR_HIP, "the fixed scratch has no 256-byte aligned device address");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PKV_OK;
}

// This step's K/V rows for the fused store of pkv_paged_decode_step.
struct FusedStore {
  const void* k_new;
  int64_t k_stride;
  const void* v_new;
  int64_t v_stride;
  const int32_t* slot_mapping;
};

// A shared-prefix plan (device words from pkv_decode_prefix_plan).
struct PrefixArg {
  const int32_t* plan;
  int32_t items;
};

// Checks for the merge (and shared by the split) entry points.
pkv_status check_decode_common(pkv_dtype dtype, int32_t batch, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_context_len, int32_t num_splits,
                               const int32_t* context_lens, const void* out,
                               const void* workspace, size_t workspace_bytes,
                               pkv::DecodePlan* plan, bool use_scratch) {
  if (elem_bytes(dtype) == 0) return fail(PKV_ERR_INVALID, "unknown dtype %d", (int)dtype);
  if (batch < 0) return fail(PKV_ERR_INVALID, "batch (%d) < 0", batch);
  if (max_context_len < 0 || num_splits < 0)
    return fail(PKV_ERR_INVALID, "max_context_len and num_splits must be >= 0");
  pkv_status st = check_geometry(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != PKV_OK) return st;
  if (pkv::decode_heads_per_wg(num_q_heads / num_kv_heads) == 0)
    return fail(PKV_ERR_UNSUPPORTED, "GQA group size %d is not supported",
                num_q_heads / num_kv_heads);
  if (batch == 0) return PKV_OK;
  if (!context_lens || !out)
    return fail(PKV_ERR_INVALID, "null context_lens or out with batch = %d", batch);
  if (!aligned16(out)) return fail(PKV_ERR_INVALID, "out must be 16-byte aligned");
  if (!pkv::plan_decode(batch, num_q_heads, num_kv_heads, max_context_len, num_splits,
                        block_size, plan))
    return fail(PKV_ERR_UNSUPPORTED, "no decode plan for these arguments");
  if (use_scratch) {
    if (plan->workspace_bytes > (size_t)PKV_NOALLOC_SCRATCH_BYTES)
      return fail(PKV_ERR_WORKSPACE,
                  "this decode step needs %zu bytes of split-K partials, more than the %zu "
                  "bytes of the library's fixed scratch; use pkv_paged_decode_step with a "
                  "caller workspace (or fewer splits)",
                  plan->workspace_bytes, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
    return PKV_OK;
  }
  if (workspace_bytes < plan->workspace_bytes || (plan->workspace_bytes && !workspace))
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                workspace ? workspace_bytes : (size_t)0, plan->workspace_bytes);
  if (plan->workspace_bytes && !aligned16(workspace))
    return fail(PKV_ERR_INVALID, "workspace must be 16-byte aligned");
  return PKV_OK;
}

pkv_status decode_parts(int parts, pkv_dtype dtype, const void* q, int64_t q_token_stride,
                        const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t max_context_len, int32_t batch, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int64_t num_blocks, float scale, int32_t num_splits, void* out,
                        void* workspace, size_t workspace_bytes, void* stream,
                        const FusedStore* fs = nullptr, bool use_scratch = false,
                        const PrefixArg* pa = nullptr) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PKV_ERR_INVALID, "unknown dtype %d", (int)dtype);
  pkv_status st = check_geometry(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != PKV_OK) return st;
  if (parts & kSplitOnly) {
    if (max_blocks_per_seq < 0 || num_blocks < 0)
      return fail(PKV_ERR_INVALID, "max_blocks_per_seq and num_blocks must be >= 0");
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
      return fail(PKV_ERR_INVALID, "max_context_len (%d) > max_blocks_per_seq (%d) * block_size",
                  max_context_len, max_blocks_per_seq);
  }
  pkv::DecodePlan plan;
  st = check_decode_common(dtype, batch, num_q_heads, num_kv_heads, head_dim,
                                      block_size, max_context_len, num_splits, context_lens, out,
                                      workspace, workspace_bytes, &plan, use_scratch);
  if (st != PKV_OK || batch == 0) return st;
  if (parts & kSplitOnly) {
    if (!q) return fail(PKV_ERR_INVALID, "null q with batch = %d", batch);
    if (max_context_len > 0 && (!k_cache || !v_cache || !block_tables || num_blocks == 0))
      return fail(PKV_ERR_INVALID,
                  "null cache or block table (or no blocks) with max_context_len = %d",
                  max_context_len);
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
      return fail(PKV_ERR_INVALID, "q, k_cache and v_cache must be 16-byte aligned");
    if ((st = check_stride("q_token_stride", q_token_stride, (int64_t)num_q_heads * head_dim,
                           eb)) != PKV_OK)
      return st;
    if (!isfinite(scale)) return fail(PKV_ERR_INVALID, "scale must be finite (got %g)", (double)scale);
  }
  if (fs) {
    if (!fs->k_new || !fs->v_new || !fs->slot_mapping || !k_cache || !v_cache)
      return fail(PKV_ERR_INVALID, "null k_new, v_new, slot_mapping or cache with batch = %d",
                  batch);
    if (num_blocks == 0) return fail(PKV_ERR_INVALID, "num_blocks is 0 but rows are to be stored");
    if (!aligned16(fs->k_new) || !aligned16(fs->v_new))
      return fail(PKV_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if ((st = check_stride("k_new_token_stride", fs->k_stride, row, eb)) != PKV_OK) return st;
    if ((st = check_stride("v_new_token_stride", fs->v_stride, row, eb)) != PKV_OK) return st;
    if (num_blocks * block_size > (int64_t)INT32_MAX + 1)
      return fail(PKV_ERR_UNSUPPORTED, "num_blocks * block_size exceeds the int32 slot range");
  }
  if (pa && pa->items != 0) {
    if (pa->items < 0) return fail(PKV_ERR_INVALID, "prefix_items (%d) < 0", pa->items);
    if (dtype != PKV_BF16)
      return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode supports bf16 only");
    if (pkv::kPlanMembers / (num_q_heads / num_kv_heads) < 2)
      return fail(PKV_ERR_INVALID, "no shared-prefix plan has items for GQA group size %d",
                  num_q_heads / num_kv_heads);
    if (!pa->plan || ((uintptr_t)pa->plan & 3) != 0)
      return fail(PKV_ERR_INVALID, "prefix_plan must be a non-null, 4-byte aligned pointer");
    const int64_t grid = (int64_t)plan.nsplit * batch * num_kv_heads * plan.head_chunks +
                         (int64_t)pa->items * num_kv_heads;
    if (grid > INT32_MAX)
      return fail(PKV_ERR_UNSUPPORTED, "too many workgroups (%lld) for one launch", (long long)grid);
  }
  pkv::DecodeLaunch l;
  l.q = q;
  l.q_stride = q_token_stride;
  l.k_cache = k_cache;
  l.v_cache = v_cache;
  l.block_tables = block_tables;
  l.max_blocks = max_blocks_per_seq;
  l.context_lens = context_lens;
  l.batch = batch;
  l.num_q_heads = num_q_heads;
  l.num_kv_heads = num_kv_heads;
  l.block_size = block_size;
  l.scale = scale;
  l.out = out;
  l.workspace = plan.workspace_bytes ? (float*)workspace : nullptr;
  if (use_scratch && plan.workspace_bytes) {
    // every host argument has been checked: the first HIP call of this path
    void* ptr = nullptr;
    if ((st = scratch_for_current_device(&ptr)) != PKV_OK) return st;
    l.workspace = (float*)ptr;
  }
  if (pa && pa->items > 0 && (parts & kSplitOnly)) {
    l.prefix_plan = pa->plan;
    l.prefix_items = pa->items;
  }
  if (fs) {
    l.k_new = fs->k_new;
    l.k_new_stride = fs->k_stride;
    l.v_new = fs->v_new;
    l.v_new_stride = fs->v_stride;
    l.slot_mapping = fs->slot_mapping;
  }
  if (parts & kSplitOnly) {
    st = hip_status(pkv::launch_decode_split(eb, plan, l, (hipStream_t)stream),
                    "paged_decode split launch");
    if (st != PKV_OK) return st;
  }
  if (parts & kMergeOnly)
    st = hip_status(pkv::launch_decode_merge(eb, plan, l, (hipStream_t)stream),
                    "paged_decode merge launch");
  return st;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_decode(pkv_dtype dtype, const void* q, int64_t q_token_stride,
                            const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t max_context_len, int32_t batch,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int64_t num_blocks, float scale,
                            int32_t num_splits, void* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_parts(kSplitAndMerge, dtype, q, q_token_stride, k_cache, v_cache, block_tables,
                      max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, num_splits, out,
                      workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_decode_step(pkv_dtype dtype, const void* q, int64_t q_token_stride,
                                 const void* k_new, int64_t k_new_token_stride, const void* v_new,
                                 int64_t v_new_token_stride, const int32_t* slot_mapping,
                                 void* k_cache, void* v_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t max_context_len, int32_t batch, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int64_t num_blocks, float scale, int32_t num_splits, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  const FusedStore fs{k_new, k_new_token_stride, v_new, v_new_token_stride, slot_mapping};
  return decode_parts(kSplitAndMerge, dtype, q, q_token_stride, k_cache, v_cache, block_tables,
                      max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, num_splits, out,
                      workspace, workspace_bytes, stream, &fs);
}

pkv_status pkv_paged_decode_step_noalloc(pkv_dtype dtype, const void* q, int64_t q_token_stride,
                                         const void* k_new, int64_t k_new_token_stride,
                                         const void* v_new, int64_t v_new_token_stride,
                                         const int32_t* slot_mapping, void* k_cache,
                                         void* v_cache, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                                         int32_t max_context_len, int32_t batch,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size,
                                         int64_t num_blocks, float scale, int32_t num_splits,
                                         void* out, void* stream) {
  const FusedStore fs{k_new, k_new_token_stride, v_new, v_new_token_stride, slot_mapping};
  return decode_parts(kSplitAndMerge, dtype, q, q_token_stride, k_cache, v_cache, block_tables,
                      max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, num_splits, out,
                      nullptr, 0, stream, &fs, /*use_scratch=*/true);
}

int64_t pkv_decode_prefix_plan_words(int32_t batch, int32_t max_context_len,
                                     int32_t split_tokens) {
  if (batch < 0 || max_context_len < 0 || split_tokens <= 0) return -1;
  return pkv::prefix_plan_words_bound(batch, max_context_len, split_tokens);
}

pkv_status pkv_decode_prefix_plan(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t batch,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t block_size,
                                  int32_t split_tokens, int32_t* plan, int64_t plan_words,
                                  int32_t* num_items, int64_t* words_written) {
  if (batch < 0 || max_blocks_per_seq < 0)
    return fail(PKV_ERR_INVALID, "batch and max_blocks_per_seq must be >= 0");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  if (!pkv::block_size_supported(block_size))
    return fail(PKV_ERR_UNSUPPORTED,
                "block_size %d is not supported (16, 32, or a multiple of 64 up to %d)",
                block_size, pkv::kMaxBlockSize);
  if (split_tokens <= 0 || split_tokens % 64 != 0)
    return fail(PKV_ERR_INVALID, "split_tokens (%d) must be a positive multiple of 64",
                split_tokens);
  if (!plan || !num_items) return fail(PKV_ERR_INVALID, "null plan or num_items");
  if (batch > 0 && (!block_tables || !context_lens))
    return fail(PKV_ERR_INVALID, "null block_tables or context_lens with batch = %d", batch);
  for (int b = 0; b < batch; ++b)
    if ((int64_t)context_lens[b] > (int64_t)max_blocks_per_seq * block_size)
      return fail(PKV_ERR_INVALID,
                  "context_lens[%d] (%d) > max_blocks_per_seq (%d) * block_size", b,
                  context_lens[b], max_blocks_per_seq);
  int32_t items = 0;
  const int64_t words = pkv::build_prefix_plan(block_tables, max_blocks_per_seq, context_lens,
                                               batch, block_size, num_q_heads / num_kv_heads,
                                               split_tokens, plan, plan_words, &items);
  if (words < 0)
    return fail(PKV_ERR_WORKSPACE,
                "plan buffer of %lld words is too small (pkv_decode_prefix_plan_words gives a "
                "size that always suffices)",
                (long long)plan_words);
  *num_items = items;
  if (words_written) *words_written = words;
  return PKV_OK;
}

pkv_status pkv_paged_decode_prefix(pkv_dtype dtype, const void* q, int64_t q_token_stride,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t max_context_len,
                                   int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                   float scale, int32_t num_splits, const int32_t* prefix_plan,
                                   int32_t prefix_items, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const PrefixArg pa{prefix_plan, prefix_items};
  return decode_parts(kSplitAndMerge, dtype, q, q_token_stride, k_cache, v_cache, block_tables,
                      max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, num_splits, out,
                      workspace, workspace_bytes, stream, nullptr, false, &pa);
}

pkv_status pkv_paged_decode_step_prefix(
    pkv_dtype dtype, const void* q, int64_t q_token_stride, const void* k_new,
    int64_t k_new_token_stride, const void* v_new, int64_t v_new_token_stride,
    const int32_t* slot_mapping, void* k_cache, void* v_cache, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, float scale, int32_t num_splits,
    const int32_t* prefix_plan, int32_t prefix_items, void* out, void* workspace,
    size_t workspace_bytes, void* stream) {
  const FusedStore fs{k_new, k_new_token_stride, v_new, v_new_token_stride, slot_mapping};
  const PrefixArg pa{prefix_plan, prefix_items};
  return decode_parts(kSplitAndMerge, dtype, q, q_token_stride, k_cache, v_cache, block_tables,
                      max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, num_splits, out,
                      workspace, workspace_bytes, stream, &fs, false, &pa);
}

pkv_status pkv_paged_decode_partials(pkv_dtype dtype, const void* q, int64_t q_token_stride,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t max_context_len,
                                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                     float scale, int32_t num_splits, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return decode_parts(kSplitOnly, dtype, q, q_token_stride, k_cache, v_cache, block_tables,
                      max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, num_splits, out,
                      workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_decode_merge(pkv_dtype dtype, const int32_t* context_lens,
                                  int32_t max_context_len, int32_t batch, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_splits, void* out, const void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_parts(kMergeOnly, dtype, nullptr, 0, nullptr, nullptr, nullptr, 0, context_lens,
                      max_context_len, batch, num_q_heads, num_kv_heads, head_dim, block_size, 0,
                      1.0f, num_splits, out, const_cast<void*>(workspace), workspace_bytes,
                      stream);
}

pkv_status pkv_paged_prefill_varlen(pkv_dtype dtype, const void* q, int64_t q_token_stride,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* cu_seqlens_q, int32_t max_seqlen_q,
                                    const int32_t* context_lens, int32_t max_context_len,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                    float scale, int32_t causal, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PKV_ERR_INVALID, "unknown dtype %d", (int)dtype);
  if (batch < 0 || max_seqlen_q < 0 || max_context_len < 0 || max_blocks_per_seq < 0 ||
      num_blocks < 0)
    return fail(PKV_ERR_INVALID,
                "batch, max_seqlen_q, max_context_len, max_blocks_per_seq and num_blocks must be "
                ">= 0");
  if (causal != 1) return fail(PKV_ERR_INVALID, "causal must be 1 (got %d)", causal);
  pkv_status st = check_geometry(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != PKV_OK) return st;
  if (dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "paged_prefill_varlen supports bf16 only");
  if (!pkv::prefill_supported_group(num_q_heads / num_kv_heads))
    return fail(PKV_ERR_UNSUPPORTED, "GQA group size %d is not supported",
                num_q_heads / num_kv_heads);
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID, "max_context_len (%d) > max_blocks_per_seq (%d) * block_size",
                max_context_len, max_blocks_per_seq);
  if (batch == 0 || max_seqlen_q == 0) return PKV_OK;
  if (!q || !cu_seqlens_q || !context_lens || !out)
    return fail(PKV_ERR_INVALID, "null q, cu_seqlens_q, context_lens or out");
  if (max_context_len > 0 && (!k_cache || !v_cache || !block_tables || num_blocks == 0))
    return fail(PKV_ERR_INVALID, "null cache or block table (or no blocks) with max_context_len = %d",
                max_context_len);
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID, "q, out, k_cache and v_cache must be 16-byte aligned");
  if ((st = check_stride("q_token_stride", q_token_stride, (int64_t)num_q_heads * head_dim, eb)) !=
      PKV_OK)
    return st;
  if (!isfinite(scale)) return fail(PKV_ERR_INVALID, "scale must be finite (got %g)", (double)scale);
  if (!workspace || ((uintptr_t)workspace & 3) != 0 ||
      workspace_bytes < pkv::prefill_workspace_bytes())
    return fail(PKV_ERR_WORKSPACE, "prefill workspace must be non-null, 4-byte aligned and >= %zu bytes",
                pkv::prefill_workspace_bytes());
  pkv::PrefillLaunch l;
  l.q = q;
  l.q_stride = q_token_stride;
  l.k_cache = k_cache;
  l.v_cache = v_cache;
  l.cu_seqlens_q = cu_seqlens_q;
  l.max_seqlen_q = max_seqlen_q;
  l.context_lens = context_lens;
  l.block_tables = block_tables;
  l.max_blocks = max_blocks_per_seq;
  l.batch = batch;
  l.num_q_heads = num_q_heads;
  l.num_kv_heads = num_kv_heads;
  l.block_size = block_size;
  l.scale = scale;
  l.out = out;
  l.workspace = workspace;
  return hip_status(pkv::launch_prefill(l, (hipStream_t)stream), "paged_prefill_varlen launch");
}

size_t pkv_paged_prefill_workspace_bytes(void) { return pkv::prefill_workspace_bytes(); }

pkv_status pkv_prefill_varlen(pkv_dtype dtype, const void* q, int64_t q_token_stride, const void* k,
                              int64_t k_token_stride, const void* v, int64_t v_token_stride,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t max_seqlen_q, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, float scale, int32_t causal,
                              void* out, void* workspace, size_t workspace_bytes, void* stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PKV_ERR_INVALID, "unknown dtype %d", (int)dtype);
  if (batch < 0 || max_seqlen_q < 0)
    return fail(PKV_ERR_INVALID, "batch and max_seqlen_q must be >= 0");
  if (causal != 1) return fail(PKV_ERR_INVALID, "causal must be 1 (got %d)", causal);
  pkv_status st = check_geometry(num_q_heads, num_kv_heads, head_dim, pkv::kBlockSize);
  if (st != PKV_OK) return st;
  if (dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "prefill_varlen supports bf16 only");
  if (!pkv::prefill_supported_group(num_q_heads / num_kv_heads))
    return fail(PKV_ERR_UNSUPPORTED, "GQA group size %d is not supported",
                num_q_heads / num_kv_heads);
  if (batch == 0 || max_seqlen_q == 0) return PKV_OK;
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k || !out)
    return fail(PKV_ERR_INVALID, "null q, k, v, cu_seqlens_q, cu_seqlens_k or out");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(PKV_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
  if ((st = check_stride("q_token_stride", q_token_stride, (int64_t)num_q_heads * head_dim, eb)) !=
      PKV_OK)
    return st;
  const int64_t kv_row = (int64_t)num_kv_heads * head_dim;
  if ((st = check_stride("k_token_stride", k_token_stride, kv_row, eb)) != PKV_OK) return st;
  if ((st = check_stride("v_token_stride", v_token_stride, kv_row, eb)) != PKV_OK) return st;
  // 64 key rows must stay inside one 32-bit buffer range
  if (k_token_stride * eb * 64 > INT32_MAX || v_token_stride * eb * 64 > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "k/v token stride too large");
  if (!isfinite(scale)) return fail(PKV_ERR_INVALID, "scale must be finite (got %g)", (double)scale);
  if (!workspace || ((uintptr_t)workspace & 3) != 0 ||
      workspace_bytes < pkv::prefill_workspace_bytes())
    return fail(PKV_ERR_WORKSPACE, "prefill workspace must be non-null, 4-byte aligned and >= %zu bytes",
                pkv::prefill_workspace_bytes());
  pkv::PrefillLaunch l;
  l.q = q;
  l.q_stride = q_token_stride;
  l.k_cache = nullptr;
  l.v_cache = nullptr;
  l.cu_seqlens_q = cu_seqlens_q;
  l.max_seqlen_q = max_seqlen_q;
  // not read when the keys come from cu_seqlens_k, but a valid array all the
  // same (batch + 1 entries), so that no load through it could fault
  l.context_lens = cu_seqlens_k;
  l.block_tables = nullptr;
  l.max_blocks = 0;
  l.batch = batch;
  l.num_q_heads = num_q_heads;
  l.num_kv_heads = num_kv_heads;
  l.scale = scale;
  l.out = out;
  l.workspace = workspace;
  l.cu_seqlens_k = cu_seqlens_k;
  l.k_rows = k;
  l.v_rows = v;
  l.k_row_stride = k_token_stride;
  l.v_row_stride = v_token_stride;
  return hip_status(pkv::launch_prefill(l, (hipStream_t)stream), "prefill_varlen launch");
}

}  // extern "C"
