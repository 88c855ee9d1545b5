/*
 * pkv.h -- C ABI of the paged KV-cache attention library (libpkv.so), gfx950.
 *
 * The library implements the per-layer hot path of a block-table KV cache as
 * the nano-vllm pages describe it:
 *   - nano-vllm source study (hk.pswp.cn), section 2 "注意力層": the attention
 *     layer first stores the fresh k/v rows into the cache at slot_mapping (a
 *     store kernel), then runs varlen attention with prefix cache in prefill
 *     and attention over the paged cache in decode;
 *   - nano-vllm architecture page (repothread.com), "Dynamische
 *     KV-Cache-Allokation" (cache indexed by block, row, kv head, head dim),
 *     "Prefill- und Decode-Vorbereitung" (slot = block id * block size + row;
 *     uncached positions run from the cached prefix length to the sequence
 *     length), "Kern-Designentscheidungen" item 1 (256-token blocks);
 *   - vLLM essay (lshu.cn), section 3.2: logical position -> (block index =
 *     pos / block size, row = pos % block size), then gather and compute.
 *
 * Conventions for every entry point
 * ---------------------------------
 * Pointers named "device" point to device memory (HBM) of the current HIP
 * device; host scalars are passed by value.  The caller owns every buffer;
 * the library never allocates, frees or synchronises.  Work is enqueued on
 * `stream` (a hipStream_t; NULL = the null stream) in stream order and runs
 * asynchronously; a PKV_OK return means the launch was enqueued.
 *
 * Element types: PKV_FP32 (float) or PKV_BF16 (bfloat16 bit patterns, uint16
 * storage).  Index arrays are int32.  Every value pointer must be 16-byte
 * aligned and every token stride must keep rows 16-byte aligned.
 *
 * KV cache layout of one layer (one tensor for K, one for V):
 *     cache[num_blocks][num_kv_heads][block_size][head_dim], dense, row-major;
 * element (p, g, o, d) is at ((p * num_kv_heads + g) * block_size + o) *
 * head_dim + d.  Physical slot s means block s / block_size, row
 * s % block_size.  This keeps the rows of one (block, kv head) contiguous.
 * head_dim must be 128.  block_size: 256 is the pages' size ("Kern-
 * Designentscheidungen" item 1) and the tuned one; also taken are 16 and 32
 * (vLLM's small pages) and every multiple of 64 up to 4096, which includes
 * all multiples of 256 (the size the architecture page's configuration
 * allows).  Outputs do not depend on the block size: the same logical K/V in
 * blocks of any supported size give bitwise the same results (when the
 * decode split plan is the same, see pkv_paged_decode_split_tokens).
 *
 * GQA: query head h reads kv head h / (num_q_heads / num_kv_heads); any
 * group size is served (decode workgroups take 1, 2, 4 or 8 query heads of a
 * group, the unused ones of a last, partial chunk masked; prefill work items
 * take 4, 2 or 1 heads, whichever divides the group).
 * Attention: out = sum_j softmax_j(scale * q . k_j) v_j over the visible keys,
 * fp32 accumulation, output in the input element type (bf16 rounded to
 * nearest even).  A query with no visible key gets a zero output row.
 *
 * Errors: host scalars and pointers are checked before any HIP call.
 *   PKV_ERR_INVALID      null pointer with a non-zero count, a count or size
 *                        < 0 (or <= 0 where a size must be positive),
 *                        num_q_heads % num_kv_heads != 0, misalignment,
 *                        max_context_len > max_blocks_per_seq * block_size,
 *                        causal != 1, a scale that is not finite (NaN, +-inf);
 *   PKV_ERR_UNSUPPORTED  a block_size outside {16, 32, 64 k <= 4096},
 *                        head_dim != 128, fp32 prefill;
 *   PKV_ERR_WORKSPACE    decode workspace smaller than required;
 *   PKV_ERR_HIP          a HIP launch reported an error.
 * A zero count (no tokens, empty batch) returns PKV_OK and launches nothing.
 * Device array *contents* are not checked: a slot outside [-1,
 * num_blocks * block_size), a block id outside [0, num_blocks) in a used
 * table column, context_lens[b] > max_context_len, or cu_seqlens_q that is not
 * non-decreasing are undefined behaviour.  pkv_last_error() describes the
 * most recent non-OK status of the calling thread.
 *
 * pkv_check_metadata() checks those contents on the host, for callers that
 * want such errors reported rather than undefined.
 *
 * Results are deterministic: a pure function of the inputs and the split
 * plan: every sum runs in a fixed order and none uses atomics (the prefill's
 * work queue does, to hand out work items, which changes no result).
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = 1,
  PKV_ERR_UNSUPPORTED = 2,
  PKV_ERR_WORKSPACE = 3,
  PKV_ERR_HIP = 4,
  PKV_ERR_NO_BLOCKS = 5 /* block manager: not enough free blocks (pkv_block_manager.h) */
} pkv_status;

typedef enum { PKV_FP32 = 0, PKV_BF16 = 1 } pkv_dtype;

/*
 * pkv_kv_store -- slot scatter of this step's K and V rows into the cache
 * (source study section 2, the store kernel; architecture page "Prefill- und
 * Decode-Vorbereitung" for the slots).
 *
 *   k, v            device, [num_tokens][num_kv_heads][head_dim]; token t's
 *                   row starts at t * k_token_stride (v_token_stride)
 *                   elements, heads are head_dim apart (so k and v may be
 *                   views into a fused qkv tensor)
 *   k_cache,v_cache device, cache layout above, num_blocks blocks; written
 *   slot_mapping    device int32 [num_tokens]; token t goes to slot
 *                   slot_mapping[t] for every kv head; -1 stores nothing
 *
 * Pure bitwise copy (no conversion); cells not addressed by a slot are left
 * unchanged.  Two tokens with the same slot are undefined behaviour.
 */
pkv_status pkv_kv_store(pkv_dtype dtype, const void* k, int64_t k_token_stride,
                        const void* v, int64_t v_token_stride, void* k_cache,
                        void* v_cache, const int32_t* slot_mapping,
                        int32_t num_tokens, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size,
                        int64_t num_blocks, void* stream);

/*
 * pkv_paged_decode_workspace_bytes -- bytes of workspace that
 * pkv_paged_decode needs for the split-K partials with the same
 * arguments (0 when the plan uses a single split).  num_splits: 0 =
 * automatic, else the number of splits of max_context_len requested.  Returns 0 for invalid or
 * unsupported arguments (pkv_paged_decode then reports the error).
 */
size_t pkv_paged_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_context_len,
                                        int32_t block_size, int32_t num_splits);

/*
 * pkv_paged_decode_split_tokens -- keys per split that pkv_paged_decode uses
 * with these arguments: a multiple of 64 up to 256, a multiple of 256 above,
 * never more than 64 blocks (62 when splits are not aligned to the blocks:
 * 16384 at block_size 256; so a requested split count is an upper bound
 * only up to that size); >= max_context_len means one split.  Returns 0 for
 * invalid or unsupported arguments.
 */
int32_t pkv_paged_decode_split_tokens(int32_t batch, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len,
                                      int32_t block_size, int32_t num_splits);

/*
 * pkv_paged_decode -- one query token per sequence attends its whole context
 * gathered through its block table (source study section 2, decode attention
 * with the KV cache; essay section 3.2, gather then compute).  Long contexts
 * are split into chunks of S keys (flash-decoding split-K); the partials are
 * merged in split order.
 *
 *   q              device, [batch][num_q_heads][head_dim]; sequence b's row
 *                  starts at b * q_token_stride elements, heads head_dim apart
 *   k_cache,v_cache device, cache layout above (read only)
 *   block_tables   device int32 [batch][max_blocks_per_seq]; column i of row
 *                  b is the physical block of logical block i; columns
 *                  >= ceil(context_lens[b] / block_size) are never read
 *   context_lens   device int32 [batch]; keys of sequence b, including the
 *                  token stored this step (the query sits at position
 *                  context_lens[b] - 1); 0 gives a zero output row
 *   max_context_len host; >= every context_lens[b]; sets the split plan
 *   scale          softmax scale (e.g. 1/sqrt(head_dim)); any finite value,
 *                  negative and zero included (zero gives the mean of the
 *                  visible V rows)
 *   num_splits     0 = automatic; otherwise the requested number of splits
 *   out            device, [batch][num_q_heads][head_dim], dense, dtype
 *   workspace      device, >= pkv_paged_decode_workspace_bytes(...) bytes,
 *                  16-byte aligned, may be NULL when that is 0; needs no
 *                  initialisation.  Calls sharing a workspace must not
 *                  overlap.  Layout: float acc[batch][num_q_heads][nsplit]
 *                  [head_dim], then float ml[batch][num_q_heads][nsplit][2],
 *                  nsplit = ceil(max_context_len / S).  For split s of a
 *                  sequence b with more than one split (keys s*S ..
 *                  min(n,(s+1)*S)-1, s*S < n), with x_j = scale*q.k_j:
 *                  ml = (m, l), m = max_j x_j*log2(e), l = sum_j
 *                  2^(x_j*log2(e) - m), and acc = sum_j 2^(x_j*log2(e) - m) v_j.
 *                  A second kernel merges them (acc summed in split order):
 *                  M = max_s m_s, out = sum_s 2^(m_s-M) acc_s /
 *                  sum_s 2^(m_s-M) l_s.  pkv_paged_decode = partials + merge.
 */
pkv_status pkv_paged_decode(pkv_dtype dtype, const void* q,
                            int64_t q_token_stride, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq,
                            const int32_t* context_lens,
                            int32_t max_context_len, int32_t batch,
                            int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, float scale, int32_t num_splits,
                            void* out, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * pkv_paged_decode_partials -- the first half of pkv_paged_decode (same
 * arguments, same checks): for every split of every sequence it leaves the
 * split-K partials (acc, m, l) in the workspace, and writes the output rows
 * of sequences that have a single split.  Exposed so each half can be timed
 * and checked on its own.
 *
 * pkv_paged_decode_merge -- the second half: writes the output rows of every
 * sequence with more than one split from the partials in `workspace`
 * (layout above), in split order.  Arguments mean what they mean for
 * pkv_paged_decode and must equal those of the partials call (they fix the
 * split plan).  Launches nothing when the plan has a single split.
 */
pkv_status pkv_paged_decode_partials(
    pkv_dtype dtype, const void* q, int64_t q_token_stride, const void* k_cache,
    const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, float scale, int32_t num_splits,
    void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_decode_step -- one decode step of one layer in one call: the
 * store of this step's K/V rows (one per sequence) fused into the paged
 * decode (source study section 2: the attention layer writes k, v into the
 * cache with the store kernel, then runs decode attention over the cache;
 * architecture page "Prefill- und Decode-Vorbereitung": in decode each
 * sequence appends one token whose slot is the last position of its last
 * block).  It leaves the caches and out exactly (bitwise) as
 * pkv_kv_store(k_new, v_new, slot_mapping, num_tokens = batch) followed by
 * pkv_paged_decode(...) with the same split plan, provided the decode-step
 * invariant holds for every row b:
 *   slot_mapping[b] == -1 (no store; padding rows also have
 *   context_lens[b] == 0), or slot_mapping[b] is the slot of position
 *   context_lens[b] - 1 of sequence b, in a block that no other sequence's
 *   context includes (the block manager never appends into a shared block).
 * If the invariant is broken the store still happens, but the decode may
 * read the slot before or after it is written.
 *
 *   k_new, v_new   device [batch][num_kv_heads][head_dim] (dtype), row b at
 *                  b * *_token_stride elements
 *   slot_mapping   device int32 [batch]
 *   k_cache, v_cache  written (the stored rows) and read
 *   everything else as for pkv_paged_decode (same workspace size).
 * The split kernel does the store, so with a single split the whole step is
 * one launch; capture in a HIP graph is safe (no allocation, no memset, no
 * synchronisation).  Errors: as pkv_kv_store and pkv_paged_decode.
 */
pkv_status pkv_paged_decode_step(
    pkv_dtype dtype, const void* q, int64_t q_token_stride, const void* k_new,
    int64_t k_new_token_stride, const void* v_new, int64_t v_new_token_stride,
    const int32_t* slot_mapping, void* k_cache, void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, float scale, int32_t num_splits,
    void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_decode_step_noalloc -- pkv_paged_decode_step for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, checks and
 * results (bitwise) as pkv_paged_decode_step with the same split plan, but no
 * workspace: the split-K partials go to a fixed scratch array of
 * PKV_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on each GPU it
 * runs on, from the first call on that GPU until the process ends.  The
 * caller still passes inputs and outputs.  Nothing is allocated, freed or
 * memset per call.
 *
 *   PKV_ERR_WORKSPACE  the plan's partials need more than
 *                      PKV_NOALLOC_SCRATCH_BYTES (compare
 *                      pkv_paged_decode_workspace_bytes beforehand; fewer
 *                      splits or a smaller batch fit); checked before any
 *                      HIP call
 *   PKV_ERR_HIP        the scratch's device address could not be found
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents: calls that may overlap on one GPU (different streams,
 * threads or processes' graphs replayed concurrently) race and must be
 * serialised by the caller.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)

pkv_status pkv_paged_decode_step_noalloc(
    pkv_dtype dtype, const void* q, int64_t q_token_stride, const void* k_new,
    int64_t k_new_token_stride, const void* v_new, int64_t v_new_token_stride,
    const int32_t* slot_mapping, void* k_cache, void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, float scale, int32_t num_splits,
    void* out, void* stream);

/*
 * Shared-prefix decode.  Sequences whose block tables begin with the same
 * physical blocks hold the same K/V there (architecture page, "Hash-basiertes
 * Prefix Caching" and "Kern-Designentscheidungen" item 2: full prompt blocks
 * with a cached chained hash are given the cached block, so sequences with a
 * common prompt prefix share them).  The decode can then attend each shared
 * split once for all of them: one MFMA tile per (shared split, kv head) whose
 * columns are the members' query heads, merged per sequence with its private
 * splits by the usual split-K merge.  The grouping is this library's own rule
 * (the pages describe none), built on the host from the host copies of the
 * tables by pkv_decode_prefix_plan:
 *   - only whole decode splits (S keys: pkv_paged_decode_split_tokens) that
 *     lie before every member's last position (ctx - 1) are shared;
 *   - sequences are classed by first block id, ordered by their table rows
 *     (lexicographically, over the blocks holding keys 0 .. ctx - 2), cut into
 *     runs of 16 / G members (G = num_q_heads / num_kv_heads; G > 8 shares
 *     nothing), and a run shares k = min(common entries * B, min ctx - 1) / S
 *     splits.
 *
 * pkv_decode_prefix_plan_words -- int32 words that always suffice for the
 * plan of `batch` sequences of at most max_context_len keys at split length
 * split_tokens; -1 for negative sizes or split_tokens <= 0.
 *
 * pkv_decode_prefix_plan -- builds the plan (host code, no HIP call).
 *   block_tables   HOST int32 [batch][max_blocks_per_seq] (the decode's
 *                  tables, a host copy)
 *   context_lens   HOST int32 [batch]; each <= max_blocks_per_seq * block_size
 *   split_tokens   S of the decode call the plan is for, a positive multiple of
 *                  64 (pkv_paged_decode_split_tokens with the same arguments)
 *   plan           HOST int32 [plan_words], written: the plan (layout: S,
 *                  items, batch, G, subgroups P; skip[batch]; P records of a
 *                  member count and 16 member ids (-1 unused); items x
 *                  (subgroup, split)); copy it to the device for the decode
 *   num_items      HOST out: items (shared splits; 0 = nothing is shared)
 *   words_written  HOST out (may be NULL): words of the plan
 * Errors: PKV_ERR_INVALID (bad sizes, null pointers, a context longer than its
 * table row), PKV_ERR_UNSUPPORTED (block size), PKV_ERR_WORKSPACE (plan_words
 * too small).
 *
 * pkv_paged_decode_prefix -- pkv_paged_decode with a plan: the same
 * arguments plus
 *   prefix_plan    device int32 words of pkv_decode_prefix_plan, built from
 *                  the same tables and context lengths (4-byte aligned)
 *   prefix_items   the num_items the planner returned; 0 = pkv_paged_decode
 *                  (bitwise)
 * and the same workspace size.  bf16 only when prefix_items > 0
 * (PKV_ERR_UNSUPPORTED otherwise).  Outputs match the oracle within the same
 * tolerance as pkv_paged_decode; they are not bitwise equal to it (the shared
 * splits run on MFMA with bf16 probabilities).  A plan whose header (S,
 * items, batch, G) does not match the call is ignored: the result is then
 * pkv_paged_decode's.  A plan built from other tables or context lengths
 * gives NaN output rows for the sequences whose shared split does not hold
 * in the tables passed (the kernel checks every member's table entries and
 * context length); other malformed plan contents are undefined behaviour.
 *
 * pkv_paged_decode_step_prefix -- pkv_paged_decode_step with a plan (same
 * extra arguments): the fused store plus the shared-prefix decode.  The
 * stored row (position ctx - 1) lies past every shared split.
 */
int64_t pkv_decode_prefix_plan_words(int32_t batch, int32_t max_context_len,
                                     int32_t split_tokens);

pkv_status pkv_decode_prefix_plan(const int32_t* block_tables,
                                  int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t batch,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t block_size, int32_t split_tokens,
                                  int32_t* plan, int64_t plan_words,
                                  int32_t* num_items, int64_t* words_written);

pkv_status pkv_paged_decode_prefix(
    pkv_dtype dtype, const void* q, int64_t q_token_stride, const void* k_cache,
    const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, float scale, int32_t num_splits,
    const int32_t* prefix_plan, int32_t prefix_items, void* out,
    void* workspace, size_t workspace_bytes, void* stream);

pkv_status pkv_paged_decode_step_prefix(
    pkv_dtype dtype, const void* q, int64_t q_token_stride, const void* k_new,
    int64_t k_new_token_stride, const void* v_new, int64_t v_new_token_stride,
    const int32_t* slot_mapping, void* k_cache, void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, float scale, int32_t num_splits,
    const int32_t* prefix_plan, int32_t prefix_items, void* out,
    void* workspace, size_t workspace_bytes, void* stream);

pkv_status pkv_paged_decode_merge(pkv_dtype dtype, const int32_t* context_lens,
                                  int32_t max_context_len, int32_t batch,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size,
                                  int32_t num_splits, void* out,
                                  const void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * pkv_paged_prefill_varlen -- varlen causal prefill whose keys come from the
 * cache through the block table, including prefix blocks cached (and shared)
 * before this step (source study section 2, varlen attention with prefix
 * cache; architecture page "Prefill- und Decode-Vorbereitung" and
 * "Hash-basiertes Prefix Caching").  bf16 only.
 *
 *   q              device, packed [total_q][num_q_heads][head_dim]; query row
 *                  r starts at r * q_token_stride elements
 *   cu_seqlens_q   device int32 [batch + 1]; sequence b owns query rows
 *                  cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (n_q of them)
 *   max_seqlen_q   host; >= every n_q
 *   context_lens   device int32 [batch]; n_k, keys of sequence b after this
 *                  step's store (cached prefix plus the n_q new tokens)
 *   max_context_len host; >= every n_k
 *   block_tables   as for decode
 *   scale          softmax scale, any finite value (as for decode)
 *   causal         must be 1: query i of sequence b sits at position
 *                  n_k - n_q + i and sees keys 0 .. n_k - n_q + i
 *   out            device, [total_q][num_q_heads][head_dim], dense, bf16
 *   workspace      device, >= pkv_paged_prefill_workspace_bytes() bytes,
 *                  4-byte aligned, caller-owned: the work-queue counters of
 *                  the persistent kernel.  It must be zero-filled before its
 *                  first use; every call leaves it zero again when its
 *                  kernel ends, so one fill at allocation suffices.  Calls
 *                  that may run concurrently need distinct workspaces.  A
 *                  workspace that was not zeroed gives wrong (possibly
 *                  unwritten) output rows but no access outside the
 *                  problem: work-item ids outside the item range are
 *                  treated as an exhausted queue.
 * total_q = cu_seqlens_q[batch] is not passed; rows outside the ranges are
 * neither read nor written.  PKV_ERR_WORKSPACE: workspace null, misaligned
 * or too small.
 */
pkv_status pkv_paged_prefill_varlen(
    pkv_dtype dtype, const void* q, int64_t q_token_stride,
    const void* k_cache, const void* v_cache, const int32_t* cu_seqlens_q,
    int32_t max_seqlen_q, const int32_t* context_lens, int32_t max_context_len,
    const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, float scale, int32_t causal,
    void* out, void* workspace, size_t workspace_bytes, void* stream);

/* pkv_paged_prefill_workspace_bytes -- workspace size that
 * pkv_paged_prefill_varlen needs (independent of the problem size). */
size_t pkv_paged_prefill_workspace_bytes(void);

/*
 * pkv_prefill_varlen -- varlen causal prefill over contiguous fresh k/v, no
 * cache (source study section 2: without a prefix-cache hit the attention
 * layer runs varlen attention directly on this step's q, k, v, with
 * cu_seqlens for queries and keys).  bf16 only.
 *
 *   q              device [total_q][num_q_heads][head_dim], row stride
 *                  q_token_stride elements (as for pkv_paged_prefill_varlen)
 *   k, v           device [total_k][num_kv_heads][head_dim], row strides
 *                  k_token_stride / v_token_stride elements (views of a fused
 *                  qkv buffer are allowed)
 *   cu_seqlens_q   device int32 [batch + 1]: sequence b's queries are rows
 *                  cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (n_q of them)
 *   cu_seqlens_k   device int32 [batch + 1]: its keys are rows
 *                  cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 (n_k of them)
 *   max_seqlen_q   host; >= every n_q
 *   causal         must be 1, bottom-right aligned: query i sees keys
 *                  0 .. n_k - n_q + i (a query that sees no key gets zeros)
 *   out, workspace as for pkv_paged_prefill_varlen.
 * The result is the same as pkv_paged_prefill_varlen over a cache holding
 * the same keys (same kernel; only the tile source differs).
 */
pkv_status pkv_prefill_varlen(
    pkv_dtype dtype, const void* q, int64_t q_token_stride, const void* k,
    int64_t k_token_stride, const void* v, int64_t v_token_stride,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    int32_t max_seqlen_q, int32_t batch, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, float scale, int32_t causal,
    void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_check_metadata -- host-side range check of one step's metadata, the
 * arrays the attention entry points take on the device and never check
 * (their out-of-range contents are undefined behaviour there; see Errors
 * above).  A caller that wants such mistakes reported copies the arrays to
 * the host and calls this before launching.  Every array pointer may be
 * null: its checks are then skipped.
 *
 *   slot_mapping   host int32 [num_tokens]: each -1 or a slot in
 *                  [0, num_blocks * block_size), no slot twice (the store's
 *                  contract; architecture page "Prefill- und
 *                  Decode-Vorbereitung": every stored token has its own slot)
 *   block_tables   host int32 [batch][max_blocks_per_seq]: the columns
 *                  context_lens[b] covers hold block ids in [0, num_blocks)
 *                  (checked only with context_lens)
 *   context_lens   host int32 [batch]: each in [0, max_context_len] and
 *                  within max_blocks_per_seq * block_size
 *   cu_seqlens_q   host int32 [batch + 1]: starts >= 0, non-decreasing, no
 *                  sequence with more than max_seqlen_q query rows, and
 *                  cu_seqlens_q[batch] <= total_q (the rows of q; -1: not
 *                  checked)
 * Returns PKV_OK, or PKV_ERR_INVALID with pkv_last_error() naming the first
 * bad entry (array, index, value) or a negative count / size.  Reads only
 * the given host arrays; no HIP call.
 */
pkv_status pkv_check_metadata(const int32_t* slot_mapping, int32_t num_tokens,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, const int32_t* cu_seqlens_q,
                              int32_t batch, int32_t max_context_len, int32_t max_seqlen_q,
                              int32_t total_q, int32_t block_size, int64_t num_blocks);

/*
 * pkv_kv_block_bytes -- bytes of one block of one of K or V for one layer
 * (block_size * num_kv_heads * head_dim * element size); the pages size the
 * cache as a whole number of such blocks ("Dynamische KV-Cache-Allokation").
 * Returns -1 for invalid arguments.
 */
int64_t pkv_kv_block_bytes(pkv_dtype dtype, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size);

/* pkv_last_error -- message for the calling thread's last non-OK status
 * ("" if none).  The string is owned by the library. */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
