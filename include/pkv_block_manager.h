/*
 * pkv_block_manager.h -- C ABI of the host block manager in libpkv.so: the
 * allocation, prefix sharing and growth of the paged KV cache's blocks, and
 * the per-step metadata (slots, block tables, lengths) that the attention
 * entry points of pkv.h consume.
 *
 * What it computes follows the nano-vllm architecture page (repothread.com):
 *   "Block-Struktur und Referenzzählung"  a block has an id, a reference
 *       count, a hash (-1: none) and the token ids it holds; it returns to
 *       the free list only when its count reaches 0;
 *   "Hash-basiertes Prefix Caching"  allocation walks the sequence's blocks;
 *       a full block's hash is chained on the previous block's hash; a hit
 *       whose recorded tokens equal the block's tokens shares the block,
 *       anything else takes the first free block;
 *   "Dynamische Block-Erweiterung"  decode growth by len % block_size: 1 ->
 *       append a new block, 0 -> hash and register the block that just
 *       filled, otherwise nothing;
 *   "Block-Berechnung und Token-Appending", "Prefill- und
 *       Decode-Vorbereitung"  block counts, last-block fill, and the
 *       uncached positions / slots of a prefill step;
 *   "Prefill-Scheduling", "Decode-Scheduling mit Preemption",
 *       "Postprocessing und Abschluss-Erkennung"  admission and decode gates
 *       (can_allocate, can_append) and giving back every block of a finished
 *       or preempted sequence (deallocate).
 * The choices the pages leave open are fixed as follows:
 *   - block hash: 64-bit FNV-1a (Fowler-Noll-Vo) over the previous block's
 *     hash as 8 little-endian bytes (omitted for the first block), then each
 *     token id as 4 little-endian bytes, top bit cleared (never -1);
 *   - a hit needs the looked-up block's current hash to equal the hash
 *     looked up, as well as equal tokens: a table entry left behind by a
 *     block that was since reset or registered under another hash (same
 *     tokens after a different prefix) must not share K/V computed after a
 *     different prefix, which the chained hash exists to rule out;
 *   - after the first miss in a sequence every later block misses (cached
 *     blocks form a prefix);
 *   - a hit on a block with count 0 (freed, still registered) takes it off
 *     the free list with count 1; a hit on a used block adds 1;
 *   - a miss takes the front of the free list and resets it; a full block
 *     then records its hash and tokens and is registered (replacing an older
 *     entry for that hash);
 *   - deallocate walks the table last-to-first; a block reaching count 0 is
 *     appended to the back of the free list and keeps its hash and tokens;
 *   - can_allocate: free blocks >= the sequence's block count; can_append:
 *     free blocks >= (len % block_size == 1);
 *   - decode metadata: slot = last block * block_size + last-block fill - 1,
 *     context length = len, position = len - 1, input id = last token.
 *
 * Conventions: every pointer here is HOST memory owned by the caller; the
 * manager copies what it keeps.  Nothing here touches the GPU: the caller
 * copies the built arrays to the device (e.g. into pinned buffers, then an
 * async copy on the attention stream).  A manager is not thread-safe: one
 * thread drives it (the scheduler).  Sequences are named by caller-chosen
 * 64-bit ids.  Block tables are written row-major [num_seqs][width], padded
 * with -1.
 *
 * Errors: PKV_ERR_INVALID for a null handle or pointer, an unknown or
 * duplicate sequence id, a count out of range, an output capacity or table
 * width that is too small, or an operation in the wrong state (allocate on a
 * sequence that holds blocks, may_append on one that holds none, removing a
 * sequence that still holds blocks); PKV_ERR_NO_BLOCKS when allocate or
 * may_append needs more free blocks than there are.  A failing call changes
 * nothing.  pkv_last_error() describes the last non-OK status of the thread.
 */
#ifndef PKV_BLOCK_MANAGER_H_
#define PKV_BLOCK_MANAGER_H_

#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/* pkv_block_hash -- the chained block hash above of token_ids[0..n), chained
 * on `prefix` (-1: first block).  Returns a value >= 0, or -1 if token_ids is
 * null with n > 0 or n < 0. */
int64_t pkv_block_hash(const int32_t* token_ids, int32_t n, int64_t prefix);

/* pkv_bm_create -- a pool of num_blocks blocks (ids 0..num_blocks-1, all
 * free, free list in id order) of block_size tokens.  num_blocks >= 1,
 * block_size >= 2 (at 1 every token would both open and fill a block),
 * num_blocks * block_size <= 2^31.  *out receives the handle (release it
 * with pkv_bm_destroy). */
pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Sequences.  add: a new sequence holding a copy of token_ids[0..n), n >= 1,
 * no blocks.  append_token: one more token (the sampled one) at the end.
 * remove: forget a sequence that holds no blocks. */
pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* token_ids,
                               int32_t n);
pkv_status pkv_bm_append_token(pkv_block_manager* bm, int64_t seq_id, int32_t token_id);
pkv_status pkv_bm_remove_sequence(pkv_block_manager* bm, int64_t seq_id);

/* The block manager proper.  can_allocate / can_append write 1 or 0 to *out.
 * allocate: the sequence must hold no blocks; builds its table with prefix
 * sharing and sets its cached-token count.  deallocate: gives back every
 * block and clears the table and cached-token count.  may_append: the
 * decode-step growth for the sequence's current length, called once after
 * each append_token; a call whose table already covers the length changes
 * nothing, and a table more than the one new token behind is
 * PKV_ERR_INVALID. */
pkv_status pkv_bm_can_allocate(const pkv_block_manager* bm, int64_t seq_id, int32_t* out);
pkv_status pkv_bm_allocate(pkv_block_manager* bm, int64_t seq_id);
pkv_status pkv_bm_deallocate(pkv_block_manager* bm, int64_t seq_id);
pkv_status pkv_bm_can_append(const pkv_block_manager* bm, int64_t seq_id, int32_t* out);
pkv_status pkv_bm_may_append(pkv_block_manager* bm, int64_t seq_id);

/* Queries.  num_free_blocks: -1 for a null handle.  sequence: its length,
 * cached-token count and table length.  block_table: the table into
 * out[0..capacity) (capacity >= table length).  block: a block's count, hash
 * (-1: none) and number of recorded tokens.  free_blocks: the free list,
 * front first, into out[0..capacity) (capacity >= number of free blocks). */
int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm);
pkv_status pkv_bm_sequence(const pkv_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                           int32_t* num_cached_tokens, int32_t* num_table_blocks);
pkv_status pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* out,
                              int32_t capacity);
pkv_status pkv_bm_block(const pkv_block_manager* bm, int32_t block_id, int32_t* ref_count,
                        int64_t* hash, int32_t* num_tokens);
pkv_status pkv_bm_free_blocks(const pkv_block_manager* bm, int32_t* out, int32_t capacity);

/* pkv_bm_prefill_sizes -- for the prefill builder: *num_tokens = sum over the
 * sequences of (length - cached tokens), *max_table = longest table. */
pkv_status pkv_bm_prefill_sizes(const pkv_block_manager* bm, const int64_t* seq_ids,
                                int32_t num_seqs, int32_t* num_tokens, int32_t* max_table);

/* pkv_bm_build_prefill -- metadata of one prefill step over seq_ids (each
 * allocated), in order:
 *   input_ids, positions, slot_mapping  [token_capacity >= num_tokens]: the
 *       uncached tokens, their positions (cached length .. length-1) and
 *       their slots (block id * block_size + row);
 *   cu_seqlens_q, cu_seqlens_k  [num_seqs + 1]: cumulative uncached and
 *       total lengths (the layout pkv_paged_prefill_varlen takes);
 *   block_tables  [num_seqs][width], width >= the longest table;
 *   *max_seqlen_q, *max_seqlen_k.
 * input_ids and positions may be null (not written). */
pkv_status pkv_bm_build_prefill(const pkv_block_manager* bm, const int64_t* seq_ids,
                                int32_t num_seqs, int32_t width, int32_t* input_ids,
                                int32_t* positions, int32_t* slot_mapping,
                                int32_t token_capacity, int32_t* cu_seqlens_q,
                                int32_t* cu_seqlens_k, int32_t* block_tables,
                                int32_t* max_seqlen_q, int32_t* max_seqlen_k);

/* pkv_bm_build_decode -- metadata of one decode step over seq_ids (each after
 * may_append), one entry per sequence: input_ids (last token), positions
 * (length - 1), slot_mapping (slot of the last token), context_lens
 * (length); block_tables [num_seqs][width]; *max_context_len.  input_ids and
 * positions may be null.  The arrays feed pkv_paged_decode_step directly. */
pkv_status pkv_bm_build_decode(const pkv_block_manager* bm, const int64_t* seq_ids,
                               int32_t num_seqs, int32_t width, int32_t* input_ids,
                               int32_t* positions, int32_t* slot_mapping, int32_t* context_lens,
                               int32_t* block_tables, int32_t* max_context_len);

/* Batch forms of one engine step's host work (one call per step instead of
 * one per sequence; the same results as the per-sequence calls in order).
 * pkv_bm_append_tokens: append_token(seq_ids[i], token_ids[i]) for each i.
 * pkv_bm_decode_step: may_append for each listed sequence (in order), then
 * pkv_bm_build_decode over them.  A sequence may be listed once.  Every
 * check (ids, states, width, and the number of new blocks the step needs
 * against the free blocks: PKV_ERR_NO_BLOCKS) runs before anything changes,
 * so the scheduler preempts and retries on failure as it would after
 * can_append. */
pkv_status pkv_bm_append_tokens(pkv_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                                const int32_t* token_ids);
pkv_status pkv_bm_decode_step(pkv_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                              int32_t width, int32_t* input_ids, int32_t* positions,
                              int32_t* slot_mapping, int32_t* context_lens,
                              int32_t* block_tables, int32_t* max_context_len);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H_ */
