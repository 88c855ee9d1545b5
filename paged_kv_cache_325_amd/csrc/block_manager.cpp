// Host block manager of the paged KV cache (C ABI in pkv_block_manager.h).
//
// Operation (nano-vllm architecture page, "Block-Struktur und
// Referenzzählung", "Hash-basiertes Prefix Caching", "Dynamische
// Block-Erweiterung", "Prefill- und Decode-Vorbereitung"): a pool of
// fixed-size blocks with reference counts; full blocks are deduplicated by a
// hash chained over the sequence's prefix, confirmed by comparing tokens;
// decode grows a sequence one block at a time and registers each block as
// it fills.
//
// Data structures, sized for pools of 10^4..10^6 blocks and batches of a few
// hundred sequences per step:
//   * blocks: flat arrays (count, hash, recorded-token count) plus one flat
//     [num_blocks][block_size] token store, so no per-block allocation;
//   * free list: an intrusive doubly linked list over block ids, so popping
//     the front, appending at the back and taking a registered block out of
//     the middle (a hit on a freed block) are all O(1);
//   * hash -> block id: an open-addressing table (linear probing, power-of-
//     two capacity >= 2 x num_blocks, never more than half full because
//     every live entry names a distinct block);
//   * sequences: an unordered_map from id to tokens, table and cached count.
// Every entry point validates first and mutates only once nothing can fail,
// so a failing call leaves the manager unchanged.
#include <string.h>

#include <unordered_map>
#include <vector>

#include "pkv_block_manager.h"
#include "pkv_error.h"

namespace {

using pkv::fail;

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;
constexpr uint64_t kHashMask = 0x7fffffffffffffffull;

inline uint64_t fnv_bytes(uint64_t h, uint64_t word, int nbytes) {
  for (int i = 0; i < nbytes; ++i) {
    h ^= (word >> (8 * i)) & 0xffu;
    h *= kFnvPrime;
  }
  return h;
}

// 64-bit FNV-1a over [prefix as 8 LE bytes if != -1][tokens as 4 LE bytes].
int64_t chain_hash(const int32_t* tokens, int32_t n, int64_t prefix) {
  uint64_t h = kFnvOffset;
  if (prefix != -1) h = fnv_bytes(h, (uint64_t)prefix, 8);
  for (int32_t i = 0; i < n; ++i) h = fnv_bytes(h, (uint32_t)tokens[i], 4);
  return (int64_t)(h & kHashMask);
}

struct Sequence {
  std::vector<int32_t> tokens;
  std::vector<int32_t> table;
  int32_t num_cached_tokens = 0;
  uint64_t stamp = 0;  // last batch call that listed it (duplicate check)

  int32_t len() const { return (int32_t)tokens.size(); }
};

}  // namespace

struct pkv_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  // per block
  std::vector<int32_t> ref_count;
  std::vector<int64_t> hash;
  std::vector<int32_t> ntok;    // recorded tokens (block_size once hashed, else 0)
  std::vector<int32_t> tokens;  // [num_blocks][block_size]
  // free list
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> is_free;
  int32_t head = -1, tail = -1, nfree = 0;
  // hash -> block id (open addressing; key -1 = empty slot)
  std::vector<int64_t> ht_key;
  std::vector<int32_t> ht_val;
  uint64_t ht_mask = 0;
  size_t ht_used = 0;  // occupied slots, live or stale
  std::unordered_map<int64_t, Sequence> seqs;
  uint64_t batch_calls = 0;

  int32_t nblocks_of(int32_t len) const { return (len + block_size - 1) / block_size; }

  // ---- free list ----------------------------------------------------------
  void push_back_free(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    is_free[b] = 1;
    ++nfree;
  }
  void unlink_free(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    is_free[b] = 0;
    --nfree;
  }

  // ---- hash table ---------------------------------------------------------
  uint64_t slot_of(int64_t key) const {
    // hashes are already well mixed: take the low bits
    return (uint64_t)key & ht_mask;
  }
  int32_t ht_get(int64_t key) const {
    for (uint64_t i = slot_of(key);; i = (i + 1) & ht_mask) {
      if (ht_key[i] == -1) return -1;
      if (ht_key[i] == key) return ht_val[i];
    }
  }
  void ht_put(int64_t key, int32_t val) {
    for (uint64_t i = slot_of(key);; i = (i + 1) & ht_mask) {
      if (ht_key[i] == -1 || ht_key[i] == key) {
        ht_used += ht_key[i] == -1;
        ht_key[i] = key;
        ht_val[i] = val;
        return;
      }
    }
  }
  // An entry goes stale when its block is reset or registered under another
  // hash; a stale entry can never produce a hit (a hit needs the block's own
  // hash to match), so stale entries are dropped whenever the table would
  // pass half full.  Live entries name distinct blocks, so at most
  // num_blocks <= capacity / 2 - 1 remain and lookups stay short.
  void ht_maybe_compact() {
    if (2 * (ht_used + 1) <= ht_key.size()) return;
    std::vector<int64_t> keys(ht_key.size(), -1);
    std::vector<int32_t> vals(ht_key.size(), -1);
    keys.swap(ht_key);
    vals.swap(ht_val);
    ht_used = 0;
    for (size_t i = 0; i < keys.size(); ++i) {
      const int32_t b = vals[i];
      if (keys[i] != -1 && hash[b] == keys[i]) ht_put(keys[i], b);
    }
  }
  void register_block(int32_t b, int64_t h, const int32_t* toks) {
    hash[b] = h;
    ntok[b] = block_size;
    memcpy(&tokens[(size_t)b * block_size], toks, sizeof(int32_t) * block_size);
    ht_maybe_compact();
    ht_put(h, b);
  }

  // ---- single blocks ------------------------------------------------------
  int32_t take_block(int32_t b) {  // reset and take a free block
    unlink_free(b);
    ref_count[b] = 1;
    hash[b] = -1;
    ntok[b] = 0;
    return b;
  }
  void release_block(int32_t b) {
    if (--ref_count[b] == 0) push_back_free(b);
  }
  bool tokens_equal(int32_t b, const int32_t* toks) const {
    return ntok[b] == block_size &&
           memcmp(&tokens[(size_t)b * block_size], toks, sizeof(int32_t) * block_size) == 0;
  }
};

namespace {

pkv_status find_seq(const pkv_block_manager* bm, int64_t id, const Sequence** out) {
  if (!bm) return fail(PKV_ERR_INVALID, "null block manager");
  auto it = bm->seqs.find(id);
  if (it == bm->seqs.end())
    return fail(PKV_ERR_INVALID, "unknown sequence id %lld", (long long)id);
  *out = &it->second;
  return PKV_OK;
}

pkv_status find_seq(pkv_block_manager* bm, int64_t id, Sequence** out) {
  const Sequence* s = nullptr;
  const pkv_status st = find_seq(static_cast<const pkv_block_manager*>(bm), id, &s);
  *out = const_cast<Sequence*>(s);
  return st;
}

// Checks shared by the two builders: every id known and allocated, no
// duplicates are required to be absent (a sequence may appear once per step;
// the builder does not enforce it).
pkv_status check_batch(const pkv_block_manager* bm, const int64_t* ids, int32_t n,
                       std::vector<const Sequence*>* out) {
  if (!bm) return fail(PKV_ERR_INVALID, "null block manager");
  if (n < 0) return fail(PKV_ERR_INVALID, "num_seqs (%d) < 0", n);
  if (n > 0 && !ids) return fail(PKV_ERR_INVALID, "seq_ids is null");
  out->resize(n);
  for (int32_t i = 0; i < n; ++i) {
    const Sequence* s = nullptr;
    if (pkv_status st = find_seq(bm, ids[i], &s)) return st;
    if (s->table.empty())
      return fail(PKV_ERR_INVALID, "sequence %lld holds no blocks", (long long)ids[i]);
    (*out)[i] = s;
  }
  return PKV_OK;
}

// may_append's checks: *need = 1 when the sequence's newest token opens a
// block.  Called once per appended token, the table is one block short
// exactly then; a table that already covers the length needs nothing.
pkv_status check_growth(const pkv_block_manager* bm, const Sequence& s, int64_t seq_id,
                        int32_t* need) {
  if (s.table.empty())
    return fail(PKV_ERR_INVALID, "sequence %lld holds no blocks (allocate first)",
                (long long)seq_id);
  const int32_t nb = bm->nblocks_of(s.len());
  const int32_t nt = (int32_t)s.table.size();
  const bool opens = s.len() % bm->block_size == 1 && nt == nb - 1;
  if (!opens && nt != nb)
    return fail(PKV_ERR_INVALID,
                "sequence %lld: %d tokens but %d blocks (one may_append per appended token)",
                (long long)seq_id, s.len(), nt);
  *need = opens ? 1 : 0;
  return PKV_OK;
}

// may_append's effect, once check_growth passed and a free block is there if
// one is needed.
void grow(pkv_block_manager* bm, Sequence* s) {
  const int32_t B = bm->block_size;
  const int32_t nb = bm->nblocks_of(s->len());
  const int32_t nt = (int32_t)s->table.size();
  const int32_t r = s->len() % B;
  if (r == 1 && nt == nb - 1) {  // the new token opens a block
    s->table.push_back(bm->take_block(bm->head));
  } else if (r == 0 && bm->hash[s->table.back()] == -1) {
    // the new token fills the last block: hash and register it
    const int32_t last = s->table.back();
    const int64_t prefix = nt > 1 ? bm->hash[s->table[nb - 2]] : -1;
    const int32_t* toks = s->tokens.data() + (size_t)(nb - 1) * B;
    bm->register_block(last, chain_hash(toks, B, prefix), toks);
  }
}

void write_table(const Sequence& s, int32_t width, int32_t* row) {
  const int32_t n = (int32_t)s.table.size();
  memcpy(row, s.table.data(), sizeof(int32_t) * n);
  for (int32_t j = n; j < width; ++j) row[j] = -1;
}

}  // namespace

extern "C" {

int64_t pkv_block_hash(const int32_t* token_ids, int32_t n, int64_t prefix) {
  if (n < 0 || (n > 0 && !token_ids)) return -1;
  return chain_hash(token_ids, n, prefix);
}

pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_block_manager** out) {
  if (!out) return fail(PKV_ERR_INVALID, "out is null");
  *out = nullptr;
  if (num_blocks < 1 || block_size < 2)
    return fail(PKV_ERR_INVALID, "num_blocks (%d) must be >= 1 and block_size (%d) >= 2",
                num_blocks, block_size);
  if ((int64_t)num_blocks * block_size > (int64_t)1 << 31)
    return fail(PKV_ERR_INVALID, "num_blocks * block_size (%lld) exceeds the int32 slot range",
                (long long)num_blocks * block_size);
  auto* bm = new pkv_block_manager;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref_count.assign(num_blocks, 0);
  bm->hash.assign(num_blocks, -1);
  bm->ntok.assign(num_blocks, 0);
  bm->tokens.assign((size_t)num_blocks * block_size, 0);
  bm->prev.assign(num_blocks, -1);
  bm->next.assign(num_blocks, -1);
  bm->is_free.assign(num_blocks, 0);
  for (int32_t b = 0; b < num_blocks; ++b) bm->push_back_free(b);
  size_t cap = 16;
  while (cap < 2 * (size_t)num_blocks + 2) cap <<= 1;
  bm->ht_key.assign(cap, -1);
  bm->ht_val.assign(cap, -1);
  bm->ht_mask = cap - 1;
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* token_ids,
                               int32_t n) {
  if (!bm) return fail(PKV_ERR_INVALID, "null block manager");
  if (n < 1) return fail(PKV_ERR_INVALID, "a sequence needs at least one token (n = %d)", n);
  if (!token_ids) return fail(PKV_ERR_INVALID, "token_ids is null");
  if (bm->seqs.count(seq_id))
    return fail(PKV_ERR_INVALID, "sequence id %lld already exists", (long long)seq_id);
  Sequence& s = bm->seqs[seq_id];
  s.tokens.assign(token_ids, token_ids + n);
  return PKV_OK;
}

pkv_status pkv_bm_append_token(pkv_block_manager* bm, int64_t seq_id, int32_t token_id) {
  Sequence* s = nullptr;
  if (pkv_status st = find_seq(bm, seq_id, &s)) return st;
  if (s->len() == 0x7fffffff) return fail(PKV_ERR_INVALID, "sequence is at the int32 limit");
  s->tokens.push_back(token_id);
  return PKV_OK;
}

pkv_status pkv_bm_remove_sequence(pkv_block_manager* bm, int64_t seq_id) {
  Sequence* s = nullptr;
  if (pkv_status st = find_seq(bm, seq_id, &s)) return st;
  if (!s->table.empty())
    return fail(PKV_ERR_INVALID, "sequence %lld still holds %zu blocks (deallocate first)",
                (long long)seq_id, s->table.size());
  bm->seqs.erase(seq_id);
  return PKV_OK;
}

pkv_status pkv_bm_can_allocate(const pkv_block_manager* bm, int64_t seq_id, int32_t* out) {
  const Sequence* s = nullptr;
  if (pkv_status st = find_seq(bm, seq_id, &s)) return st;
  if (!out) return fail(PKV_ERR_INVALID, "out is null");
  *out = bm->nfree >= bm->nblocks_of(s->len()) ? 1 : 0;
  return PKV_OK;
}

pkv_status pkv_bm_allocate(pkv_block_manager* bm, int64_t seq_id) {
  Sequence* s = nullptr;
  if (pkv_status st = find_seq(bm, seq_id, &s)) return st;
  if (!s->table.empty())
    return fail(PKV_ERR_INVALID, "sequence %lld already holds blocks", (long long)seq_id);
  const int32_t B = bm->block_size;
  const int32_t nb = bm->nblocks_of(s->len());
  if (bm->nfree < nb)
    return fail(PKV_ERR_NO_BLOCKS, "sequence %lld needs %d blocks, %d free", (long long)seq_id,
                nb, bm->nfree);
  s->table.reserve(nb);
  int64_t h = -1;
  bool missed = false;
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t* toks = s->tokens.data() + (size_t)i * B;
    const bool full = (i + 1) * (int64_t)B <= s->len();
    h = full ? chain_hash(toks, B, h) : -1;
    int32_t b = -1;
    if (!missed && full) {
      const int32_t cand = bm->ht_get(h);
      if (cand >= 0 && bm->hash[cand] == h && bm->tokens_equal(cand, toks)) b = cand;
    }
    if (b < 0) missed = true;
    if (missed) {
      b = bm->take_block(bm->head);
      if (full) bm->register_block(b, h, toks);
    } else {
      s->num_cached_tokens += B;
      if (bm->is_free[b]) {  // freed but still registered: take it back
        bm->unlink_free(b);
        bm->ref_count[b] = 1;
      } else {
        ++bm->ref_count[b];
      }
    }
    s->table.push_back(b);
  }
  return PKV_OK;
}

pkv_status pkv_bm_deallocate(pkv_block_manager* bm, int64_t seq_id) {
  Sequence* s = nullptr;
  if (pkv_status st = find_seq(bm, seq_id, &s)) return st;
  for (auto it = s->table.rbegin(); it != s->table.rend(); ++it) bm->release_block(*it);
  s->table.clear();
  s->num_cached_tokens = 0;
  return PKV_OK;
}

pkv_status pkv_bm_can_append(const pkv_block_manager* bm, int64_t seq_id, int32_t* out) {
  const Sequence* s = nullptr;
  if (pkv_status st = find_seq(bm, seq_id, &s)) return st;
  if (!out) return fail(PKV_ERR_INVALID, "out is null");
  const int32_t need = s->len() % bm->block_size == 1 ? 1 : 0;
  *out = bm->nfree >= need ? 1 : 0;
  return PKV_OK;
}

pkv_status pkv_bm_may_append(pkv_block_manager* bm, int64_t seq_id) {
  Sequence* s = nullptr;
  if (pkv_status st = find_seq(bm, seq_id, &s)) return st;
  int32_t need = 0;
  if (pkv_status st = check_growth(bm, *s, seq_id, &need)) return st;
  if (bm->nfree < need)
    return fail(PKV_ERR_NO_BLOCKS, "sequence %lld needs a block, none free", (long long)seq_id);
  grow(bm, s);
  return PKV_OK;
}

int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) { return bm ? bm->nfree : -1; }

pkv_status pkv_bm_sequence(const pkv_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                           int32_t* num_cached_tokens, int32_t* num_table_blocks) {
  const Sequence* s = nullptr;
  if (pkv_status st = find_seq(bm, seq_id, &s)) return st;
  if (num_tokens) *num_tokens = s->len();
  if (num_cached_tokens) *num_cached_tokens = s->num_cached_tokens;
  if (num_table_blocks) *num_table_blocks = (int32_t)s->table.size();
  return PKV_OK;
}

pkv_status pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* out,
                              int32_t capacity) {
  const Sequence* s = nullptr;
  if (pkv_status st = find_seq(bm, seq_id, &s)) return st;
  const int32_t n = (int32_t)s->table.size();
  if (capacity < n) return fail(PKV_ERR_INVALID, "capacity %d < table length %d", capacity, n);
  if (n > 0 && !out) return fail(PKV_ERR_INVALID, "out is null");
  if (n > 0) memcpy(out, s->table.data(), sizeof(int32_t) * n);
  return PKV_OK;
}

pkv_status pkv_bm_block(const pkv_block_manager* bm, int32_t block_id, int32_t* ref_count,
                        int64_t* hash, int32_t* num_tokens) {
  if (!bm) return fail(PKV_ERR_INVALID, "null block manager");
  if (block_id < 0 || block_id >= bm->num_blocks)
    return fail(PKV_ERR_INVALID, "block id %d outside [0, %d)", block_id, bm->num_blocks);
  if (ref_count) *ref_count = bm->ref_count[block_id];
  if (hash) *hash = bm->hash[block_id];
  if (num_tokens) *num_tokens = bm->ntok[block_id];
  return PKV_OK;
}

pkv_status pkv_bm_free_blocks(const pkv_block_manager* bm, int32_t* out, int32_t capacity) {
  if (!bm) return fail(PKV_ERR_INVALID, "null block manager");
  if (capacity < bm->nfree)
    return fail(PKV_ERR_INVALID, "capacity %d < free blocks %d", capacity, bm->nfree);
  if (bm->nfree > 0 && !out) return fail(PKV_ERR_INVALID, "out is null");
  int32_t i = 0;
  for (int32_t b = bm->head; b >= 0; b = bm->next[b]) out[i++] = b;
  return PKV_OK;
}

pkv_status pkv_bm_prefill_sizes(const pkv_block_manager* bm, const int64_t* seq_ids,
                                int32_t num_seqs, int32_t* num_tokens, int32_t* max_table) {
  std::vector<const Sequence*> seqs;
  if (pkv_status st = check_batch(bm, seq_ids, num_seqs, &seqs)) return st;
  int64_t tok = 0;
  int32_t mt = 0;
  for (const Sequence* s : seqs) {
    tok += s->len() - s->num_cached_tokens;
    mt = (int32_t)s->table.size() > mt ? (int32_t)s->table.size() : mt;
  }
  if (tok > 0x7fffffff) return fail(PKV_ERR_INVALID, "step holds more than 2^31 tokens");
  if (num_tokens) *num_tokens = (int32_t)tok;
  if (max_table) *max_table = mt;
  return PKV_OK;
}

pkv_status pkv_bm_build_prefill(const pkv_block_manager* bm, const int64_t* seq_ids,
                                int32_t num_seqs, int32_t width, int32_t* input_ids,
                                int32_t* positions, int32_t* slot_mapping,
                                int32_t token_capacity, int32_t* cu_seqlens_q,
                                int32_t* cu_seqlens_k, int32_t* block_tables,
                                int32_t* max_seqlen_q, int32_t* max_seqlen_k) {
  int32_t ntok = 0, mt = 0;
  if (pkv_status st = pkv_bm_prefill_sizes(bm, seq_ids, num_seqs, &ntok, &mt)) return st;
  if (width < mt) return fail(PKV_ERR_INVALID, "width %d < longest table %d", width, mt);
  if (token_capacity < ntok)
    return fail(PKV_ERR_INVALID, "token_capacity %d < uncached tokens %d", token_capacity, ntok);
  if ((ntok > 0 && !slot_mapping) || !cu_seqlens_q || !cu_seqlens_k ||
      (num_seqs > 0 && width > 0 && !block_tables))
    return fail(PKV_ERR_INVALID, "an output array is null");
  const int32_t B = bm->block_size;
  int32_t t = 0, mq = 0, mk = 0;
  cu_seqlens_q[0] = cu_seqlens_k[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Sequence& s = bm->seqs.find(seq_ids[i])->second;
    const int32_t n = s.len(), c = s.num_cached_tokens;
    for (int32_t p = c; p < n; ++p, ++t) {
      if (input_ids) input_ids[t] = s.tokens[p];
      if (positions) positions[t] = p;
      slot_mapping[t] = s.table[p / B] * B + p % B;
    }
    cu_seqlens_q[i + 1] = cu_seqlens_q[i] + (n - c);
    cu_seqlens_k[i + 1] = cu_seqlens_k[i] + n;
    mq = n - c > mq ? n - c : mq;
    mk = n > mk ? n : mk;
    write_table(s, width, block_tables + (size_t)i * width);
  }
  if (max_seqlen_q) *max_seqlen_q = mq;
  if (max_seqlen_k) *max_seqlen_k = mk;
  return PKV_OK;
}

pkv_status pkv_bm_build_decode(const pkv_block_manager* bm, const int64_t* seq_ids,
                               int32_t num_seqs, int32_t width, int32_t* input_ids,
                               int32_t* positions, int32_t* slot_mapping, int32_t* context_lens,
                               int32_t* block_tables, int32_t* max_context_len) {
  std::vector<const Sequence*> seqs;
  if (pkv_status st = check_batch(bm, seq_ids, num_seqs, &seqs)) return st;
  if (num_seqs > 0 && (!slot_mapping || !context_lens || !block_tables))
    return fail(PKV_ERR_INVALID, "an output array is null");
  const int32_t B = bm->block_size;
  for (const Sequence* s : seqs) {
    const int32_t nt = (int32_t)s->table.size();
    if (nt != bm->nblocks_of(s->len()))
      return fail(PKV_ERR_INVALID, "a sequence of %d tokens holds %d blocks (may_append first)",
                  s->len(), nt);
    if (width < nt) return fail(PKV_ERR_INVALID, "width %d < table length %d", width, nt);
  }
  int32_t mk = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Sequence& s = *seqs[i];
    const int32_t n = s.len();
    const int32_t last_fill = n - (bm->nblocks_of(n) - 1) * B;
    if (input_ids) input_ids[i] = s.tokens.back();
    if (positions) positions[i] = n - 1;
    slot_mapping[i] = s.table.back() * B + last_fill - 1;
    context_lens[i] = n;
    mk = n > mk ? n : mk;
    write_table(s, width, block_tables + (size_t)i * width);
  }
  if (max_context_len) *max_context_len = mk;
  return PKV_OK;
}

pkv_status pkv_bm_append_tokens(pkv_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                                const int32_t* token_ids) {
  if (!bm) return fail(PKV_ERR_INVALID, "null block manager");
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "num_seqs (%d) < 0", num_seqs);
  if (num_seqs > 0 && (!seq_ids || !token_ids))
    return fail(PKV_ERR_INVALID, "seq_ids or token_ids is null");
  std::vector<Sequence*> seqs(num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (pkv_status st = find_seq(bm, seq_ids[i], &seqs[i])) return st;
    if (seqs[i]->len() == 0x7fffffff)
      return fail(PKV_ERR_INVALID, "sequence %lld is at the int32 limit", (long long)seq_ids[i]);
  }
  for (int32_t i = 0; i < num_seqs; ++i) seqs[i]->tokens.push_back(token_ids[i]);
  return PKV_OK;
}

pkv_status pkv_bm_decode_step(pkv_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                              int32_t width, int32_t* input_ids, int32_t* positions,
                              int32_t* slot_mapping, int32_t* context_lens,
                              int32_t* block_tables, int32_t* max_context_len) {
  if (!bm) return fail(PKV_ERR_INVALID, "null block manager");
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "num_seqs (%d) < 0", num_seqs);
  if (num_seqs > 0 && !seq_ids) return fail(PKV_ERR_INVALID, "seq_ids is null");
  if (num_seqs > 0 && (!slot_mapping || !context_lens || !block_tables))
    return fail(PKV_ERR_INVALID, "an output array is null");
  std::vector<Sequence*> seqs(num_seqs);
  int32_t need = 0;
  const uint64_t stamp = ++bm->batch_calls;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (pkv_status st = find_seq(bm, seq_ids[i], &seqs[i])) return st;
    if (seqs[i]->stamp == stamp)
      return fail(PKV_ERR_INVALID, "sequence %lld listed twice", (long long)seq_ids[i]);
    seqs[i]->stamp = stamp;
    int32_t n1 = 0;
    if (pkv_status st = check_growth(bm, *seqs[i], seq_ids[i], &n1)) return st;
    need += n1;
    if (width < bm->nblocks_of(seqs[i]->len()))
      return fail(PKV_ERR_INVALID, "width %d < table length %d", width,
                  bm->nblocks_of(seqs[i]->len()));
  }
  if (bm->nfree < need)
    return fail(PKV_ERR_NO_BLOCKS, "the step needs %d new blocks, %d free", need, bm->nfree);
  for (Sequence* s : seqs) grow(bm, s);
  return pkv_bm_build_decode(bm, seq_ids, num_seqs, width, input_ids, positions, slot_mapping,
                             context_lens, block_tables, max_context_len);
}

}  // extern "C"
