"""Plain-Python block manager: block allocation, prefix sharing and growth of
a paged KV cache, plus the per-step metadata (slots, tables, lengths) that the
attention kernels consume.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module, and this module imports nothing from it.

Sources, cited by page title and section (nano-vllm architecture page,
"Architektur im Überblick", repothread.com, unless noted):

* "Block-Struktur und Referenzzählung": a block carries its id, a reference
  count, a hash (-1 while it has none) and the token ids it holds; a block is
  given back only when its count drops to 0.
* "Hash-basiertes Prefix Caching": allocation walks the blocks of a sequence;
  a full block gets a hash chained on the hash of the block before it (a
  partial block gets -1); a table lookup hit whose recorded tokens equal the
  block's tokens shares that block (count + 1, cached tokens + block size);
  anything else takes the first free block.
* "Dynamische Block-Erweiterung": growth in decode has three cases on
  len(seq) % block_size: 1 -> a new block is taken and appended to the
  table; 0 -> the last block has just filled, so it gets its chained hash,
  records its tokens and is entered in the hash table; otherwise nothing.
* "Block-Berechnung und Token-Appending": num_blocks = ceil(len / B); tokens
  in the last block = len - (num_blocks - 1) B; appending a token extends
  the token list.
* "Prefill- und Decode-Vorbereitung": prefill computes the positions from the
  cached-prefix length to the sequence length, and writes the slots of the
  uncached blocks (slot = block id * B + row).
* "Prefill-Scheduling", "Decode-Scheduling mit Preemption" and
  "Postprocessing und Abschluss-Erkennung": can_allocate gates admission,
  can_append gates a decode step, and both preemption and completion give
  back every block of the sequence (deallocate).
* "Kern-Designentscheidungen" item 2 and the source study ("Nano-vLLM
  源碼學習", hk.pswp.cn), section 1 "BlockManager": blocks are found by hash
  through a hash -> block id table.

Readings where the pages are silent or only sketch a step:
  H1 the block hash is 64-bit FNV-1a (the published definition of Fowler,
     Noll and Vo: offset basis 0xcbf29ce484222325, prime 0x100000001b3, xor
     each byte then multiply) over the previous block's hash as 8
     little-endian bytes (left out for the first block) followed by each
     token id as 4 little-endian bytes (int32), with the top bit cleared so
     that a hash is never the -1 sentinel.  The pages use xxHash; any hash
     serves, since a hit also compares the tokens.
  H2 once a block of a sequence misses, every later block misses too: the
     cached blocks form a prefix, which the prefill preparation assumes (it
     computes from the cached-prefix length on).
  H3 a hit on a block whose count is 0 (given back, but still in the hash
     table) takes it out of the free list with count 1; a hit on a block in
     use adds 1 to its count.
  H4 a miss takes the block at the front of the free list and resets it
     (count 1, hash -1, no tokens); if the sequence's block is full, the
     block then records the hash and tokens and the hash table maps the hash
     to it (replacing an older entry).
  H5 deallocate walks the table from its last block to its first; a block
     whose count drops to 0 goes to the back of the free list and keeps its
     hash and tokens (a later identical prefix can still hit it); the
     sequence's table and cached-token count are cleared.
  H6 can_allocate: free blocks >= the sequence's block count; can_append:
     free blocks >= 1 when len % B == 1, else always.
  H7 in may_append the length already counts the token this step decodes; a
     full last block is hashed on the hash of the block before it (-1 for the
     first block).
  H8 decode metadata: slot = last block * B + tokens in the last block - 1,
     context length = len, position = len - 1, input id = the last token;
     tables are padded with -1 to the requested width.

  H9 a hit also needs the block's current hash to equal the looked-up hash:
     the listing compares only tokens, but a hash-table entry can outlive
     its block's registration (the block was reset, or registered again
     under another hash -- the same tokens after a different prefix), and
     such an entry must not share K/V that were computed after a different
     prefix, which is what chaining the hash on the prefix is for.
Every function here is pinned by CPU tests (published FNV test vectors, a
hand-worked scenario under tests/golden/, invariants over seeded random
operation streams, and planted mistakes); none is "parity unpinned".
"""

from __future__ import annotations

FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3
_MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a of a byte string (published definition)."""
    h = FNV64_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) & _MASK64
    return h


def block_hash_bytes(token_ids, prefix: int) -> bytes:
    """The bytes a block hash covers (reading H1)."""
    out = bytearray()
    if prefix != -1:
        out += (prefix & _MASK64).to_bytes(8, "little")
    for t in token_ids:
        out += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
    return bytes(out)


def compute_hash(token_ids, prefix: int = -1) -> int:
    """Chained block hash (reading H1); never -1."""
    return fnv1a64(block_hash_bytes(token_ids, prefix)) & ((1 << 63) - 1)


class Sequence:
    """The block-manager view of one request (architecture page, "Sequenz-
    Status und Eigenschaften", "Block-Berechnung und Token-Appending"): its
    token ids, the physical blocks holding them in logical order, and how
    many leading tokens were found in the cache when it was admitted."""

    def __init__(self, seq_id: int, token_ids, block_size: int):
        self.seq_id = seq_id
        self.token_ids = [int(t) for t in token_ids]
        self.block_size = block_size
        self.num_cached_tokens = 0
        self.block_table: list[int] = []

    def __len__(self) -> int:
        return len(self.token_ids)

    @property
    def num_blocks(self) -> int:
        """ceil(len / B)."""
        return -(-len(self.token_ids) // self.block_size)

    @property
    def num_cached_blocks(self) -> int:
        return self.num_cached_tokens // self.block_size

    @property
    def last_block_num_tokens(self) -> int:
        """Tokens held by the last block: len - (num_blocks - 1) B."""
        return len(self.token_ids) - (self.num_blocks - 1) * self.block_size

    def block(self, i: int) -> list[int]:
        """Token ids of logical block i."""
        lo = i * self.block_size
        return self.token_ids[lo:lo + self.block_size]

    def append_token(self, token_id: int) -> None:
        self.token_ids.append(int(token_id))


class BlockManager:
    """A pool of ``num_blocks`` physical blocks with reference counts and
    hash-based prefix sharing (architecture page, "Block-Struktur und
    Referenzzählung", "Hash-basiertes Prefix Caching", "Dynamische
    Block-Erweiterung").

    State, one entry per physical block:
      count[b]     number of sequences whose table holds b (0: b is free);
      recorded[b]  (hash, tokens) b was registered with when it held a full
                   block, or None; kept when b is given back (H5) and
                   dropped when b is handed out for new contents (H4);
    and for the pool:
      index        hash -> the block most recently registered under it
                   (an entry can be stale, see H9);
      free         the free blocks in hand-out order (front first).
    """

    def __init__(self, num_blocks: int, block_size: int):
        assert num_blocks >= 1 and block_size >= 2  # at 1 a token opens and fills a block
        self.block_size = block_size
        self.count = [0] * num_blocks
        self.recorded: list = [None] * num_blocks
        self.index: dict[int, int] = {}
        self.free: list[int] = list(range(num_blocks))

    def state(self, b: int):
        """(count, registered hash or -1, number of recorded tokens) of block b."""
        rec = self.recorded[b]
        return self.count[b], (-1 if rec is None else rec[0]), (0 if rec is None else len(rec[1]))

    # -- moves of single blocks ----------------------------------------------
    def _fresh(self) -> int:
        """Hand out the front free block for new contents (H4)."""
        b = self.free.pop(0)
        assert self.count[b] == 0
        self.count[b] = 1
        self.recorded[b] = None
        return b

    def _take(self, b: int) -> None:
        """One more sequence holds cached block b; a given-back block leaves
        the free list (H3)."""
        if self.count[b] == 0:
            self.free.remove(b)
        self.count[b] += 1

    def _register(self, b: int, h: int, tokens) -> None:
        """Block b now holds a full block with chained hash h (H4, H7)."""
        self.recorded[b] = (h, tuple(tokens))
        self.index[h] = b

    def _holds(self, b: int, h: int, tokens) -> bool:
        """Block b is registered under h with exactly these tokens (H9)."""
        return self.recorded[b] == (h, tuple(tokens))

    # -- allocation -------------------------------------------------------------
    def chained_hashes(self, seq: Sequence) -> list[int]:
        """One entry per logical block: the hash of a full block, chained on
        the hash of the block before it (H1); -1 for a partial last block."""
        out, prev = [], -1
        for i in range(seq.num_blocks):
            tokens = seq.block(i)
            if len(tokens) < self.block_size:
                out.append(-1)
            else:
                prev = compute_hash(tokens, prev)
                out.append(prev)
        return out

    def cache_hits(self, seq: Sequence, hashes) -> list[bool]:
        """Which logical blocks are served from the cache: the longest run of
        leading blocks whose hash finds a block holding that hash and those
        tokens (H2: nothing after the first miss; H9)."""
        hits = []
        for i, h in enumerate(hashes):
            b = self.index.get(h) if h != -1 else None
            if b is None or not self._holds(b, h, seq.block(i)) or (hits and not hits[-1]):
                hits.append(False)
            else:
                hits.append(True)
        return hits

    def can_allocate(self, seq: Sequence) -> bool:
        return len(self.free) >= seq.num_blocks  # H6

    def allocate(self, seq: Sequence) -> None:
        """Give a newly admitted sequence its blocks: cached ones for its
        cache hits, fresh ones from the front of the free list for the rest;
        every full block ends up registered under its chained hash."""
        assert not seq.block_table
        hashes = self.chained_hashes(seq)
        hits = self.cache_hits(seq, hashes)
        table = []
        for i, (h, hit) in enumerate(zip(hashes, hits)):
            if hit:
                b = self.index[h]
                self._take(b)
            else:
                b = self._fresh()
            if h != -1:
                self._register(b, h, seq.block(i))
            table.append(b)
        seq.block_table = table
        seq.num_cached_tokens = self.block_size * sum(hits)

    def deallocate(self, seq: Sequence) -> None:
        """Give back a finished or preempted sequence's blocks, last logical
        block first; a block nobody holds any more joins the back of the free
        list with its registration intact (H5)."""
        for b in seq.block_table[::-1]:
            self.count[b] -= 1
            if self.count[b] == 0:
                self.free.append(b)
        seq.num_cached_tokens = 0
        seq.block_table = []

    # -- decode growth ------------------------------------------------------------
    def can_append(self, seq: Sequence) -> bool:
        opens_block = len(seq) % self.block_size == 1
        return len(self.free) >= (1 if opens_block else 0)  # H6

    def may_append(self, seq: Sequence) -> None:
        """After a decoded token was appended (H7): a token that opens a block
        gets a fresh one; a token that fills the last block seals it (hash
        chained on the previous block's, tokens recorded, entered in the
        index); any other token needs nothing."""
        fill = len(seq) % self.block_size
        last = seq.block_table[-1]
        if fill == 1:
            assert self.recorded[last] is not None
            seq.block_table.append(self._fresh())
        elif fill == 0:
            assert self.recorded[last] is None
            tail = seq.block_table[-2] if len(seq.block_table) > 1 else None
            prev = -1 if tail is None else self.recorded[tail][0]
            tokens = seq.block(seq.num_blocks - 1)
            self._register(last, compute_hash(tokens, prev), tokens)
        else:
            assert self.recorded[last] is None


# -- per-step metadata (architecture page, "Prefill- und Decode-Vorbereitung")


def _padded_tables(seqs, width: int):
    tables = []
    for s in seqs:
        assert len(s.block_table) <= width
        tables.append(list(s.block_table) + [-1] * (width - len(s.block_table)))
    return tables


def prepare_prefill(seqs, width: int) -> dict:
    """Metadata of one prefill step: the uncached tokens' ids, positions and
    slots; cumulative query and key lengths; padded block tables."""
    input_ids, positions, slots = [], [], []
    cu_q, cu_k = [0], [0]
    for s in seqs:
        n = len(s)
        input_ids += s.token_ids[s.num_cached_tokens:]
        positions += list(range(s.num_cached_tokens, n))
        cu_q.append(cu_q[-1] + n - s.num_cached_tokens)
        cu_k.append(cu_k[-1] + n)
        for i in range(s.num_cached_blocks, s.num_blocks):
            start = s.block_table[i] * s.block_size
            count = s.block_size if i != s.num_blocks - 1 else s.last_block_num_tokens
            slots += list(range(start, start + count))
    return {
        "input_ids": input_ids, "positions": positions, "slot_mapping": slots,
        "cu_seqlens_q": cu_q, "cu_seqlens_k": cu_k,
        "max_seqlen_q": max([b - a for a, b in zip(cu_q, cu_q[1:])], default=0),
        "max_seqlen_k": max([b - a for a, b in zip(cu_k, cu_k[1:])], default=0),
        "block_tables": _padded_tables(seqs, width),
    }


def prepare_decode(seqs, width: int) -> dict:
    """Metadata of one decode step (reading H8)."""
    return {
        "input_ids": [s.token_ids[-1] for s in seqs],
        "positions": [len(s) - 1 for s in seqs],
        "slot_mapping": [s.block_table[-1] * s.block_size + s.last_block_num_tokens - 1
                         for s in seqs],
        "context_lens": [len(s) for s in seqs],
        "max_context_len": max([len(s) for s in seqs], default=0),
        "block_tables": _padded_tables(seqs, width),
    }
