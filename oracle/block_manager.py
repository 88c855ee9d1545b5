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


class Block:
    """One physical block (architecture page, "Block-Struktur und
    Referenzzählung")."""

    def __init__(self, block_id: int):
        self.block_id = block_id
        self.ref_count = 0
        self.hash = -1
        self.token_ids: list[int] = []

    def update(self, h: int, token_ids) -> None:
        self.hash = h
        self.token_ids = list(token_ids)

    def reset(self) -> None:
        self.ref_count = 1
        self.hash = -1
        self.token_ids = []


class Sequence:
    """The block-manager view of one request (architecture page, "Sequenz-
    Status und Eigenschaften", "Block-Berechnung und Token-Appending")."""

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
        return (len(self) + self.block_size - 1) // self.block_size

    @property
    def num_cached_blocks(self) -> int:
        return self.num_cached_tokens // self.block_size

    @property
    def last_block_num_tokens(self) -> int:
        return len(self) - (self.num_blocks - 1) * self.block_size

    def block(self, i: int) -> list[int]:
        return self.token_ids[i * self.block_size:(i + 1) * self.block_size]

    def append_token(self, token_id: int) -> None:
        self.token_ids.append(int(token_id))


class BlockManager:
    """Block pool with reference counts and hash-based prefix sharing
    (architecture page, "Hash-basiertes Prefix Caching", "Dynamische
    Block-Erweiterung")."""

    def __init__(self, num_blocks: int, block_size: int):
        assert num_blocks >= 1 and block_size >= 2  # at 1 a token opens and fills a block
        self.block_size = block_size
        self.blocks = [Block(i) for i in range(num_blocks)]
        self.hash_to_block_id: dict[int, int] = {}
        self.free_block_ids: list[int] = list(range(num_blocks))  # front = index 0
        self.used_block_ids: set[int] = set()

    # -- single blocks ------------------------------------------------------
    def _allocate_block(self, block_id: int) -> Block:
        block = self.blocks[block_id]
        assert block.ref_count == 0
        block.reset()
        self.free_block_ids.remove(block_id)
        self.used_block_ids.add(block_id)
        return block

    def _deallocate_block(self, block_id: int) -> None:
        assert self.blocks[block_id].ref_count == 0
        self.used_block_ids.remove(block_id)
        self.free_block_ids.append(block_id)

    # -- sequences -------------------------------------------------------------
    def can_allocate(self, seq: Sequence) -> bool:
        return len(self.free_block_ids) >= seq.num_blocks  # H6

    def allocate(self, seq: Sequence) -> None:
        assert not seq.block_table
        h = -1
        missed = False
        for i in range(seq.num_blocks):
            token_ids = seq.block(i)
            h = compute_hash(token_ids, h) if len(token_ids) == self.block_size else -1
            block_id = self.hash_to_block_id.get(h, -1)
            if (block_id == -1 or self.blocks[block_id].hash != h  # H9
                    or self.blocks[block_id].token_ids != token_ids):
                missed = True  # H2: no hit after the first miss
            if missed:
                block = self._allocate_block(self.free_block_ids[0])  # H4
            else:
                seq.num_cached_tokens += self.block_size
                if block_id in self.used_block_ids:
                    block = self.blocks[block_id]
                    block.ref_count += 1
                else:  # H3: given back but still registered
                    block = self._allocate_block(block_id)
            if h != -1:
                block.update(h, token_ids)
                self.hash_to_block_id[h] = block.block_id
            seq.block_table.append(block.block_id)

    def deallocate(self, seq: Sequence) -> None:
        for block_id in reversed(seq.block_table):  # H5
            block = self.blocks[block_id]
            block.ref_count -= 1
            if block.ref_count == 0:
                self._deallocate_block(block_id)
        seq.num_cached_tokens = 0
        seq.block_table = []

    def can_append(self, seq: Sequence) -> bool:
        need = 1 if len(seq) % self.block_size == 1 else 0  # H6
        return len(self.free_block_ids) >= need

    def may_append(self, seq: Sequence) -> None:
        table = seq.block_table
        last = self.blocks[table[-1]]
        r = len(seq) % self.block_size
        if r == 1:  # the new token opens a block
            assert last.hash != -1
            block = self._allocate_block(self.free_block_ids[0])
            table.append(block.block_id)
        elif r == 0:  # the new token fills the last block (H7)
            assert last.hash == -1
            token_ids = seq.block(seq.num_blocks - 1)
            prefix = self.blocks[table[-2]].hash if len(table) > 1 else -1
            h = compute_hash(token_ids, prefix)
            last.update(h, token_ids)
            self.hash_to_block_id[h] = last.block_id
        else:
            assert last.hash == -1


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
