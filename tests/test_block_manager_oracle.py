"""Pins of the CPU block-manager oracle against facts that do not come from
it: the published FNV-1a test vectors, the byte layout of the chained hash
written out by hand, a hand-worked scenario (tests/golden/), invariants over
seeded request streams, and a collision case whose outcome is derived by
hand.  The last group plants plausible mistakes in the oracle and checks that
a pin catches each one."""

from __future__ import annotations

import pytest

from oracle import block_manager as bm
from tests.bm_scenario import OracleAdapter, run_golden, run_stream
from workloads.requests import request_stream


# ---------------------------------------------------------------------------
# the hash
# ---------------------------------------------------------------------------

def test_fnv1a64_published_vectors():
    # test vectors published with the FNV definition (Fowler, Noll, Vo)
    assert bm.fnv1a64(b"") == 0xCBF29CE484222325
    assert bm.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert bm.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_hash_byte_layout():
    # first block: tokens only, int32 little-endian
    assert bm.block_hash_bytes([1, 256, -1], -1) == bytes(
        [1, 0, 0, 0, 0, 1, 0, 0, 0xFF, 0xFF, 0xFF, 0xFF])
    # later block: the previous hash as 8 little-endian bytes first
    assert bm.block_hash_bytes([7], 0x0102030405060708) == bytes(
        [8, 7, 6, 5, 4, 3, 2, 1, 7, 0, 0, 0])
    # the top bit is cleared, so no hash equals the -1 sentinel
    for p in (-1, 0, 12345):
        h = bm.compute_hash([3, 1, 4, 1], p)
        assert 0 <= h < 2 ** 63
    # "a" is byte 0x61: one token 0x61 hashes 4 bytes, not 1
    assert bm.compute_hash([0x61], -1) != bm.fnv1a64(b"a") & (2 ** 63 - 1)
    assert bm.compute_hash([0x61], -1) == bm.fnv1a64(b"a\0\0\0") & (2 ** 63 - 1)


# ---------------------------------------------------------------------------
# the hand-worked scenario
# ---------------------------------------------------------------------------

def test_golden_scenario():
    run_golden(OracleAdapter)


def test_collision_does_not_cache_a_non_prefix_block(monkeypatch):
    # Reading H2 under hash collisions: with a hash that depends only on the
    # block index, Y's first block finds X's first block (different tokens:
    # miss) and its second block finds X's second block (equal tokens).
    # Cached tokens must form a prefix, so Y caches nothing and takes two new
    # blocks (2 and 3 from the free list [2, 3]).
    monkeypatch.setattr(bm, "compute_hash", lambda toks, prefix=-1: prefix + 1)
    a = OracleAdapter(4, 4)
    a.add("X", [1, 2, 3, 4, 5, 6, 7, 8])
    a.allocate("X")
    a.add("Y", [9, 9, 9, 9, 5, 6, 7, 8])
    a.allocate("Y")
    assert a.table("X") == [0, 1]
    assert a.cached("Y") == 0 and a.table("Y") == [2, 3]
    assert [a.block(b)[0] for b in range(4)] == [1, 1, 1, 1]


# ---------------------------------------------------------------------------
# invariants over seeded request streams
# ---------------------------------------------------------------------------

def _check_invariants(kind, batch, adapters):
    a = adapters[0]
    B = a.block_size
    live = {s: seq for s, seq in a.seqs.items() if seq.block_table}
    counts = {}
    for seq in live.values():
        for b in seq.block_table:
            counts[b] = counts.get(b, 0) + 1
    free = a.free()
    assert len(free) == len(set(free))
    for b in range(len(a.bm.count)):
        assert a.bm.count[b] == counts.get(b, 0), f"block {b} count"
        assert (a.bm.count[b] == 0) == (b in free), f"block {b} free-list membership"
    # sequences of this step have had their table brought up to their length
    # (allocate or may_append); the other running ones hold a sampled token
    # that their next decode step's may_append will place
    for seq in (a.seqs[s] for s in batch):
        nb = seq.num_blocks
        assert len(seq.block_table) == nb
        assert seq.num_cached_tokens % B == 0 and seq.num_cached_tokens <= len(seq)
        prefix = -1
        for i, b in enumerate(seq.block_table[:-1] if len(seq) % B else seq.block_table):
            h = bm.fnv1a64(bm.block_hash_bytes(seq.block(i), prefix)) & (2 ** 63 - 1)
            assert a.bm.recorded[b] is not None, "a full block is registered"
            assert list(a.bm.recorded[b][1]) == seq.block(i), "a full block records its tokens"
            assert a.bm.recorded[b][0] == h, \
                "a full block carries the chained hash of its sequence"
            prefix = h
    if kind == "decode":
        for s in batch:  # the block holding the decoded token is private
            assert a.bm.count[a.seqs[s].block_table[-1]] == 1


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_invariants_over_request_streams(seed):
    B, N = 4, 14
    reqs = request_stream(seed, 30, B, vocab=6, max_suffix=9, max_decode=10)
    a = OracleAdapter(N, B)
    stats = run_stream([a], reqs, seed, N, on_step=_check_invariants)
    # the streams exercise sharing, reuse of freed cached blocks and preemption
    assert stats["cached_tokens"] > 0 and stats["freed_hits"] > 0
    assert stats["preemptions"] > 0
    assert stats["finished"] == len(reqs)


# ---------------------------------------------------------------------------
# planted mistakes: each plausible error in the oracle fails a pin above
# ---------------------------------------------------------------------------

def _fails(fn):
    with pytest.raises(AssertionError):
        fn()


def test_planted_mistakes_are_caught(monkeypatch):
    cls = bm.BlockManager
    orig_allocate = cls.allocate

    # 1. hash not chained on the previous block
    with monkeypatch.context() as m:
        real = bm.compute_hash
        m.setattr(bm, "compute_hash", lambda toks, prefix=-1: real(toks, -1))
        _fails(test_golden_scenario)

    # 2. hit tested on tokens only (reading H9 dropped)
    with monkeypatch.context() as m:
        m.setattr(cls, "_holds", lambda self, b, h, toks: self.recorded[b] is not None
                  and self.recorded[b][1] == tuple(toks))
        _fails(test_golden_scenario)

    # 3. no miss-latch: hits allowed after a miss (reading H2 dropped)
    def hits_anywhere(self, seq, hashes):
        return [h != -1 and self.index.get(h) is not None
                and self._holds(self.index[h], h, seq.block(i)) for i, h in enumerate(hashes)]

    with monkeypatch.context() as m:
        m.setattr(cls, "cache_hits", hits_anywhere)
        _fails(lambda: test_collision_does_not_cache_a_non_prefix_block(m))

    # 4. deallocate first-to-last instead of last-to-first
    def deallocate_forward(self, seq):
        for b in seq.block_table:
            self.count[b] -= 1
            if self.count[b] == 0:
                self.free.append(b)
        seq.num_cached_tokens = 0
        seq.block_table = []

    with monkeypatch.context() as m:
        m.setattr(cls, "deallocate", deallocate_forward)
        _fails(test_golden_scenario)

    # 5. a miss takes the back of the free list
    with monkeypatch.context() as m:
        def alloc_back(self, seq):
            self.free.reverse()
            try:
                orig_allocate(self, seq)
            finally:
                self.free.reverse()
        m.setattr(cls, "allocate", alloc_back)
        _fails(test_golden_scenario)

    # 6. a hit on a freed block is counted but left in the free list
    def take_in_place(self, b):
        self.count[b] += 1

    with monkeypatch.context() as m:
        m.setattr(cls, "_take", take_in_place)
        _fails(test_golden_scenario)

    # 7. may_append opens a block when the last one fills (off by one)
    def may_append_off(self, seq):
        if len(seq) % self.block_size == 0:
            seq.block_table.append(self._fresh())

    with monkeypatch.context() as m:
        m.setattr(cls, "may_append", may_append_off)
        _fails(test_golden_scenario)

    # 8. decode slot one row too far
    with monkeypatch.context() as m:
        real_dec = bm.prepare_decode

        def dec_off(seqs, width):
            d = real_dec(seqs, width)
            d["slot_mapping"] = [s + 1 for s in d["slot_mapping"]]
            return d
        m.setattr(bm, "prepare_decode", dec_off)
        _fails(test_golden_scenario)

    # 9. prefill slots written from the first block, not the first uncached one
    with monkeypatch.context() as m:
        real_pre = bm.prepare_prefill

        def pre_off(seqs, width):
            d = real_pre(seqs, width)
            slots = []
            for s in seqs:
                n_unc = len(s) - s.num_cached_tokens
                slots += [s.block_table[p // s.block_size] * s.block_size + p % s.block_size
                          for p in range(n_unc)]
            d["slot_mapping"] = slots
            return d
        m.setattr(bm, "prepare_prefill", pre_off)
        _fails(test_golden_scenario)

    # 10. can_append asks for a block when the last one is full (len % B == 0)
    with monkeypatch.context() as m:
        m.setattr(cls, "can_append",
                  lambda self, seq: len(self.free) >= (len(seq) % self.block_size == 0))
        _fails(test_golden_scenario)

    # 11. a freed block forgets its registration (reading H5: it keeps it)
    with monkeypatch.context() as m:
        orig_dealloc = cls.deallocate

        def dealloc_forget(self, seq):
            held = list(seq.block_table)
            orig_dealloc(self, seq)
            for b in held:
                if self.count[b] == 0:
                    self.recorded[b] = None
        m.setattr(cls, "deallocate", dealloc_forget)
        _fails(test_golden_scenario)

    # the unpatched oracle still passes
    test_golden_scenario()
