"""CPU pins of the shared-prefix plan oracle (``oracle/prefix_plan.py``).

The plan is this library's own rule (the pages fix only that equal leading
table entries are the same physical K/V: nano-vllm architecture page,
"Hash-basiertes Prefix Caching").  It is pinned by:
  * a hand-worked example (``tests/golden/prefix_plan_example.json``, the
    working written out in the file);
  * brute-force checks of what makes a plan correct, on seeded random
    batches with prefix trees: every key of a shared split lies in the same
    physical block for all members and before each member's last position;
    no sequence is in two subgroups; skip counts match the items;
  * brute-force maximality: one more split would break one of those;
  * planted mistakes: each plausible error in the oracle fails one of the
    above.
"""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

from oracle import prefix_plan as pp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefix_plan_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_example():
    d = _golden()
    for c in d["cases"]:
        got = pp.prefix_plan(d["block_tables"], d["context_lens"], d["block_size"], c["group"],
                             c["split_tokens"])
        assert got == c["words"], (c["group"], c["split_tokens"])


def random_batch(seed: int, block_size: int, split: int):
    """A decode batch whose tables share prefixes the way hash-based prefix
    caching makes them: a few prompt trees (a chain of shared blocks, with
    branches that share a shorter part), private blocks after the shared
    part, context lengths that often sit on multiples of the split length;
    plus some whole-table copies, which share the block of the last
    position as well."""
    rng = np.random.default_rng(seed)
    batch = int(rng.integers(2, 24))
    next_id = [0]

    def fresh(n):
        ids = list(range(next_id[0], next_id[0] + n))
        next_id[0] += n
        return ids

    trees = []
    for _ in range(int(rng.integers(1, 4))):
        trunk = fresh(int(rng.integers(1, 12)))
        branches = [trunk[: int(rng.integers(0, len(trunk) + 1))] + fresh(int(rng.integers(0, 6)))
                    for _ in range(int(rng.integers(1, 4)))]
        trees.append(branches)
    tables, ctx = [], []
    for _ in range(batch):
        if tables and rng.random() < 0.15:
            # a copy of an earlier sequence's table, the block of its last
            # position included (identical block ids are identical K/V to
            # the plan), with the same or a shorter context
            src = int(rng.integers(len(tables)))
            n = ctx[src] if rng.random() < 0.5 else int(rng.integers(1, ctx[src] + 1))
            tables.append(tables[src][: -(-n // block_size)])
            ctx.append(n)
            continue
        if rng.random() < 0.15:
            shared = []
        else:
            tree = trees[int(rng.integers(len(trees)))]
            shared = tree[int(rng.integers(len(tree)))]
        choice = rng.random()
        if choice < 0.3:
            n = int(rng.integers(1, 4)) * split + int(rng.integers(0, 2))  # on / just past S
        elif choice < 0.4:
            n = int(rng.integers(1, split + 2))
        else:
            n = int(rng.integers(1, (len(shared) + 4) * block_size + 1))
        # the shared blocks are full blocks before the last position
        full = (n - 1) // block_size
        nblk = -(-n // block_size)
        row = shared[:full] + fresh(nblk - min(full, len(shared)))
        tables.append(row[:nblk])
        ctx.append(n)
    width = max(len(r) for r in tables)
    tables = [r + [-1] * (width - len(r)) for r in tables]
    return tables, ctx


def shareable(tables, ctx, members, s, B, S) -> bool:
    """Brute force: keys s*S .. (s+1)*S - 1 of every member lie before its
    last position and in the same physical block for all members."""
    for b in members:
        if (s + 1) * S > ctx[b] - 1:
            return False
    for j in range(s * S, (s + 1) * S):
        ids = {tables[b][j // B] for b in members}
        if len(ids) != 1:
            return False
    return True


def check_plan(words, tables, ctx, B, group, S):
    """Every property a plan must have; raises AssertionError otherwise."""
    S_, batch, skip, subgroups, items = pp.decode_plan(words)
    assert S_ == S and batch == len(ctx)
    R = pp.MEMBER_SLOTS // group
    seen = set()
    for members in subgroups:
        assert 2 <= len(members) <= R
        assert len(set(members)) == len(members)
        assert not (seen & set(members))
        seen |= set(members)
    per_sub = {}
    for p, s in items:
        assert 0 <= p < len(subgroups)
        per_sub.setdefault(p, []).append(s)
        assert shareable(tables, ctx, subgroups[p], s, B, S), (p, s)
    for p, members in enumerate(subgroups):
        ks = per_sub.get(p, [])
        assert ks == list(range(len(ks))) and ks, p
        for b in members:
            assert skip[b] == len(ks)
        # maximal: the next split cannot be shared by this run
        assert not shareable(tables, ctx, members, len(ks), B, S), p
    for b in range(batch):
        if b not in seen:
            assert skip[b] == 0


CASES = [(seed, B, S, G) for seed, (B, S, G) in enumerate(
    [(16, 64, 4), (16, 64, 2), (16, 128, 8), (32, 64, 1), (64, 64, 4), (256, 256, 4),
     (256, 512, 4), (16, 256, 4), (64, 128, 2), (512, 256, 8)] * 6)]


@pytest.mark.parametrize("seed,B,S,G", CASES)
def test_random_plans_are_correct_and_maximal(seed, B, S, G):
    tables, ctx = random_batch(1000 + seed, B, S)
    words = pp.prefix_plan(tables, ctx, B, G, S)
    assert len(words) <= pp.plan_words_bound(len(ctx), max(ctx), S)
    check_plan(words, tables, ctx, B, G, S)


def test_random_plans_share_something():
    # the generator makes sharing common: most batches yield a subgroup
    hits = 0
    for seed, B, S, G in CASES:
        tables, ctx = random_batch(1000 + seed, B, S)
        hits += pp.prefix_plan(tables, ctx, B, G, S)[1] > 0
    assert hits > len(CASES) // 3


def test_groups_above_eight_share_nothing():
    tables, ctx = random_batch(7, 16, 64)
    for G in (16, 32):
        words = pp.prefix_plan(tables, ctx, 16, G, 64)
        assert words[1] == 0 and words[4] == 0 and words[5:] == [0] * len(ctx)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

def _random_failures():
    bad = 0
    for seed, B, S, G in CASES:
        tables, ctx = random_batch(1000 + seed, B, S)
        try:
            check_plan(pp.prefix_plan(tables, ctx, B, G, S), tables, ctx, B, G, S)
        except AssertionError:
            bad += 1
    return bad


def test_planted_mistakes_are_caught(monkeypatch):
    assert _random_failures() == 0
    with monkeypatch.context() as m:  # one block too many counted as common
        orig = pp.common_prefix
        m.setattr(pp, "common_prefix", lambda rows: orig(rows) + 1)
        assert _random_failures() > 0
    with monkeypatch.context() as m:  # the last position counted as shareable
        m.setattr(pp, "shared_splits",
                  lambda lcp, B, ctxs, S: min(lcp * B, min(ctxs)) // S)
        assert _random_failures() > 0
    with monkeypatch.context() as m:  # the block of the last position compared too
        m.setattr(pp, "needed_blocks", lambda n, B: -(-n // B))
        with pytest.raises(AssertionError):
            test_worked_example()
    with monkeypatch.context() as m:  # a split short of the maximum
        orig_k = pp.shared_splits
        m.setattr(pp, "shared_splits", lambda *a: max(orig_k(*a) - 1, 0))
        assert _random_failures() > 0
    with monkeypatch.context() as m:  # members left in batch order (no sort)
        m.setattr(pp, "sorted", lambda xs, key=None: list(xs), raising=False)
        with pytest.raises(AssertionError):
            test_worked_example()
