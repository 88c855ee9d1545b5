"""GPU: the shared-prefix decode (pkv_paged_decode_prefix and the fused
pkv_paged_decode_step_prefix) against the fp64 oracle.

Sequences whose tables begin with the same physical blocks (architecture
page, "Hash-basiertes Prefix Caching": a cached full prompt block is shared
by id) have those splits attended once per subgroup on MFMA and merged with
their private splits.  The attention is the same, so the oracle is the plain
decode (oracle/ref.py) of the post-store cache; the plan words the library
builds are compared with oracle/prefix_plan.py first.  Cases: GQA groups 1,
2, 4 and 8 (16, 8, 4 and 2 members per subgroup), block sizes 16, 32, 64,
256 and 512, the automatic split plan and forced ones, classes larger than
one subgroup, the full prefix-shared long-context workload; a plan built for
other tables (NaN rows for the subgroup, the rest exact), and plans that do
not match the call (ignored: bitwise the plain decode)."""

from __future__ import annotations


import numpy as np
import pytest
import torch

import paged_kv_cache_325_amd as pkv
from oracle import prefix_plan as pp
from oracle import ref
from tests.gpu_helpers import announce, assert_close, check_inputs, store, to_device
from tests.oracle_helpers import expected, q64, sequence_view, stored_bits
from workloads import Spec, bits_view, build, config

pytestmark = pytest.mark.gpu


def _split_tokens(w, num_splits):
    return pkv.pkv_paged_decode_split_tokens(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                             w.max_context_len, w.block_size, num_splits)


def _plan(w, num_splits):
    """The library's plan for the workload's host tables, checked word for
    word against the oracle's, on the GPU."""
    S = _split_tokens(w, num_splits)
    plan, items = pkv.pkv_decode_prefix_plan(w.block_tables, w.context_lens, w.num_q_heads,
                                             w.num_kv_heads, w.block_size, S)
    want = pp.prefix_plan(w.block_tables.tolist(), w.context_lens.tolist(), w.block_size,
                          w.num_q_heads // w.num_kv_heads, S)
    assert plan.tolist() == want
    return plan.cuda(), items, S


def _spec(name, hq, hkv, ctx, groups, shared, seed, block_size=256):
    return Spec(name, "decode", "bf16", hq, hkv, ctx, [1] * len(ctx), seed, share_group=groups,
                shared_blocks=shared, block_size=block_size)


# (spec, forced split counts); shared_blocks count blocks of the spec's size
CASES = [
    # G = 4: a subgroup of 4 and one of 2; two unshared sequences
    (_spec("pfx-g4", 8, 2, [3000, 2600, 4100, 3333, 700, 900, 5000, 1500],
           [0, 0, 0, 0, 1, 1, -1, -1], [8, 8, 8, 8, 2, 2, 0, 0], 9701), [0, 8, 40]),
    # G = 1: 18 sequences of one class -> runs of 16 and 2
    (_spec("pfx-g1", 2, 2, [1200 + 37 * b for b in range(18)], [0] * 18, [4] * 18, 9702),
     [0, 10]),
    # G = 2, 16-token blocks: long shared runs of small blocks
    (_spec("pfx-g2-b16", 4, 2, [900, 1000, 777, 1300, 650, 640],
           [0, 0, 0, 1, 1, -1], [40, 40, 40, 30, 30, 0], 9703, block_size=16), [0, 6]),
    # G = 8: runs of 2; a class of 5 -> 2 + 2 + (1 dropped)
    (_spec("pfx-g8", 8, 1, [2000, 2100, 1900, 2500, 2222, 3000],
           [0, 0, 0, 0, 0, -1], [6, 6, 6, 6, 6, 0], 9704), [0, 12]),
    # G = 5: runs of 3 (15 of the 16 columns)
    (_spec("pfx-g5", 10, 2, [1800, 1900, 2000, 1700, 2100], [0, 0, 0, 1, 1], [5, 5, 5, 4, 4],
           9709), [0, 9]),
    # G = 8 with 16-token blocks (the fused kernel re-reads the new row)
    (_spec("pfx-g8-b16", 8, 1, [1300, 1250, 1400, 1100], [0, 0, 1, 1], [50, 50, 40, 40], 9708,
           block_size=16), [0, 6]),
    # 32-token blocks and 64-token blocks
    (_spec("pfx-g4-b32", 8, 2, [1100, 1000, 1200, 600], [0, 0, 0, -1], [20, 20, 20, 0], 9705,
           block_size=32), [0, 5]),
    (_spec("pfx-g4-b64", 8, 2, [1500, 1400, 1300, 1700], [0, 0, 1, 1], [10, 10, 12, 12], 9706,
           block_size=64), [0, 7]),
    # 512-token blocks: splits shorter than a block
    (_spec("pfx-g4-b512", 8, 2, [3000, 2900, 2000, 3100], [0, 0, 0, 0], [3, 3, 3, 3], 9707,
           block_size=512), [0, 12]),
]
PARAMS = [(spec, n) for spec, splits in CASES for n in splits]


@pytest.mark.parametrize("spec,num_splits", PARAMS,
                         ids=[f"{s.name}-splits{n}" for s, n in PARAMS])
def test_prefix_decode_matches_oracle(spec, num_splits):
    w = build(spec)
    d = to_device(w)
    check_inputs(d)
    plan, items, S = _plan(w, num_splits)
    if num_splits == 0 or S < 1024:
        assert items > 0, f"nothing shared at split length {S}"
    want = expected(w)
    kcb, vcb = stored_bits(w)
    k_pre, v_pre = d.k_cache.clone(), d.v_cache.clone()

    announce(f"{spec.name} splits {num_splits} (S {S}, {items} items): fused step with plan")
    out_step = pkv.pkv_paged_decode_step_prefix(
        d.q, d.k, d.v, d.slot_mapping, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
        w.max_context_len, w.scale, plan, items, num_splits=num_splits)
    torch.cuda.synchronize()
    assert np.array_equal(bits_view(d.k_cache.cpu()), kcb)
    assert np.array_equal(bits_view(d.v_cache.cpu()), vcb)
    assert_close(out_step.double().cpu().numpy(), want, f"{spec.name} fused step with plan")

    announce(f"{spec.name} splits {num_splits}: store, then decode with plan")
    d.k_cache.copy_(k_pre)
    d.v_cache.copy_(v_pre)
    store(d)
    out = pkv.pkv_paged_decode_prefix(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                      w.max_context_len, w.scale, plan, items,
                                      num_splits=num_splits)
    plain = pkv.pkv_paged_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                 w.max_context_len, w.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    assert_close(got, want, f"{spec.name} decode with plan")
    # the fused form computes the same splits the same way
    assert torch.equal(out.view(torch.int16), out_step.view(torch.int16))
    # sequences outside every subgroup are untouched by the plan: bitwise
    # the plain decode
    _, _, skip, _, _ = pp.decode_plan(plan.cpu().tolist())
    alone = [b for b in range(w.batch) if skip[b] == 0]
    if alone:
        assert torch.equal(out[alone].view(torch.int16), plain[alone].view(torch.int16))
    # and the shared splits really ran on the MFMA path: its bf16
    # probabilities round differently from the plain decode's fp32 ones
    grouped = [b for b in range(w.batch) if skip[b] > 0]
    if grouped:
        assert not torch.equal(out[grouped].view(torch.int16), plain[grouped].view(torch.int16))


def test_prefix_decode_without_items_is_the_plain_decode():
    spec = CASES[0][0]
    w = build(spec)
    d = to_device(w)
    check_inputs(d)
    store(d)
    announce("plan without items / no plan: plain decode")
    plain = pkv.pkv_paged_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                 w.max_context_len, w.scale)
    empty = pkv.pkv_paged_decode_prefix(d.q, d.k_cache, d.v_cache, d.block_tables,
                                        d.context_lens, w.max_context_len, w.scale, None, 0)
    torch.cuda.synchronize()
    assert torch.equal(empty.view(torch.int16), plain.view(torch.int16))


def test_plan_for_another_call_is_ignored():
    """A plan whose header does not match the call (another split length,
    another batch size) is ignored: bitwise the plain decode."""
    spec = CASES[0][0]
    w = build(spec)
    d = to_device(w)
    check_inputs(d)
    store(d)
    plan, items, S = _plan(w, 8)
    S_other = _split_tokens(w, 40)
    assert S_other != S
    announce("plan built for another split length")
    plain = pkv.pkv_paged_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                 w.max_context_len, w.scale, num_splits=40)
    other = pkv.pkv_paged_decode_prefix(d.q, d.k_cache, d.v_cache, d.block_tables,
                                        d.context_lens, w.max_context_len, w.scale, plan, items,
                                        num_splits=40)
    torch.cuda.synchronize()
    assert torch.equal(other.view(torch.int16), plain.view(torch.int16))
    announce("plan with a different batch word")
    bad = plan.clone()
    bad[2] += 1
    other = pkv.pkv_paged_decode_prefix(d.q, d.k_cache, d.v_cache, d.block_tables,
                                        d.context_lens, w.max_context_len, w.scale, bad, items,
                                        num_splits=8)
    plain8 = pkv.pkv_paged_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                  w.max_context_len, w.scale, num_splits=8)
    torch.cuda.synchronize()
    assert torch.equal(other.view(torch.int16), plain8.view(torch.int16))


def test_plan_for_other_tables_gives_nan_rows():
    """The plan claims sharing that the tables passed no longer have (one
    member's shared blocks moved to private copies of the same K/V): the
    kernel's check turns that subgroup's rows into NaN; every other row is
    still the oracle's."""
    spec = CASES[0][0]
    w = build(spec)
    d = to_device(w)
    check_inputs(d)
    store(d)
    plan, items, S = _plan(w, 8)
    _, _, skip, subgroups, _ = pp.decode_plan(plan.cpu().tolist())
    victim_group = subgroups[0]
    b = victim_group[1]
    bt = w.block_tables.copy()
    nshared = -(-skip[b] * S // w.block_size)  # the blocks of its shared splits
    ids = [int(x) for x in bt[b, :nshared]]
    extra = torch.tensor(ids, device="cuda", dtype=torch.long)
    kc2 = torch.cat([d.k_cache, d.k_cache[extra]]).contiguous()
    vc2 = torch.cat([d.v_cache, d.v_cache[extra]]).contiguous()
    bt[b, :nshared] = np.arange(w.num_blocks, w.num_blocks + nshared)
    bt_d = torch.from_numpy(bt).cuda()
    announce("plan built for other tables")
    out = pkv.pkv_paged_decode_prefix(d.q, kc2, vc2, bt_d, d.context_lens, w.max_context_len,
                                      w.scale, plan, items, num_splits=8)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    assert np.isnan(got[victim_group]).all()
    rest = [x for x in range(w.batch) if x not in victim_group]
    assert_close(got[rest], expected(w)[rest], "rows outside the broken subgroup")


def test_prefix_shared_workload_full_size():
    """The prefix-shared long-context workload (16 sequences, groups of 4
    sharing a 4096-token prefix) at full size with the automatic split plan:
    every sequence against the oracle, for the decode and the fused step."""
    w = config(5)
    d = to_device(w)
    check_inputs(d)
    plan, items, S = _plan(w, 0)
    assert items > 0
    k_pre, v_pre = d.k_cache.clone(), d.v_cache.clone()
    announce(f"prefix-shared workload: fused step with plan ({items} items, S {S})")
    out_step = pkv.pkv_paged_decode_step_prefix(
        d.q, d.k, d.v, d.slot_mapping, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
        w.max_context_len, w.scale, plan, items)
    torch.cuda.synchronize()
    d.k_cache.copy_(k_pre)
    d.v_cache.copy_(v_pre)
    del k_pre, v_pre
    announce("prefix-shared workload: store, then decode with plan")
    store(d)
    out = pkv.pkv_paged_decode_prefix(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                      w.max_context_len, w.scale, plan, items)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_step.view(torch.int16))
    got = out.double().cpu().numpy()
    del d
    torch.cuda.empty_cache()
    kcb, vcb = stored_bits(w)
    q = q64(w)
    worst = 0.0
    for b in range(w.batch):
        kc, vc, row = sequence_view(w, kcb, vcb, b)
        want = ref.decode(q[b : b + 1], kc, vc, row[None, :], w.context_lens[b : b + 1], w.scale)
        assert_close(got[b : b + 1], want, f"prefix-shared workload sequence {b}")
        worst = max(worst, float(np.abs(got[b : b + 1] - want).max()))
    announce(f"prefix-shared workload with plan: all {w.batch} sequences within tolerance "
             f"(worst max-abs {worst:.3g})")
