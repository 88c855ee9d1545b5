"""Block sizes other than 256 (16, 32 and multiples of 64 up to 4096, which
include every multiple of 256): store, decode, the fused decode step and the
paged prefill against the CPU oracle on the small parity cases re-drawn at
each block size, and a layout invariant -- the same logical K/V laid out in
blocks of another size give bitwise the outputs of the 256-token layout."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_325_amd as pkv
from tests.gpu_helpers import announce, assert_close, attend, check_inputs, store, to_device
from tests.oracle_helpers import expected, stored_bits
from workloads import Spec, bits_view, build, config, small_specs

pytestmark = pytest.mark.gpu

SIZES = [16, 32, 64, 128, 512, 768, 1024]


def at_block_size(spec, B):
    """The spec with blocks of B tokens; shared prefixes keep (at most) the
    same number of tokens, rounded down to whole blocks."""
    shared = None
    if spec.shared_blocks:
        shared = [min(s * 256 // B, (c - n) // B) for s, c, n in
                  zip(spec.shared_blocks, spec.context_lens, spec.new_tokens)]
    return dataclasses.replace(spec, name=f"{spec.name}-B{B}", block_size=B,
                               shared_blocks=shared, seed=spec.seed + B)


CASES = [(s, B) for B in SIZES for s in small_specs()
         if s.name in ("dec-bf16-g2-ragged", "dec-fp32-g2", "dec-bf16-shared", "dec-bf16-g8",
                       "dec-bf16-empty-ctx", "pre-bf16-g4", "pre-bf16-g2", "pre-bf16-g8")]


@pytest.mark.parametrize("spec,B", CASES, ids=[f"{s.name}-B{B}" for s, B in CASES])
def test_block_size_against_oracle(spec, B):
    w = build(at_block_size(spec, B))
    d = to_device(w)
    check_inputs(d)
    announce(f"block size {B}: {w.spec.name}")
    store(d)
    out = attend(d)
    torch.cuda.synchronize()
    kcb, vcb = stored_bits(w)
    assert np.array_equal(bits_view(d.k_cache.cpu()), kcb)
    assert np.array_equal(bits_view(d.v_cache.cpu()), vcb)
    assert_close(out.to(torch.float64).cpu().numpy(), expected(w), w.spec.name)
    if w.spec.mode == "decode":
        for splits in (1, 3):
            o2 = attend(d, num_splits=splits)
            torch.cuda.synchronize()
            assert_close(o2.to(torch.float64).cpu().numpy(), expected(w),
                         f"{w.spec.name} splits={splits}")


@pytest.mark.parametrize("B", [16, 32, 512])
@pytest.mark.parametrize("name", ["dec-bf16-g2-ragged", "dec-bf16-g8"])
def test_fused_step_at_block_size(name, B):
    # dec-bf16-g8: 8 query heads per workgroup, whose fused kernel at blocks
    # of 16 or 32 tokens reads the new row again in its last chunk
    spec = [s for s in small_specs() if s.name == name][0]
    w = build(at_block_size(spec, B))
    a, b = to_device(w), to_device(w)
    check_inputs(a)
    announce(f"fused step at block size {B}: {name}")
    store(a)
    ref_out = attend(a)
    out = pkv.pkv_paged_decode_step(b.q, b.k, b.v, b.slot_mapping, b.k_cache, b.v_cache,
                                    b.block_tables, b.context_lens, w.max_context_len, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))
    assert torch.equal(a.v_cache.view(torch.int16), b.v_cache.view(torch.int16))


def _relayout(w, B2, seed):
    """The post-store caches of w re-laid out in shuffled blocks of B2 tokens
    (logical rows of each sequence copied out; cells outside every context
    stay NaN), with matching tables."""
    kcb, vcb = stored_bits(w)
    B, batch = w.block_size, w.batch
    nb2 = [-(-int(c) // B2) for c in w.context_lens]
    pool = max(1, sum(nb2))
    perm = np.random.default_rng(seed).permutation(pool)
    nan = np.uint16(0x7FC1)
    k2 = np.full((pool, w.num_kv_heads, B2, w.head_dim), nan, np.uint16)
    v2 = np.full_like(k2, nan)
    tables = np.full((batch, max(1, max(nb2))), -1, np.int32)
    cur = 0
    for b in range(batch):
        n = int(w.context_lens[b])
        tables[b, :nb2[b]] = perm[cur:cur + nb2[b]]
        cur += nb2[b]
        pos = np.arange(n)
        src_blk = w.block_tables[b, pos // B].astype(np.int64)
        dst_blk = tables[b, pos // B2].astype(np.int64)
        k2[dst_blk, :, pos % B2] = kcb[src_blk, :, pos % B]
        v2[dst_blk, :, pos % B2] = vcb[src_blk, :, pos % B]
    return k2, v2, tables


def _t(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("B2", [16, 32, 64, 512, 1024])
@pytest.mark.parametrize("name", ["dec-bf16-g2-ragged", "dec-bf16-g4-long", "pre-bf16-g4",
                                  "pre-bf16-g2"])
def test_layout_invariance_bitwise(name, B2):
    spec = [s for s in small_specs() if s.name == name][0]
    w = build(spec)
    d = to_device(w)
    check_inputs(d)
    announce(f"layout invariance {name} at block size {B2}")
    store(d)
    ref_out = attend(d)
    k2, v2, tables = _relayout(w, B2, 77 + B2)
    kc, vc = _t(k2), _t(v2)
    tab = torch.from_numpy(tables).cuda()
    ctx = d.context_lens
    if spec.mode == "decode":
        out = pkv.pkv_paged_decode(d.q, kc, vc, tab, ctx, w.max_context_len, w.scale)
    else:
        out = pkv.pkv_paged_prefill_varlen(d.q, kc, vc, d.cu_seqlens_q, w.max_seqlen_q, ctx,
                                           w.max_context_len, tab, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))


@pytest.mark.parametrize("B2", [16, 1024])
@pytest.mark.parametrize("index", [2, 3])
def test_full_size_layout_invariance_bitwise(index, B2):
    # the 64-sequence decode and the prefill workload (checked against the
    # oracle in their 256-token layout by the parity tests) re-laid out in
    # blocks of 16 and 1024 tokens: outputs bitwise unchanged
    w = config(index)
    d = to_device(w)
    check_inputs(d)
    announce(f"full-size layout invariance, workload {index}, block size {B2}")
    store(d)
    ref_out = attend(d)
    k2, v2, tables = _relayout(w, B2, 99 + B2)
    kc, vc = _t(k2), _t(v2)
    del k2, v2
    tab = torch.from_numpy(tables).cuda()
    if w.spec.mode == "decode":
        # the same split plan (the cap binds at neither block size here)
        S = pkv.pkv_paged_decode_split_tokens(w.batch, w.num_q_heads, w.num_kv_heads, 128,
                                              w.max_context_len, 256, 0)
        assert S == pkv.pkv_paged_decode_split_tokens(w.batch, w.num_q_heads, w.num_kv_heads,
                                                      128, w.max_context_len, B2, 0)
        out = pkv.pkv_paged_decode(d.q, kc, vc, tab, d.context_lens, w.max_context_len, w.scale)
    else:
        out = pkv.pkv_paged_prefill_varlen(d.q, kc, vc, d.cu_seqlens_q, w.max_seqlen_q,
                                           d.context_lens, w.max_context_len, tab, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))


# (block size, requested splits, context lengths, q heads, kv heads).  With
# 16- or 32-token blocks a split is capped at 64 blocks (1024 / 2048 keys), so
# the plan differs from the one at 256-token blocks: a forced single split of
# a 4096-key context becomes 4 (or 2) splits, and the automatic plan of a
# 256-sequence batch with one 20000-key context (1024 units, splits of 2560
# keys at 256-token blocks) is capped as well.  The merge must plan with the
# caches' block size, or the rows of split sequences are never written.
_LONG_AUTO = [20000, 9000, 3000] + [int(x) for x in
                                    np.random.default_rng(9301).integers(1, 400, 253)]
TWO_CALL_CASES = [
    (16, 1, [4096, 1500, 700, 2049, 1], 8, 2),
    (32, 1, [4096, 1500, 700, 2049, 1], 8, 2),
    (16, 0, _LONG_AUTO, 8, 4),
    (32, 0, _LONG_AUTO, 8, 4),
]


@pytest.mark.parametrize("B,splits,ctx,hq,hkv", TWO_CALL_CASES,
                         ids=[f"B{c[0]}-splits{c[1]}-batch{len(c[2])}" for c in TWO_CALL_CASES])
def test_two_call_decode_plans_with_block_size(B, splits, ctx, hq, hkv):
    """pkv_paged_decode_partials then pkv_paged_decode_merge through the
    binding at small blocks: bitwise equal to the one-call decode, every
    output row written, and within tolerance of the oracle."""
    w = build(Spec(f"two-call-B{B}-s{splits}", "decode", "bf16", hq, hkv, ctx, [1] * len(ctx),
                   9300 + B + splits, block_size=B))
    args = (w.batch, hq, hkv, 128, w.max_context_len)
    here = pkv.pkv_paged_decode_split_tokens(*args, B, splits)
    at256 = pkv.pkv_paged_decode_split_tokens(*args, 256, splits)
    assert here < at256 and here < w.max_context_len, (here, at256)
    d = to_device(w)
    check_inputs(d)
    announce(f"two-call decode at block size {B}, splits {splits}: store + one-call decode")
    store(d)
    whole = attend(d, num_splits=splits)
    announce(f"two-call decode at block size {B}, splits {splits}: partials + merge")
    out = torch.full_like(whole, float("nan"))
    out, ws = pkv.pkv_paged_decode_partials(d.q, d.k_cache, d.v_cache, d.block_tables,
                                            d.context_lens, w.max_context_len, w.scale,
                                            out=out, num_splits=splits)
    pkv.pkv_paged_decode_merge(d.context_lens, w.max_context_len, hq, hkv, B, out, ws,
                               num_splits=splits)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any(), "rows left unwritten by partials + merge"
    assert torch.equal(whole.view(torch.int16), out.view(torch.int16))
    assert_close(out.double().cpu().numpy(), expected(w), w.spec.name)
