"""GPU parity on seeded random shapes: each case draws the mode (decode or
prefill), the dtype, the GQA group (odd and above 8 included), the cache
block size, the batch, ragged and empty lengths, shared prefixes, skipped
stores, table padding, the softmax scale (negative and zero included) and
the decode split count from its seed, then checks the store bit-exact and
attention against the CPU oracle within the parity tolerance.  Decode
batches where every sequence stores a token also run the one-call fused
step (bitwise the two calls); prefill cases also run the prefill over the
same keys gathered into contiguous rows (bitwise the paged prefill).  A
second set draws batches whose tables share prefix blocks in several
classes and runs the shared-prefix decode with the host planner's plan (the
plan word for word against the oracle's, attention against the oracle, the
fused form bitwise the two-call form).  The fixed cases elsewhere cover each
feature on its own; these cover them in combination."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_325_amd as pkv
from oracle import prefix_plan as pp
from tests.gpu_helpers import announce, assert_close, attend, check_inputs, store, to_device
from tests.oracle_helpers import expected, stored_bits
from workloads import Spec, bits_view, build

pytestmark = pytest.mark.gpu

BLOCK_SIZES = [16, 32, 64, 128, 192, 256, 512, 1024]
SEEDS = list(range(80))


def random_spec(seed: int) -> tuple[Spec, int]:
    """A small random case (the oracle finishes it in well under a second)
    and the decode split count to use (0: the automatic plan)."""
    r = np.random.default_rng(32_500 + seed)
    mode = "decode" if r.random() < 0.55 else "prefill"
    dtype = "fp32" if mode == "decode" and r.random() < 0.25 else "bf16"
    group = int(r.choice([1, 2, 3, 4, 5, 6, 8, 12, 16]))
    hkv = int(r.choice([1, 2]))
    B = int(r.choice(BLOCK_SIZES))
    batch = int(r.integers(1, 8))
    ctx, new = [], []
    for _ in range(batch):
        if mode == "decode":
            c = int(r.choice([0, 1, 2, int(r.integers(3, 400)), int(r.integers(400, 3000))],
                             p=[0.05, 0.1, 0.05, 0.4, 0.4]))
            ctx.append(c)
            new.append(1 if c > 0 else 0)
        else:
            c = int(r.integers(1, 1800))
            kind = r.random()
            n = c if kind < 0.35 else (0 if kind < 0.45 else (1 if kind < 0.55 else int(r.integers(1, c + 1))))
            ctx.append(c)
            new.append(n)
    # a shared prefix for a pair of neighbours, in whole blocks before both
    # sequences' stored rows
    share_group = shared_blocks = None
    if batch >= 2 and r.random() < 0.3:
        b0 = int(r.integers(0, batch - 1))
        room = min((ctx[b0] - new[b0]) // B, (ctx[b0 + 1] - new[b0 + 1]) // B)
        if room >= 1:
            k = int(r.integers(1, room + 1))
            share_group = [-1] * batch
            shared_blocks = [0] * batch
            share_group[b0] = share_group[b0 + 1] = 0
            shared_blocks[b0] = shared_blocks[b0 + 1] = k
    n_new = sum(new)
    skip = [int(r.integers(0, n_new))] if n_new > 1 and r.random() < 0.2 else []
    scale = None
    u = r.random()
    if u < 0.1:
        scale = -0.09
    elif u < 0.15:
        scale = 0.0
    elif u < 0.25:
        scale = float(r.uniform(0.2, 0.5))
    q_scale = 4.0 if r.random() < 0.15 else 1.0
    pad = int(r.integers(0, 3))
    splits = int(r.choice([0, 0, 1, 2, 3, 5, 8, 24, 40])) if mode == "decode" else 0
    # an all-empty batch still gets a (poisoned) one-block cache: a cache of
    # no blocks has no storage, and the library refuses a null cache with
    # token rows to store (even rows whose slot is -1)
    pool = 1 if sum(ctx) == 0 else None
    spec = Spec(f"rand{seed}-{mode}-{dtype}-g{group}x{hkv}-B{B}-b{batch}", mode, dtype,
                group * hkv, hkv, ctx, new, 33_000 + seed, skip=skip, share_group=share_group,
                shared_blocks=shared_blocks, block_size=B, scale=scale, q_scale=q_scale,
                pad_columns=pad, pool_blocks=pool)
    return spec, splits


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_against_oracle(seed):
    spec, splits = random_spec(seed)
    w = build(spec)
    d = to_device(w)
    check_inputs(d)
    announce(f"{spec.name} (splits {splits}): store")
    store(d)
    announce(f"{spec.name}: attention")
    out = attend(d, num_splits=splits)
    torch.cuda.synchronize()
    kcb, vcb = stored_bits(w)
    assert np.array_equal(bits_view(d.k_cache.cpu()), kcb), "k_cache differs from the oracle store"
    assert np.array_equal(bits_view(d.v_cache.cpu()), vcb), "v_cache differs from the oracle store"
    assert_close(out.to(torch.float64).cpu().numpy(), expected(w), spec.name)

    if spec.mode == "decode" and all(n == 1 for n in spec.new_tokens):
        e = to_device(w)
        announce(f"{spec.name}: fused step")
        fused = pkv.pkv_paged_decode_step(e.q, e.k, e.v, e.slot_mapping, e.k_cache, e.v_cache,
                                          e.block_tables, e.context_lens, w.max_context_len,
                                          w.scale, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(fused.view(torch.int8), out.view(torch.int8)), "fused step differs"
        assert torch.equal(e.k_cache.view(torch.int8), d.k_cache.view(torch.int8))

    if spec.mode == "prefill":
        # the same keys as contiguous rows, gathered from the post-store cache
        blk, row = [], []
        for b in range(w.batch):
            j = np.arange(int(w.context_lens[b]))
            blk.append(w.block_tables[b][j // w.block_size])
            row.append(j % w.block_size)
        blk = torch.from_numpy(np.concatenate(blk).astype(np.int64)).cuda()
        row = torch.from_numpy(np.concatenate(row).astype(np.int64)).cuda()
        k = d.k_cache[blk, :, row, :].contiguous()
        v = d.v_cache[blk, :, row, :].contiguous()
        cu_k = np.concatenate([[0], np.cumsum(w.context_lens)]).astype(np.int32)
        announce(f"{spec.name}: contiguous prefill")
        contig = pkv.pkv_prefill_varlen(d.q, k, v, d.cu_seqlens_q, torch.from_numpy(cu_k).cuda(),
                                        w.max_seqlen_q, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(contig.view(torch.int16), out.view(torch.int16)), "contiguous differs"


def random_prefix_spec(seed: int) -> tuple[Spec, int]:
    """A random decode batch (bf16) whose sequences fall into sharing
    classes: each class shares its first blocks (per member, between one and
    all the blocks before the member's new token), plus a few unshared
    sequences; and the split count (0: the automatic plan)."""
    r = np.random.default_rng(34_500 + seed)
    group = int(r.choice([1, 2, 3, 4, 5, 6, 8]))
    hkv = int(r.choice([1, 2]))
    B = int(r.choice([16, 32, 64, 128, 256, 512]))
    classes = int(r.integers(1, 4))
    ctx, groups = [], []
    for c in range(classes):
        members = int(r.integers(2, 7))
        base = int(r.integers(3 * B, 3 * B + 2400))
        for _ in range(members):
            n = base + int(r.integers(-B, B))
            ctx.append(n)
            groups.append(c)
    for _ in range(int(r.integers(0, 3))):
        ctx.append(int(r.integers(1, 2500)))
        groups.append(-1)
    shared = [0] * len(ctx)
    for c in range(classes):
        idx = [b for b in range(len(ctx)) if groups[b] == c]
        room = min((ctx[b] - 1) // B for b in idx)
        k = int(r.integers(max(1, room // 2), room + 1))
        for b in idx:
            shared[b] = k
    splits = int(r.choice([0, 0, 4, 9, 16]))
    spec = Spec(f"randpfx{seed}-g{group}x{hkv}-B{B}-b{len(ctx)}", "decode", "bf16", group * hkv,
                hkv, ctx, [1] * len(ctx), 35_000 + seed, share_group=groups, shared_blocks=shared,
                block_size=B)
    return spec, splits


@pytest.mark.parametrize("seed", list(range(24)))
def test_random_prefix_decode_against_oracle(seed):
    spec, splits = random_prefix_spec(seed)
    w = build(spec)
    d = to_device(w)
    check_inputs(d)
    S = pkv.pkv_paged_decode_split_tokens(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                          w.max_context_len, w.block_size, splits)
    plan, items = pkv.pkv_decode_prefix_plan(w.block_tables, w.context_lens, w.num_q_heads,
                                             w.num_kv_heads, w.block_size, S)
    assert plan.tolist() == pp.prefix_plan(w.block_tables.tolist(), w.context_lens.tolist(),
                                           w.block_size, w.num_q_heads // w.num_kv_heads, S)
    plan = plan.cuda()
    k_pre, v_pre = d.k_cache.clone(), d.v_cache.clone()
    announce(f"{spec.name} (splits {splits}, S {S}, {items} items): fused step with plan")
    out_step = pkv.pkv_paged_decode_step_prefix(
        d.q, d.k, d.v, d.slot_mapping, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
        w.max_context_len, w.scale, plan, items, num_splits=splits)
    torch.cuda.synchronize()
    kcb, vcb = stored_bits(w)
    assert np.array_equal(bits_view(d.k_cache.cpu()), kcb)
    assert np.array_equal(bits_view(d.v_cache.cpu()), vcb)
    want = expected(w)
    assert_close(out_step.double().cpu().numpy(), want, f"{spec.name} fused step with plan")
    d.k_cache.copy_(k_pre)
    d.v_cache.copy_(v_pre)
    announce(f"{spec.name}: store, then decode with plan")
    store(d)
    out = pkv.pkv_paged_decode_prefix(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                      w.max_context_len, w.scale, plan, items, num_splits=splits)
    torch.cuda.synchronize()
    assert_close(out.double().cpu().numpy(), want, f"{spec.name} decode with plan")
    assert torch.equal(out.view(torch.int16), out_step.view(torch.int16))
