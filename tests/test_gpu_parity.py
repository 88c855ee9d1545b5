"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Store: bit-exact over the whole cache.  Attention: within max-abs 2e-2 and
mean-abs 2e-3 of the fp64 oracle (bf16 or fp32 inputs, fp32 accumulation).
Small cases and the five full-size workloads are checked on every output
row; the full-size ones in the launch configuration the benchmark uses
(automatic split plan)."""

import dataclasses
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_325_amd as pkv
from oracle import ref
from tests.gpu_helpers import (DeviceWorkload, announce, assert_close, attend, check_inputs,
                               store, to_device)
from tests.oracle_helpers import expected, q64, sequence_view, stored_bits
from workloads import Spec, bits_view, build, config, small_specs

pytestmark = pytest.mark.gpu

SMALL = small_specs()
SMALL_IDS = [s.name for s in SMALL]


def _cache_bits(t: torch.Tensor) -> np.ndarray:
    return bits_view(t.cpu())


def _run_step(w, num_splits=0):
    d = to_device(w)
    check_inputs(d)
    announce(f"{w.spec.name}: kv_store")
    store(d)
    announce(f"{w.spec.name}: attention (num_splits={num_splits})")
    out = attend(d, num_splits=num_splits)
    torch.cuda.synchronize()
    return d, out


# ---------------------------------------------------------------------------
# small cases: every row
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("spec", SMALL, ids=SMALL_IDS)
def test_small_store_bit_exact(spec):
    w = build(spec)
    d, _ = _run_step(w)
    kcb, vcb = stored_bits(w)
    assert np.array_equal(_cache_bits(d.k_cache), kcb)
    assert np.array_equal(_cache_bits(d.v_cache), vcb)


@pytest.mark.parametrize("spec", SMALL, ids=SMALL_IDS)
def test_small_attention(spec):
    w = build(spec)
    _, out = _run_step(w)
    want = expected(w)
    assert_close(out.to(torch.float64).cpu().numpy(), want, spec.name)
    if w.dtype == "fp32":  # fp32 inputs: much tighter than the bf16 bound
        assert np.abs(out.to(torch.float64).cpu().numpy() - want).max() < 1e-4


@pytest.mark.parametrize("scale", [-0.5, -1 / math.sqrt(128), 0.0])
@pytest.mark.parametrize("name", ["pre-bf16-g4", "pre-bf16-g2", "dec-bf16-g4-long"])
def test_any_finite_scale(name, scale):
    """A negative or zero softmax scale is a legal input: the result is
    softmax(scale * q.k) all the same (the prefill kernel masks before it
    scales, so it computes scale * q.k exactly as |scale| * (-q).k, or as
    1 * (0.k) for a zero scale)."""
    spec = dataclasses.replace([s for s in SMALL if s.name == name][0], scale=scale,
                               name=f"{name}-scale{scale:+.3f}")
    w = build(spec)
    _, out = _run_step(w)
    assert_close(out.to(torch.float64).cpu().numpy(), expected(w), spec.name)


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 64])
def test_decode_forced_splits(splits):
    w = build([s for s in SMALL if s.name == "dec-bf16-g4-long"][0])
    _, out = _run_step(w, num_splits=splits)
    assert_close(out.to(torch.float64).cpu().numpy(), expected(w), f"splits={splits}")


def test_decode_more_than_64_splits():
    # 100 requested splits of a 16 k context: splits of 192 keys, 86 of them,
    # so the merge takes its loop over more than one group of 64 splits
    w = build(Spec("dec-long-86", "decode", "bf16", 8, 2, [16384, 9000, 300], [1] * 3, 9201))
    S = pkv.pkv_paged_decode_split_tokens(w.batch, 8, 2, 128, w.max_context_len, 256, 100)
    assert S == 192 and -(-16384 // S) > 64
    _, out = _run_step(w, num_splits=100)
    assert_close(out.to(torch.float64).cpu().numpy(), expected(w), "86 splits")


# Compacted split units (the plan has >= 16 splits of >= 512 keys): lengths
# on and off split multiples, an empty context, a context of 1, sequences
# shorter than one split and one spanning all of them.  At 32 requested
# splits of a 20 000-key context the plan has 27 splits of 768 keys.
COMPACT_CTX = [20000, 0, 1, 767, 768, 769, 1536, 15360, 8193, 300, 0, 12000]


@pytest.mark.parametrize("hq,hkv", [(16, 8), (8, 2)], ids=["g2", "g4"])
def test_compacted_units_ragged_and_empty(hq, hkv):
    spec = Spec(f"dec-compact-h{hq}-{hkv}", "decode", "bf16", hq, hkv, COMPACT_CTX,
                [0 if c == 0 else 1 for c in COMPACT_CTX], 9211)
    w = build(spec)
    S = pkv.pkv_paged_decode_split_tokens(w.batch, hq, hkv, 128, w.max_context_len, 256, 32)
    nsplit = -(-w.max_context_len // S)
    assert S >= 512 and nsplit >= 16  # the compacted mode's bounds
    d = to_device(w)
    check_inputs(d)
    k_pre, v_pre = d.k_cache.clone(), d.v_cache.clone()
    announce(f"{spec.name}: fused step, compacted units")
    out_step = pkv.pkv_paged_decode_step(d.q, d.k, d.v, d.slot_mapping, d.k_cache, d.v_cache,
                                         d.block_tables, d.context_lens, w.max_context_len,
                                         w.scale, num_splits=32)
    d.k_cache.copy_(k_pre)
    d.v_cache.copy_(v_pre)
    d2, out = _run_step(w, num_splits=32)
    torch.cuda.synchronize()
    want = expected(w)
    assert_close(out.to(torch.float64).cpu().numpy(), want, "compacted units")
    assert torch.equal(out.view(torch.int16), out_step.view(torch.int16))
    for b, c in enumerate(COMPACT_CTX):
        if c == 0:
            assert (out[b].float() == 0).all()


@pytest.mark.parametrize("block_size", [256, 16, 64, 1024])
def test_long_prefill_table_beyond_registers(block_size):
    # one 12 k-token sequence whose first 8 k tokens are cached: at 16-token
    # blocks its table has 768 entries, past the 128 a workgroup keeps in
    # registers, so the copies read the rest through scalar loads (at 64:
    # 192 entries, the block walker through all three sources; at 1024 the
    # walker crosses a block every 16 tiles); the last 512 query rows,
    # sampled, against the oracle
    ctx, new = 12288, 4096
    w = build(Spec(f"pre-long-B{block_size}", "prefill", "bf16", 8, 2, [ctx], [new], 9202,
                   block_size=block_size))
    d, out = _run_step(w)
    rows = list(range(new - 512, new, 7)) + [0, 1, 63, 64, 1000]
    kcb, vcb = stored_bits(w)
    want = ref.prefill(q64(w), ref.widen(kcb, "bf16"), ref.widen(vcb, "bf16"), w.cu_seqlens_q,
                       w.context_lens, w.block_tables, w.scale, rows=rows)
    got = out.to(torch.float64).cpu().numpy()
    assert_close(got[rows], want[rows], f"long prefill at block size {block_size}")


def test_split_partials_in_workspace():
    """The split-K partials (acc, m, l) the decode kernel leaves in the
    workspace match the oracle's partials for the same split size."""
    w = build([s for s in SMALL if s.name == "dec-bf16-g4-long"][0])
    d = to_device(w)
    check_inputs(d)
    store(d)
    splits = 4
    args = (w.batch, w.num_q_heads, w.num_kv_heads, 128, w.max_context_len, 256, splits)
    S = pkv.pkv_paged_decode_split_tokens(*args)
    nbytes = pkv.pkv_paged_decode_workspace_bytes(*args)
    ns = -(-w.max_context_len // S)
    assert nbytes >= w.batch * w.num_q_heads * ns * 130 * 4
    nacc_ml = w.batch * w.num_q_heads * ns * 130
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    announce("workspace partials: decode")
    attend(d, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    nacc = w.batch * w.num_q_heads * ns * 128
    acc = ws[:nacc].view(w.batch, w.num_q_heads, ns, 128).cpu().double().numpy()
    ml = ws[nacc:nacc_ml].view(w.batch, w.num_q_heads, ns, 2).cpu().double().numpy()
    kcb, vcb = stored_bits(w)
    parts = ref.decode_partials(q64(w), ref.widen(kcb, w.dtype), ref.widen(vcb, w.dtype),
                                w.block_tables, w.context_lens, w.scale, S)
    log2e = 1.0 / math.log(2.0)
    checked = 0
    for b, (pacc, pm, pl) in enumerate(parts):
        nsb = pacc.shape[0]
        if nsb <= 1:
            continue  # single-split sequences write their output directly
        for s in range(nsb):
            for h in range(w.num_q_heads):
                assert abs(ml[b, h, s, 0] - pm[s, h] * log2e) < 1e-3
                assert abs(ml[b, h, s, 1] - pl[s, h]) <= 2e-3 * pl[s, h]
                scale = max(1.0, np.abs(pacc[s, h]).max())
                assert np.abs(acc[b, h, s] - pacc[s, h]).max() <= 2e-2 * scale
                checked += 1
    assert checked > 0
    announce("workspace partials: reuse")
    out2 = attend(d, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert_close(out2.double().cpu().numpy(), expected(w), "reused workspace")


# 5 requested splits: 1-5 per sequence (the merge's one-wavefront forms);
# 24: splits of 256 keys, 12-20 per long sequence (the plan has more than 16,
# so the four-wavefront merge runs, and takes the one-wavefront form for the
# sequence with 12); 100: splits of 64 keys, up to 79 (more than one group of
# 64 splits in the four-wavefront form).
@pytest.mark.parametrize("splits", [5, 24, 100])
def test_merge_of_oracle_partials(splits):
    """The merge entry point alone: fed the oracle's split partials (written
    into the documented workspace layout), it must produce the oracle's
    merged output."""
    w = build([s for s in SMALL if s.name == "dec-bf16-g4-long"][0])
    args = (w.batch, w.num_q_heads, w.num_kv_heads, 128, w.max_context_len, 256, splits)
    S = pkv.pkv_paged_decode_split_tokens(*args)
    ns = -(-w.max_context_len // S)
    kcb, vcb = stored_bits(w)
    kc, vc = ref.widen(kcb, w.dtype), ref.widen(vcb, w.dtype)
    q = q64(w)
    parts = ref.decode_partials(q, kc, vc, w.block_tables, w.context_lens, w.scale, S)
    acc = np.zeros((w.batch, w.num_q_heads, ns, 128), np.float32)
    ml = np.zeros((w.batch, w.num_q_heads, ns, 2), np.float32)
    log2e = 1.0 / math.log(2.0)
    want = np.zeros((w.batch, w.num_q_heads, 128))
    merged_rows = []
    for b, (pacc, pm, pl) in enumerate(parts):
        nsb = pacc.shape[0]
        if nsb <= 1:
            continue
        merged_rows.append(b)
        acc[b, :, :nsb] = pacc.transpose(1, 0, 2)
        ml[b, :, :nsb, 0] = (pm * log2e).T
        ml[b, :, :nsb, 1] = pl.T
        want[b] = ref.merge_partials(pacc, pm, pl)
    assert merged_rows, "the case must split some sequences"
    nbytes = pkv.pkv_paged_decode_workspace_bytes(*args)
    host = np.concatenate([acc.ravel(), ml.ravel()])
    assert host.size * 4 == nbytes
    ws = torch.from_numpy(host).cuda()
    out = torch.full((w.batch, w.num_q_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ctx = torch.from_numpy(w.context_lens).cuda()
    announce(f"merge of oracle partials, {ns} splits")
    pkv.pkv_paged_decode_merge(ctx, w.max_context_len, w.num_q_heads, w.num_kv_heads,
                               w.block_size, out, ws,
                               num_splits=splits)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    assert_close(got[merged_rows], want[merged_rows], "merge")
    # rows of single-split sequences are not touched by the merge
    others = [b for b in range(w.batch) if b not in merged_rows]
    assert torch.isnan(out[others].float()).all()


def _bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Bits of float32 values rounded to bfloat16, to nearest even (finite
    values only)."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


# Partials with every m_s = 0 and l_s = 1: each weight 2^(m_s - M) is 1
# exactly and the denominator is the split count, a power of two, so the
# merged row is exactly bf16(fp32 sum of acc_s taken in split order / ns).
# Each acc element is +-2^20 (signs balanced over the splits, in a random
# order) plus a standard normal: the running sum's rounding then depends on
# the order of the additions far beyond bf16's resolution of the result
# (on the CPU, summing these rows in reverse order changes 46-98 % of the
# bf16 outputs of each sequence, and as four interleaved partial sums of 16
# rows per group, 88-97 % of those with more than 16 splits).  16 requested
# splits: 16/8/4 per sequence (the one-wavefront merge kernel); 64: 64/32/16
# (the four-wavefront kernel, staged and not); 128: 128/64/32 (two groups
# of 64).
@pytest.mark.parametrize("splits", [16, 64, 128])
def test_merge_sums_in_split_order_bitwise(splits):
    batch, hq, hkv, max_ctx = 3, 8, 2, 16384
    ctx = np.array([16384, 8192, 4096], np.int32)
    S = pkv.pkv_paged_decode_split_tokens(batch, hq, hkv, 128, max_ctx, 256, splits)
    nsplit = -(-max_ctx // S)
    assert nsplit == splits
    r = np.random.default_rng(31_000 + splits)
    acc = r.standard_normal((batch, hq, nsplit, 128)).astype(np.float32)
    for b in range(batch):
        ns = -(-int(ctx[b]) // S)
        signs = np.where(np.arange(ns) % 2 == 0, 1.0, -1.0)
        big = np.stack([np.stack([r.permutation(signs) for _ in range(128)], -1)
                        for _ in range(hq)], 0)  # [hq, ns, 128]
        acc[b, :, :ns] += (big * 2.0 ** 20).astype(np.float32)
    ml = np.zeros((batch, hq, nsplit, 2), np.float32)
    ml[..., 1] = 1.0
    host = np.concatenate([acc.ravel(), ml.ravel()])
    assert host.size * 4 == pkv.pkv_paged_decode_workspace_bytes(batch, hq, hkv, 128, max_ctx,
                                                                 256, splits)
    ws = torch.from_numpy(host).cuda()
    out = torch.zeros((batch, hq, 128), dtype=torch.bfloat16, device="cuda")
    announce(f"merge in split order, {splits} splits")
    pkv.pkv_paged_decode_merge(torch.from_numpy(ctx).cuda(), max_ctx, hq, hkv, 256, out, ws,
                               num_splits=splits)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(batch):
        ns = -(-int(ctx[b]) // S)
        total = np.zeros((hq, 128), np.float32)
        for sp in range(ns):
            total = (total + acc[b, :, sp]).astype(np.float32)
        want = _bf16_rne_bits(total * np.float32(1.0 / ns))
        assert np.array_equal(got[b], want), (b, ns)


def test_partials_then_merge_equals_decode_bit_exact():
    w = build([s for s in SMALL if s.name == "dec-bf16-g2-ragged"][0])
    d = to_device(w)
    check_inputs(d)
    store(d)
    announce("decode in one call")
    whole = pkv.pkv_paged_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                 w.max_context_len, w.scale, num_splits=6)
    announce("decode in two calls")
    out, ws = pkv.pkv_paged_decode_partials(d.q, d.k_cache, d.v_cache, d.block_tables,
                                            d.context_lens, w.max_context_len, w.scale,
                                            num_splits=6)
    pkv.pkv_paged_decode_merge(d.context_lens, w.max_context_len, w.num_q_heads,
                               w.num_kv_heads, w.block_size, out, ws, num_splits=6)
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16), out.view(torch.int16))


# ---------------------------------------------------------------------------
# invariants on the GPU result
# ---------------------------------------------------------------------------

def _decode_out(d, **kw):
    out = attend(d, **kw)
    torch.cuda.synchronize()
    return out.clone()


def test_decode_deterministic_and_permutation_bit_exact():
    w = build([s for s in SMALL if s.name == "dec-bf16-g4-long"][0])
    d = to_device(w)
    check_inputs(d)
    store(d)
    announce("determinism: decode twice")
    a = _decode_out(d)
    b = _decode_out(d)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # permute the physical blocks and the table: reduction order is logical,
    # so the result must not change by a single bit
    pi = torch.from_numpy(np.random.default_rng(5).permutation(w.num_blocks)).cuda()
    kc2 = torch.empty_like(d.k_cache)
    vc2 = torch.empty_like(d.v_cache)
    kc2[pi] = d.k_cache
    vc2[pi] = d.v_cache
    bt = d.block_tables.long()
    bt2 = torch.where(bt >= 0, pi[bt.clamp(min=0)], bt).int().contiguous()
    announce("permutation: decode on permuted pool")
    c = pkv.pkv_paged_decode(d.q, kc2, vc2, bt2, d.context_lens, w.max_context_len, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def _private_copies(w, d):
    """The same logical K/V with every shared block duplicated into a block
    of its own: (k_cache, v_cache, block_tables) on the GPU."""
    bt = w.block_tables.copy()
    extra = []
    nxt = w.num_blocks
    for b in range(w.batch):
        for i in range(bt.shape[1]):
            if bt[b, i] >= 0 and int(bt[b, i]) in w.shared_physical:
                extra.append(int(bt[b, i]))
                bt[b, i] = nxt
                nxt += 1
    idx = torch.tensor(extra, device="cuda", dtype=torch.long)
    kc2 = torch.cat([d.k_cache, d.k_cache[idx]]).contiguous()
    vc2 = torch.cat([d.v_cache, d.v_cache[idx]]).contiguous()
    return kc2, vc2, torch.from_numpy(bt).cuda()


# Sequences 0/1 share 6 blocks, 2/3 one block (sequence 3's only full one),
# 4/5 share none, 6/7 share 3 of which 7 uses 2, and 8 shares with nobody;
# shared runs start on and off split boundaries under the split plans below.
PAIR_CTX = [3000, 2500, 600, 257, 900, 900, 1800, 700, 1500]
PAIR_GROUPS = [0, 0, 1, 1, -1, -1, 2, 2, -1]
PAIR_SHARED = [6, 6, 1, 1, 0, 0, 3, 2, 0]


@pytest.mark.parametrize("splits", [0, 1, 3, 16])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 2), (2, 2), (8, 1)],
                         ids=["g4", "g2", "g1", "g8"])
def test_pairs_sharing_blocks_bitwise_equal_private(hq, hkv, splits):
    """Prefix-shared blocks give identical outputs: decode and the fused step
    over shared prefix blocks are bitwise equal to the same K/V in private
    blocks (where no two tables match), for every GQA group size and several
    split plans, and match the oracle."""
    w = build(Spec(f"pairs-h{hq}-{hkv}", "decode", "bf16", hq, hkv, PAIR_CTX, [1] * 9,
                   9601 + hq + hkv, share_group=PAIR_GROUPS, shared_blocks=PAIR_SHARED))
    d = to_device(w)
    check_inputs(d)
    kc2, vc2, bt2 = _private_copies(w, d)
    announce(f"pairs h{hq}/{hkv} splits {splits}: fused step, shared and private")
    k_pre, v_pre = d.k_cache.clone(), d.v_cache.clone()
    out_step = pkv.pkv_paged_decode_step(d.q, d.k, d.v, d.slot_mapping, d.k_cache, d.v_cache,
                                         d.block_tables, d.context_lens, w.max_context_len,
                                         w.scale, num_splits=splits)
    kc3, vc3, _ = _private_copies(w, dataclasses.replace(d, k_cache=k_pre, v_cache=v_pre))
    out_step2 = pkv.pkv_paged_decode_step(d.q, d.k, d.v, d.slot_mapping, kc3, vc3, bt2,
                                          d.context_lens, w.max_context_len, w.scale,
                                          num_splits=splits)
    announce(f"pairs h{hq}/{hkv} splits {splits}: decode, shared and private")
    store(d)
    kc2, vc2, _ = _private_copies(w, d)
    a = pkv.pkv_paged_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                             w.max_context_len, w.scale, num_splits=splits)
    c = pkv.pkv_paged_decode(d.q, kc2, vc2, bt2, d.context_lens, w.max_context_len, w.scale,
                             num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert torch.equal(out_step.view(torch.int16), a.view(torch.int16))
    assert torch.equal(out_step2.view(torch.int16), a.view(torch.int16))
    assert_close(a.double().cpu().numpy(), expected(w), w.spec.name)


def test_shared_prefix_equals_private_copies_bit_exact():
    w = build([s for s in SMALL if s.name == "dec-bf16-shared"][0])
    d = to_device(w)
    check_inputs(d)
    store(d)
    announce("shared prefix: decode")
    a = _decode_out(d)
    kc2, vc2, bt2 = _private_copies(w, d)
    announce("shared prefix: decode on private copies")
    c = pkv.pkv_paged_decode(d.q, kc2, vc2, bt2, d.context_lens, w.max_context_len, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_context_one_returns_v_row_bit_exact(dtype):
    w = build(Spec("ctx1", "decode", dtype, 8, 2, [1, 1, 1, 1], [1] * 4, 4242))
    d, out = _run_step(w)
    v = d.v.contiguous()  # the stored V rows, [batch, Hkv, D]
    for h in range(8):
        assert torch.equal(out[:, h], v[:, h // 4]), f"head {h}"


def test_prefill_single_query_matches_decode():
    ctx = [1, 300, 513, 1024, 2000]
    wp = build(Spec("p1", "prefill", "bf16", 8, 2, ctx, [1] * 5, 777))
    dp, outp = _run_step(wp)
    # the same inputs through decode
    announce("decode of the same single queries")
    outd = pkv.pkv_paged_decode(dp.q, dp.k_cache, dp.v_cache, dp.block_tables, dp.context_lens,
                                wp.max_context_len, wp.scale)
    torch.cuda.synchronize()
    assert_close(outp.double().cpu().numpy(), outd.double().cpu().numpy(), "prefill vs decode")
    assert_close(outp.double().cpu().numpy(), expected(wp), "prefill vs oracle")


def test_mixed_chunked_prefill_and_decode_batch():
    # one varlen call holding decode rows (one query at the end of a long
    # context), chunks of a prompt whose earlier chunks are cached (queries
    # in the middle of the context), a fresh prompt and a chunk that ends on
    # a block boundary: the batch a chunked-prefill scheduler mixes
    ctx = [1500, 700, 257, 1024, 3000, 64, 512]
    new = [1, 300, 257, 512, 1, 64, 1]
    w = build(Spec("mixed", "prefill", "bf16", 16, 8, ctx, new, 778,
                   share_group=[0, 0, -1, -1, 0, -1, -1], shared_blocks=[2, 1, 0, 0, 2, 0, 0]))
    d, out = _run_step(w)
    assert_close(out.double().cpu().numpy(), expected(w), "mixed batch")
    # each decode row equals pkv_paged_decode of that sequence alone
    rows = [int(w.cu_seqlens_q[b]) for b in range(w.batch) if new[b] == 1]
    seqs = [b for b in range(w.batch) if new[b] == 1]
    sel = torch.tensor(seqs, device=d.q.device)
    q1 = d.q[torch.tensor(rows, device=d.q.device)].contiguous()
    outd = pkv.pkv_paged_decode(q1, d.k_cache, d.v_cache, d.block_tables[sel].contiguous(),
                                d.context_lens[sel].contiguous(), w.max_context_len, w.scale)
    torch.cuda.synchronize()
    assert_close(out[torch.tensor(rows, device=d.q.device)].double().cpu().numpy(),
                 outd.double().cpu().numpy(), "decode rows of the mixed batch vs decode")


@pytest.mark.parametrize("spec", [
    Spec("pre-tiny-1item", "prefill", "bf16", 4, 1, [40], [40], 801),
    Spec("pre-tiny-6items", "prefill", "bf16", 4, 1, [70, 20], [70, 20], 802),
    Spec("pre-g4-42items", "prefill", "bf16", 8, 2, [100, 300, 7], [100, 200, 7], 803),
], ids=lambda s: s.name)
def test_prefill_workspace_reset_and_small_grids(spec):
    """The persistent prefill kernel's work-queue counters: an explicit
    workspace is zero again after every call, repeated calls are bitwise
    identical, and grids with fewer work items than queues are complete."""
    w = build(spec)
    d = to_device(w)
    check_inputs(d)
    store(d)
    ws = torch.zeros(pkv.pkv_paged_prefill_workspace_bytes() // 4, dtype=torch.int32,
                     device="cuda")
    outs = []
    for i in range(3):
        announce(f"{spec.name}: prefill call {i} with an explicit workspace")
        outs.append(pkv.pkv_paged_prefill_varlen(d.q, d.k_cache, d.v_cache, d.cu_seqlens_q,
                                                 w.max_seqlen_q, d.context_lens,
                                                 w.max_context_len, d.block_tables, w.scale,
                                                 workspace=ws))
        torch.cuda.synchronize()
        assert int(ws.abs().sum()) == 0, "workspace not reset"
    for o in outs[1:]:
        assert torch.equal(outs[0], o)
    assert_close(outs[0].double().cpu().numpy(), expected(w), spec.name)


def test_prefill_workspace_not_zeroed_is_contained():
    """A workspace whose queue counters were never zeroed (here every counter
    holds -2^30) breaks the work queues, not memory: every ticket is outside
    the item range, so each queue counts as exhausted, the kernel ends and no
    output row is touched.  A zeroed workspace then gives the oracle's
    result."""
    w = build([s for s in SMALL if s.name == "pre-bf16-g4"][0])
    d = to_device(w)
    check_inputs(d)
    store(d)
    n = pkv.pkv_paged_prefill_workspace_bytes() // 4
    bad = torch.full((n,), -(1 << 30), dtype=torch.int32, device="cuda")
    out = torch.full((w.num_tokens, w.num_q_heads, 128), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    announce("prefill with a workspace that was not zeroed")
    pkv.pkv_paged_prefill_varlen(d.q, d.k_cache, d.v_cache, d.cu_seqlens_q, w.max_seqlen_q,
                                 d.context_lens, w.max_context_len, d.block_tables, w.scale,
                                 out=out, workspace=bad)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    announce("prefill with a zeroed workspace after it")
    good = torch.zeros(n, dtype=torch.int32, device="cuda")
    pkv.pkv_paged_prefill_varlen(d.q, d.k_cache, d.v_cache, d.cu_seqlens_q, w.max_seqlen_q,
                                 d.context_lens, w.max_context_len, d.block_tables, w.scale,
                                 out=out, workspace=good)
    torch.cuda.synchronize()
    assert int(good.abs().sum()) == 0
    assert_close(out.double().cpu().numpy(), expected(w), "after a bad workspace")


# ---------------------------------------------------------------------------
# the five full-size workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_config(index):
    """Whole step at full size, in the benchmark's launch configuration
    (automatic split plan): the store bit-exact over both caches, then the
    attention output of every sequence (decode, one sequence at a time
    through a mini-cache of its own blocks) or of every query row of every
    head (prefill) against the oracle."""
    w = config(index)
    d, out_t = _run_step(w)
    out = out_t.double().cpu().numpy()
    kcb, vcb = stored_bits(w)
    assert np.array_equal(_cache_bits(d.k_cache), kcb), "k_cache after store"
    assert np.array_equal(_cache_bits(d.v_cache), vcb), "v_cache after store"
    del d
    q = q64(w)
    if w.spec.mode == "decode":
        worst = 0.0
        for b in range(w.batch):
            kc, vc, row = sequence_view(w, kcb, vcb, b)
            want = ref.decode(q[b : b + 1], kc, vc, row[None, :], w.context_lens[b : b + 1],
                              w.scale)
            assert_close(out[b : b + 1], want, f"config {index} sequence {b}")
            worst = max(worst, float(np.abs(out[b : b + 1] - want).max()))
        announce(f"config {index}: all {w.batch} sequences within tolerance "
                 f"(worst max-abs {worst:.3g})")
    else:
        kc, vc = ref.widen(kcb, w.dtype), ref.widen(vcb, w.dtype)
        want = ref.prefill(q, kc, vc, w.cu_seqlens_q, w.context_lens, w.block_tables, w.scale)
        assert_close(out, want, f"config {index}, all {w.num_tokens} query rows")
        announce(f"config {index}: all {w.num_tokens} query rows x {w.num_q_heads} heads "
                 f"within tolerance (max-abs {float(np.abs(out - want).max()):.3g})")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("table_cols", [1, 0], ids=["table-1col", "table-0col"])
def test_decode_all_contexts_empty(dtype, table_cols):
    """A batch in which no sequence has a key (every context length 0,
    max_context_len 0): every output row is written as 0 (no mass to
    normalise), by the plain decode and by the fused step with every slot
    -1, and the cache is left untouched."""
    batch, hq, hkv, d, B = 3, 8, 2, 128, 256
    g = torch.Generator().manual_seed(4711)
    q = torch.randn(batch, hq, d, generator=g).to(dtype).cuda()
    k_new = torch.randn(batch, hkv, d, generator=g).to(dtype).cuda()
    v_new = torch.randn(batch, hkv, d, generator=g).to(dtype).cuda()
    k_cache = torch.randn(1, hkv, B, d, generator=g).to(dtype).cuda()
    v_cache = torch.randn(1, hkv, B, d, generator=g).to(dtype).cuda()
    k0, v0 = k_cache.clone(), v_cache.clone()
    tables = torch.full((batch, table_cols), -1, dtype=torch.int32, device="cuda")
    ctx = torch.zeros(batch, dtype=torch.int32, device="cuda")
    slots = torch.full((batch,), -1, dtype=torch.int32, device="cuda")
    zeros = torch.zeros(batch, hq, d, dtype=dtype, device="cuda")
    announce(f"all-empty decode, {dtype}, {table_cols} table columns")
    out = torch.full((batch, hq, d), float("nan"), dtype=dtype, device="cuda")
    pkv.pkv_paged_decode(q, k_cache, v_cache, tables, ctx, 0, 1 / math.sqrt(d), out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, zeros)
    announce(f"all-empty fused decode step, {dtype}, {table_cols} table columns")
    out2 = torch.full((batch, hq, d), float("nan"), dtype=dtype, device="cuda")
    pkv.pkv_paged_decode_step(q, k_new, v_new, slots, k_cache, v_cache, tables, ctx, 0,
                              1 / math.sqrt(d), out=out2)
    torch.cuda.synchronize()
    assert torch.equal(out2, zeros)
    assert torch.equal(k_cache, k0) and torch.equal(v_cache, v0)
