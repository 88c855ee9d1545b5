"""Pins of the CPU oracle against facts that do not come from the oracle:
the worked example and block arithmetic of the pages, a pure-Python brute
force, torch's fp64 scaled_dot_product_attention on contiguous tensors,
closed forms and invariants.  The last group plants plausible mistakes in the
oracle and checks that a pin catches each one."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, ref
from workloads import Spec, bits_view, build, small_specs
from tests.oracle_helpers import expected, q64, stored_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# the pages' worked example and block arithmetic
# ---------------------------------------------------------------------------

def test_worked_example_address_translation():
    for c in _golden("address_translation.json")["cases"]:
        assert ref.locate(c["position"], c["page_size"]) == (c["page_index"], c["offset"])


def test_worked_example_through_store_and_gather():
    # page size 16, a two-page sequence whose pages are physical 5 and 2:
    # the token at logical position 25 must land on physical page 2, row 9.
    B, Hkv, D = 16, 1, 4
    cache = np.zeros((6, Hkv, B, D), dtype=np.uint32)
    table = [5, 2]
    k = np.arange(D, dtype=np.uint32).reshape(1, Hkv, D) + 100
    slot = np.array([table[1] * B + 9], dtype=np.int32)  # page index 1, offset 9
    kc, vc = ref.kv_store(k, k, cache, cache, slot, B)
    assert (kc[2, 0, 9] == k[0, 0]).all()
    assert kc.sum() == k.sum()
    rows = ref.gather(kc, table, 26)
    assert (rows[25, 0] == k[0, 0]).all()


def test_block_arithmetic():
    g = _golden("block_arithmetic.json")
    for c in g["cases"]:
        assert ref.num_blocks(c["num_tokens"], g["block_size"]) == c["num_blocks"]
        assert ref.last_block_tokens(c["num_tokens"], g["block_size"]) == c["last_block_tokens"]


# ---------------------------------------------------------------------------
# store
# ---------------------------------------------------------------------------

def test_store_skips_minus_one_and_touches_nothing_else():
    w = build(small_specs()[0])  # has one skipped slot
    kcb, vcb = stored_bits(w)
    before_k, before_v = bits_view(w.k_cache), bits_view(w.v_cache)
    kb = bits_view(w.k.contiguous())
    changed = np.zeros(kcb.shape[:1] + kcb.shape[2:3], dtype=bool)  # [nblk, B]
    for t, s in enumerate(w.slot_mapping):
        if s < 0:
            continue
        p, o = divmod(int(s), w.block_size)
        assert (kcb[p, :, o] == kb[t]).all()
        changed[p, o] = True
    mask = ~changed[:, None, :, None] & np.ones_like(kcb, dtype=bool)
    assert (kcb[mask] == before_k[mask]).all()
    assert (vcb[mask] == before_v[mask]).all()
    assert (w.slot_mapping == -1).sum() == 1


def test_store_copies_nan_payloads_bit_exactly():
    B, Hkv, D = 4, 2, 8
    cache = np.zeros((3, Hkv, B, D), dtype=np.uint16)
    k = np.full((2, Hkv, D), 0x7F81, dtype=np.uint16)  # signalling-NaN payload
    v = np.full((2, Hkv, D), 0xFFFF, dtype=np.uint16)
    kc, vc = ref.kv_store(k, v, cache, cache, np.array([5, -1], np.int32), B)
    assert (kc[1, :, 1] == 0x7F81).all() and (vc[1, :, 1] == 0xFFFF).all()
    assert int((kc != 0).sum()) == Hkv * D


def test_widen_is_exact():
    x = torch.randn(1000, dtype=torch.float64)
    for dt, tdt in (("bf16", torch.bfloat16), ("fp32", torch.float32)):
        t = x.to(tdt)
        assert np.array_equal(ref.widen(bits_view(t), dt), t.to(torch.float64).numpy())


# ---------------------------------------------------------------------------
# brute force on tiny inputs
# ---------------------------------------------------------------------------

def _tiny(mode, seed, ctx, new, hq=4, hkv=2, **kw):
    return build(Spec(f"tiny-{mode}", mode, "fp32", hq, hkv, ctx, new, seed,
                      head_dim=8, block_size=4, **kw))


def _lists(w):
    kcb, vcb = stored_bits(w)
    kc, vc = ref.widen(kcb, "fp32"), ref.widen(vcb, "fp32")
    return q64(w), kc, vc


def test_brute_force_decode():
    w = _tiny("decode", 11, [1, 5, 12, 17, 40], [1] * 5)
    q, kc, vc = _lists(w)
    got = ref.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale)
    want = brute.decode(q.tolist(), kc.tolist(), vc.tolist(), w.block_tables.tolist(),
                        w.context_lens.tolist(), w.scale, 2, 4)
    assert np.abs(got - np.array(want)).max() < 1e-12


def test_brute_force_prefill():
    w = _tiny("prefill", 12, [7, 12, 30, 9], [7, 3, 14, 1], share_group=[-1, 0, 0, -1],
              shared_blocks=[0, 2, 3, 0])
    q, kc, vc = _lists(w)
    got = ref.prefill(q, kc, vc, w.cu_seqlens_q, w.context_lens, w.block_tables, w.scale)
    want = brute.prefill(q.tolist(), kc.tolist(), vc.tolist(), w.cu_seqlens_q.tolist(),
                         w.context_lens.tolist(), w.block_tables.tolist(), w.scale, 2, 4)
    assert np.abs(got - np.array(want)).max() < 1e-12
    # sampled rows agree with the full computation
    rows = [0, 8, 9, 23]
    part = ref.prefill(q, kc, vc, w.cu_seqlens_q, w.context_lens, w.block_tables, w.scale, rows=rows)
    assert np.abs(part[rows] - got[rows]).max() < 1e-12


# ---------------------------------------------------------------------------
# library routine: torch fp64 SDPA on contiguous (un-paged) tensors
# ---------------------------------------------------------------------------

def _paged_from_contiguous(seqs, B, rng, pool_extra=3):
    """Scatter per-sequence contiguous [n, Hkv, D] tensors into a shuffled
    block pool, one cell at a time.  Returns (cache, tables)."""
    need = [(s.shape[0] + B - 1) // B for s in seqs]
    pool = sum(need) + pool_extra
    perm = rng.permutation(pool)
    Hkv, D = seqs[0].shape[1], seqs[0].shape[2]
    cache = np.full((pool, Hkv, B, D), np.nan)
    tables = np.full((len(seqs), max(need) + 1), -1, dtype=np.int32)
    c = 0
    for b, s in enumerate(seqs):
        for i in range(need[b]):
            tables[b, i] = perm[c]
            c += 1
        for j in range(s.shape[0]):
            cache[tables[b, j // B], :, j % B, :] = s[j]
    return cache, tables


def _sdpa(q, K, V, visible):
    """q [nq, Hq, D], K/V [nk, Hkv, D]; query i sees keys < visible[i]."""
    Hq, Hkv = q.shape[1], K.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [Hq, nq, D]
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    mask = torch.arange(K.shape[0])[None, :] < torch.as_tensor(visible)[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask)
    return o.permute(1, 0, 2).numpy()


def check_sdpa_decode(seed=0):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, B = 8, 2, 16, 8
    lens = [1, 9, 31, 64]
    Ks = [rng.standard_normal((n, Hkv, D)) for n in lens]
    Vs = [rng.standard_normal((n, Hkv, D)) for n in lens]
    kc, tables = _paged_from_contiguous(Ks, B, np.random.default_rng(seed + 1))
    vc, _ = _paged_from_contiguous(Vs, B, np.random.default_rng(seed + 1))
    q = rng.standard_normal((len(lens), Hq, D))
    got = ref.decode(q, kc, vc, tables, np.array(lens), 1 / math.sqrt(D))
    err = 0.0
    for b, n in enumerate(lens):
        want = _sdpa(q[b : b + 1], Ks[b], Vs[b], [n])[0]
        err = max(err, np.abs(got[b] - want).max())
    return err


def check_sdpa_prefill(seed=0):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, B = 8, 2, 16, 8
    nk = [10, 33, 17]
    nq = [10, 5, 1]
    Ks = [rng.standard_normal((n, Hkv, D)) for n in nk]
    Vs = [rng.standard_normal((n, Hkv, D)) for n in nk]
    kc, tables = _paged_from_contiguous(Ks, B, np.random.default_rng(seed + 1))
    vc, _ = _paged_from_contiguous(Vs, B, np.random.default_rng(seed + 1))
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = rng.standard_normal((cu[-1], Hq, D))
    got = ref.prefill(q, kc, vc, cu, np.array(nk), tables, 1 / math.sqrt(D))
    err = 0.0
    for b in range(len(nk)):
        lo, hi = cu[b], cu[b + 1]
        visible = [nk[b] - nq[b] + i + 1 for i in range(nq[b])]  # bottom-right causal
        want = _sdpa(q[lo:hi], Ks[b], Vs[b], visible)
        err = max(err, np.abs(got[lo:hi] - want).max())
    return err


def check_sdpa_prefill_contiguous(seed=0):
    """prefill_contiguous against SDPA with the causal mask is_causal builds
    itself (square sequences, where top-left and bottom-right alignment
    coincide), plus an explicit bottom-right mask for n_k > n_q."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = 8, 2, 16
    nq = [12, 1, 7, 5]
    nk = [12, 1, 7, 19]
    cu_q = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(nk)]).astype(np.int32)
    q = rng.standard_normal((cu_q[-1], Hq, D))
    k = rng.standard_normal((cu_k[-1], Hkv, D))
    v = rng.standard_normal((cu_k[-1], Hkv, D))
    scale = 1 / math.sqrt(D)
    got = ref.prefill_contiguous(q, k, v, cu_q, cu_k, scale)
    err = 0.0
    for b in range(len(nq)):
        lo, hi, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if nq[b] == nk[b]:
            qt = torch.from_numpy(q[lo:hi]).permute(1, 0, 2)
            Kt = torch.from_numpy(k[k0:k1]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
            Vt = torch.from_numpy(v[k0:k1]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
            want = torch.nn.functional.scaled_dot_product_attention(
                qt, Kt, Vt, is_causal=True, scale=scale).permute(1, 0, 2).numpy()
        else:
            visible = [nk[b] - nq[b] + i + 1 for i in range(nq[b])]
            want = _sdpa(q[lo:hi], k[k0:k1], v[k0:k1], visible)
        err = max(err, np.abs(got[lo:hi] - want).max())
    return err


def test_sdpa_prefill_contiguous():
    assert check_sdpa_prefill_contiguous() < 1e-12


def test_brute_force_prefill_contiguous():
    """Including sequences with fewer keys than queries: the first queries see
    no key and must be zero."""
    rng = np.random.default_rng(21)
    Hq, Hkv, D = 4, 2, 8
    nq = [5, 3, 6, 1]
    nk = [5, 7, 2, 1]
    cu_q = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(nk)]).astype(np.int32)
    q = rng.standard_normal((cu_q[-1], Hq, D))
    k = rng.standard_normal((cu_k[-1], Hkv, D))
    v = rng.standard_normal((cu_k[-1], Hkv, D))
    got = ref.prefill_contiguous(q, k, v, cu_q, cu_k, 0.3)
    want = np.array(brute.prefill_contiguous(q.tolist(), k.tolist(), v.tolist(), cu_q.tolist(),
                                             cu_k.tolist(), 0.3, Hkv))
    assert np.abs(got - want).max() < 1e-12
    # sequence 2: 6 queries over 2 keys -- queries 0..3 see nothing
    assert np.all(got[cu_q[2] : cu_q[2] + 4] == 0.0)
    assert np.all(np.abs(got[cu_q[2] + 4 : cu_q[3]]) > 0.0)
    rows = [1, 6, 13]
    part = ref.prefill_contiguous(q, k, v, cu_q, cu_k, 0.3, rows=rows)
    assert np.abs(part[rows] - got[rows]).max() < 1e-12


def test_sdpa_decode():
    assert check_sdpa_decode() < 1e-12


def test_sdpa_prefill():
    assert check_sdpa_prefill() < 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _decode_case(ctx, seed=3, q_zero=False, k_equal=False):
    w = build(Spec("cf", "decode", "bf16", 4, 2, ctx, [1] * len(ctx), seed))
    kcb, vcb = stored_bits(w)
    kc, vc = ref.widen(kcb, "bf16"), ref.widen(vcb, "bf16")
    q = q64(w)
    if q_zero:
        q[:] = 0.0
    if k_equal:
        kc[:] = 0.25
    return w, q, kc, vc


def test_context_one_returns_v_row_exactly():
    w, q, kc, vc = _decode_case([1, 1, 1])
    out = ref.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale)
    for b in range(3):
        p = w.block_tables[b, 0]
        for h in range(4):
            assert np.array_equal(out[b, h], vc[p, h // 2, 0])


def test_zero_query_gives_mean_of_values():
    w, q, kc, vc = _decode_case([5, 300, 700], q_zero=True)
    out = ref.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale)
    for b, n in enumerate(w.context_lens):
        V = ref.gather(vc, w.block_tables[b], int(n))
        for h in range(4):
            assert np.abs(out[b, h] - V[:, h // 2].mean(axis=0)).max() < 1e-12


def test_equal_keys_give_uniform_weights_and_weights_sum_to_one():
    w, q, kc, vc = _decode_case([7, 260], k_equal=True)
    _, wts = ref.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale, return_weights=True)
    for b, n in enumerate(w.context_lens):
        for h in range(4):
            assert np.abs(wts[b][h] - 1.0 / n).max() < 1e-15
    w, q, kc, vc = _decode_case([7, 260, 1000], seed=5)
    _, wts = ref.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale, return_weights=True)
    for b in range(3):
        for h in range(4):
            assert abs(wts[b][h].sum() - 1.0) < 1e-12


def test_empty_context_gives_zero_row():
    w = build([s for s in small_specs() if s.name == "dec-bf16-empty-ctx"][0])
    out = expected(w)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.array_equal(out[2], np.zeros_like(out[2]))
    assert np.isfinite(out).all()


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_physical_block_permutation_leaves_output_unchanged():
    w = build(small_specs()[1])
    kcb, vcb = stored_bits(w)
    kc, vc = ref.widen(kcb, w.dtype), ref.widen(vcb, w.dtype)
    q = q64(w)
    base = ref.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale)
    pi = np.random.default_rng(77).permutation(w.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    bt2 = np.where(w.block_tables >= 0, pi[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    again = ref.decode(q, kc2, vc2, bt2, w.context_lens, w.scale)
    assert np.array_equal(base, again)


def test_shared_prefix_equals_private_copies():
    w = build([s for s in small_specs() if s.name == "dec-bf16-shared"][0])
    kcb, vcb = stored_bits(w)
    kc, vc = ref.widen(kcb, w.dtype), ref.widen(vcb, w.dtype)
    q = q64(w)
    base = ref.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale)
    # give every sequence its own copy of each shared block
    bt = w.block_tables.copy()
    extra_k, extra_v = [], []
    nxt = w.num_blocks
    for b in range(w.batch):
        for i in range(bt.shape[1]):
            p = bt[b, i]
            if p >= 0 and p in w.shared_physical:
                extra_k.append(kc[p])
                extra_v.append(vc[p])
                bt[b, i] = nxt
                nxt += 1
    assert extra_k, "the case must share blocks"
    kc2 = np.concatenate([kc, np.stack(extra_k)])
    vc2 = np.concatenate([vc, np.stack(extra_v)])
    again = ref.decode(q, kc2, vc2, bt, w.context_lens, w.scale)
    assert np.array_equal(base, again)


def test_prefill_rows_equal_decode_at_their_position():
    w = build([s for s in small_specs() if s.name == "pre-bf16-g4"][0])
    kcb, vcb = stored_bits(w)
    kc, vc = ref.widen(kcb, w.dtype), ref.widen(vcb, w.dtype)
    q = q64(w)
    pre = ref.prefill(q, kc, vc, w.cu_seqlens_q, w.context_lens, w.block_tables, w.scale)
    for b in range(w.batch):
        lo, hi = w.cu_seqlens_q[b], w.cu_seqlens_q[b + 1]
        nk, nq = int(w.context_lens[b]), int(hi - lo)
        for i in sorted({0, nq // 2, nq - 1}):
            pos = nk - nq + i
            dec = ref.decode(q[lo + i : lo + i + 1], kc, vc, w.block_tables[b : b + 1],
                             np.array([pos + 1]), w.scale)
            assert np.abs(dec[0] - pre[lo + i]).max() < 1e-12


@pytest.mark.parametrize("split", [1, 7, 64, 256, 1000])
def test_split_partials_merge_to_decode(split):
    w = build(small_specs()[1])
    kcb, vcb = stored_bits(w)
    kc, vc = ref.widen(kcb, w.dtype), ref.widen(vcb, w.dtype)
    q = q64(w)
    base = ref.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale)
    parts = ref.decode_partials(q, kc, vc, w.block_tables, w.context_lens, w.scale, split)
    for b, (acc, m, l) in enumerate(parts):
        assert np.abs(ref.merge_partials(acc, m, l) - base[b]).max() < 1e-12


def check_partials_against_brute_force(split=5):
    """Largest deviation of the oracle's split partials from brute force on a
    tiny paged case: m of a split must be the largest of its scores (taken
    cell by cell through the block table), l the sum of exp(score - m) over
    the split's keys and acc the sum of exp(score - m) * v over them.  (An
    error in m alone cancels in the merge, so this pins m and l directly.)"""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, D, nblk = 4, 4, 2, 8, 9
    kc = rng.standard_normal((nblk, Hkv, B, D))
    vc = rng.standard_normal((nblk, Hkv, B, D))
    ctx = np.array([13, 4, 1, 9], dtype=np.int32)
    tables = np.full((4, 4), -1, dtype=np.int32)
    perm = rng.permutation(nblk)
    tables[0, :4] = perm[:4]
    tables[1, :1] = perm[4:5]
    tables[2, :1] = perm[5:6]
    tables[3, :3] = perm[6:9]
    q = rng.standard_normal((4, Hq, D)) * 2.0
    scale = 0.37
    parts = ref.decode_partials(q, kc, vc, tables, ctx, scale, split)
    worst = 0.0
    for b in range(4):
        acc, m, l = parts[b]
        n = int(ctx[b])
        assert acc.shape[0] == -(-n // split)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            x = brute.scores(q[b][h].tolist(), kc.tolist(), tables[b].tolist(), n, g, B, scale)
            for s in range(acc.shape[0]):
                lo, hi = s * split, min(n, (s + 1) * split)
                top = max(x[lo:hi])
                e = [math.exp(v - top) for v in x[lo:hi]]
                a = [math.fsum(e[j - lo] * brute.value_row(vc.tolist(), tables[b].tolist(), j,
                                                            g, B)[d] for j in range(lo, hi))
                     for d in range(D)]
                worst = max(worst, abs(m[s, h] - top), abs(l[s, h] - math.fsum(e)) / math.fsum(e),
                            float(np.abs(acc[s, h] - np.array(a)).max()))
    return worst


@pytest.mark.parametrize("split", [1, 3, 5, 64])
def test_split_partials_against_brute_force(split):
    assert check_partials_against_brute_force(split) < 1e-12


# ---------------------------------------------------------------------------
# planted mistakes: each plausible error in the oracle fails a pin above
# ---------------------------------------------------------------------------

def test_planted_mistakes_are_caught(monkeypatch):
    good_d, good_p = check_sdpa_decode(), check_sdpa_prefill()
    assert good_d < 1e-12 and good_p < 1e-12

    with monkeypatch.context() as m:  # GQA heads interleaved instead of grouped
        m.setattr(ref, "kv_head_of", lambda h, hq, hkv: h % hkv)
        assert check_sdpa_decode() > 1e-3
    with monkeypatch.context() as m:  # top-left causal alignment
        m.setattr(ref, "visible_keys", lambda i, nq, nk: min(nk, i + 1))
        assert check_sdpa_prefill() > 1e-3
    with monkeypatch.context() as m:  # row and block swapped in the translation
        m.setattr(ref, "locate", lambda pos, B: (pos % B, pos // B))
        with pytest.raises(Exception):
            test_worked_example_address_translation()
    with monkeypatch.context() as m:  # scale dropped
        orig = ref._attend
        m.setattr(ref, "_attend", lambda q, k, v, s: orig(q, k, v, 1.0))
        assert check_sdpa_decode() > 1e-3
    with monkeypatch.context() as m:  # contiguous keys: top-left causal alignment
        m.setattr(ref, "visible_keys", lambda i, nq, nk: min(nk, i + 1))
        assert check_sdpa_prefill_contiguous() > 1e-3
    with monkeypatch.context() as m:  # contiguous keys: K and V rows swapped
        orig_c = ref.prefill_contiguous
        m.setattr(ref, "prefill_contiguous",
                  lambda q, k, v, cq, ck, s, rows=None: orig_c(q, v, k, cq, ck, s, rows))
        assert check_sdpa_prefill_contiguous() > 1e-3
    with monkeypatch.context() as m:  # split maxima offset (cancels in the merge)
        orig_p = ref.decode_partials

        def shifted(*a, **k):
            return [(acc, mm + 1.0, l) for acc, mm, l in orig_p(*a, **k)]
        m.setattr(ref, "decode_partials", shifted)
        assert check_partials_against_brute_force() > 0.5
    with monkeypatch.context() as m:  # split sums taken over the whole sequence
        orig_p = ref.decode_partials

        def whole_l(q, kc, vc, bt, ctx, scale, split):
            full = orig_p(q, kc, vc, bt, ctx, scale, 1 << 30)
            return [(acc, mm, np.broadcast_to(fl[0], l.shape).copy())
                    for (acc, mm, l), (_, _, fl) in zip(orig_p(q, kc, vc, bt, ctx, scale, split),
                                                        full)]
        m.setattr(ref, "decode_partials", whole_l)
        assert check_partials_against_brute_force() > 1e-3
    with monkeypatch.context() as m:  # off-by-one in the number of blocks read
        m.setattr(ref, "num_blocks", lambda n, B: n // B + 1 if n % B else n // B - 1 if n > B else 1)
        with pytest.raises(Exception):
            test_block_arithmetic()
