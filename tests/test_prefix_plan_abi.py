"""The shared-prefix planner of the C ABI (host code, no GPU) against the
plain-Python oracle (``oracle/prefix_plan.py``), word for word, and the host
checks of the shared-prefix entry points (rejected before any HIP call)."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_325_amd as pkv
from oracle import prefix_plan as pp
from tests.test_prefix_plan_oracle import CASES, random_batch

BF16, FP32 = pkv.PKV_BF16, pkv.PKV_FP32
OK, INVALID, UNSUPPORTED, WORKSPACE = (pkv.PKV_OK, pkv.PKV_ERR_INVALID, pkv.PKV_ERR_UNSUPPORTED,
                                       pkv.PKV_ERR_WORKSPACE)
FAKE = 0x10000


def _library_plan(tables, ctx, B, G, S):
    plan, items = pkv.pkv_decode_prefix_plan(np.asarray(tables, dtype=np.int32),
                                             np.asarray(ctx, dtype=np.int32), G, 1, B, S)
    return plan.tolist(), items


@pytest.mark.parametrize("seed,B,S,G", CASES)
def test_library_plan_equals_oracle(seed, B, S, G):
    tables, ctx = random_batch(1000 + seed, B, S)
    want = pp.prefix_plan(tables, ctx, B, G, S)
    got, items = _library_plan(tables, ctx, B, G, S)
    assert got == want
    assert items == want[1]
    assert len(got) <= pkv.pkv_decode_prefix_plan_words(len(ctx), max(ctx), S)


def test_library_plan_equals_oracle_large_batch():
    # 256 sequences over 8 prompt trees with 64-token blocks: several full
    # runs per class, long common prefixes, ties between identical rows
    rng = np.random.default_rng(42)
    B, S, G = 64, 256, 4
    trunks = [list(range(1000 * t, 1000 * t + 40)) for t in range(8)]
    tables, ctx = [], []
    nxt = 100000
    for b in range(256):
        t = trunks[int(rng.integers(8))]
        n = int(rng.integers(1, 60 * B))
        keep = min(int(rng.integers(0, 41)), (n - 1) // B)
        nblk = -(-n // B)
        row = t[:keep] + list(range(nxt, nxt + nblk - keep))
        nxt += nblk
        tables.append(row)
        ctx.append(n)
    width = max(len(r) for r in tables)
    tables = [r + [-1] * (width - len(r)) for r in tables]
    want = pp.prefix_plan(tables, ctx, B, G, S)
    assert want[1] > 100  # plenty of shared splits
    assert _library_plan(tables, ctx, B, G, S)[0] == want


def test_planner_errors():
    lib = pkv.load_library()
    bt = np.zeros((4, 8), dtype=np.int32)
    ctx = np.full(4, 100, dtype=np.int32)
    buf = np.zeros(1024, dtype=np.int32)
    items, words = ctypes.c_int32(0), ctypes.c_int64(0)

    def call(bt=bt, mb=8, ctx=ctx, batch=4, hq=8, hkv=2, bs=16, split=64, plan=buf, cap=1024,
             items_p=ctypes.byref(items)):
        return lib.pkv_decode_prefix_plan(
            None if bt is None else bt.ctypes.data, mb, None if ctx is None else ctx.ctypes.data,
            batch, hq, hkv, bs, split, None if plan is None else plan.ctypes.data, cap, items_p,
            ctypes.byref(words))

    assert call() == OK and items.value == 1 and words.value == 5 + 4 + 17 + 2
    assert call(split=0) == INVALID
    assert call(split=100) == INVALID
    assert call(batch=-1) == INVALID
    assert call(hq=6, hkv=4) == INVALID
    assert call(bs=48) == UNSUPPORTED
    assert call(bt=None) == INVALID
    assert call(plan=None) == INVALID
    assert call(items_p=None) == INVALID
    assert call(cap=8) == WORKSPACE
    assert "too small" in pkv.pkv_last_error()
    assert call(mb=6) == INVALID  # 100 keys > 6 * 16
    assert call(batch=0, bt=None, ctx=None) == OK and items.value == 0
    assert pkv.pkv_decode_prefix_plan_words(4, 100, 0) == -1
    assert pkv.pkv_decode_prefix_plan_words(-1, 100, 64) == -1
    assert pkv.pkv_decode_prefix_plan_words(4, 100, 64) == 5 + 4 + 2 * 17 + 2 * 2 * 1


def test_planner_binding_refuses_device_tensors():
    if not torch.cuda.is_available():
        with pytest.raises(ValueError):
            pkv.pkv_decode_prefix_plan(np.zeros((2, 2), np.int32), np.zeros(3, np.int32), 4, 1,
                                       16, 64)
        return
    with pytest.raises(ValueError):
        pkv.pkv_decode_prefix_plan(torch.zeros((2, 2), dtype=torch.int32, device="cuda"),
                                   torch.zeros(2, dtype=torch.int32), 4, 1, 16, 64)


def _decode_prefix(**kw):
    a = dict(dtype=BF16, q=FAKE, qs=32 * 128, kc=FAKE, vc=FAKE, bt=FAKE, mb=16, ctx=FAKE,
             maxctx=4096, batch=4, hq=32, hkv=8, d=128, bs=256, nblk=64, scale=0.088, splits=0,
             plan=FAKE, items=3, out=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    lib = pkv.load_library()
    return lib.pkv_paged_decode_prefix(a["dtype"], a["q"], a["qs"], a["kc"], a["vc"], a["bt"],
                                       a["mb"], a["ctx"], a["maxctx"], a["batch"], a["hq"],
                                       a["hkv"], a["d"], a["bs"], a["nblk"], a["scale"],
                                       a["splits"], a["plan"], a["items"], a["out"], a["ws"],
                                       a["wsb"], None)


def test_prefix_decode_errors():
    assert _decode_prefix(batch=0) == OK
    assert _decode_prefix(dtype=FP32, qs=32 * 128) == UNSUPPORTED
    assert "bf16" in pkv.pkv_last_error()
    assert _decode_prefix(items=-1) == INVALID
    assert _decode_prefix(plan=None) == INVALID
    assert _decode_prefix(plan=FAKE + 2) == INVALID
    assert _decode_prefix(hq=128, qs=128 * 128) == INVALID  # G = 16: no plan has items
    assert _decode_prefix(ws=None, wsb=0) == WORKSPACE
    assert _decode_prefix(scale=float("nan")) == INVALID
    lib = pkv.load_library()
    st = lib.pkv_paged_decode_step_prefix(
        FP32, FAKE, 32 * 128, FAKE, 8 * 128, FAKE, 8 * 128, FAKE, FAKE, FAKE, FAKE, 16, FAKE,
        4096, 4, 32, 8, 128, 256, 64, 0.088, 0, FAKE, 2, FAKE, FAKE, 1 << 30, None)
    assert st == UNSUPPORTED
    st = lib.pkv_paged_decode_step_prefix(
        BF16, FAKE, 32 * 128, None, 8 * 128, FAKE, 8 * 128, FAKE, FAKE, FAKE, FAKE, 16, FAKE,
        4096, 4, 32, 8, 128, 256, 64, 0.088, 0, FAKE, 2, FAKE, FAKE, 1 << 30, None)
    assert st == INVALID
