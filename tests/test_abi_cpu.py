"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects bad host arguments with the documented status before
touching HIP (no kernel is launched here)."""

import ctypes
import glob
import os
import re

import pytest

import paged_kv_cache_325_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

BF16, FP32 = pkv.PKV_BF16, pkv.PKV_FP32
OK, INVALID, UNSUPPORTED, WORKSPACE = pkv.PKV_OK, pkv.PKV_ERR_INVALID, pkv.PKV_ERR_UNSUPPORTED, pkv.PKV_ERR_WORKSPACE

# a fake, 16-byte aligned, never-dereferenced device address
FAKE = 0x10000


def _declared_symbols():
    """Every function declared in include/*.h."""
    syms = set()
    for name in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        syms |= set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", open(name).read()))
    return sorted(syms)


def test_library_exports_every_declared_symbol():
    lib = pkv.load_library()
    syms = _declared_symbols()
    assert set(syms) >= {"pkv_kv_store", "pkv_paged_decode", "pkv_paged_prefill_varlen",
                         "pkv_paged_decode_workspace_bytes", "pkv_last_error",
                         "pkv_bm_allocate", "pkv_bm_may_append", "pkv_bm_build_decode"}
    for s in syms:
        assert hasattr(lib, s), s
    # and nm agrees that they are exported C symbols
    raw = ctypes.CDLL(pkv.lib_path())
    for s in syms:
        getattr(raw, s)


def test_block_bytes():
    assert pkv.pkv_kv_block_bytes(BF16, 8, 128, 256) == 256 * 8 * 128 * 2
    assert pkv.pkv_kv_block_bytes(FP32, 8, 128, 256) == 256 * 8 * 128 * 4
    assert pkv.pkv_kv_block_bytes(7, 8, 128, 256) == -1
    assert pkv.pkv_kv_block_bytes(BF16, 0, 128, 256) == -1


def _store(**kw):
    a = dict(dtype=BF16, k=FAKE, ks=1024, v=FAKE, vs=1024, kc=FAKE, vc=FAKE, slots=FAKE, n=4,
             hkv=8, d=128, bs=256, nblk=16)
    a.update(kw)
    lib = pkv.load_library()
    return lib.pkv_kv_store(a["dtype"], a["k"], a["ks"], a["v"], a["vs"], a["kc"], a["vc"],
                            a["slots"], a["n"], a["hkv"], a["d"], a["bs"], a["nblk"], None)


def test_kv_store_errors():
    assert _store(n=0) == OK  # nothing to do: no launch
    assert _store(n=-1) == INVALID
    assert _store(k=None) == INVALID
    assert _store(slots=None) == INVALID
    assert _store(dtype=5) == INVALID
    assert _store(d=64) == UNSUPPORTED
    for bs in (8, 48, 100, 4160, 8192):  # supported: 16, 32, multiples of 64 up to 4096
        assert _store(bs=bs) == UNSUPPORTED, bs
    assert _store(hkv=0) == INVALID
    assert _store(ks=100) == INVALID  # smaller than a row
    assert _store(ks=1028) == INVALID  # rows not 16-byte aligned
    assert _store(k=FAKE + 2) == INVALID
    assert _store(nblk=0) == INVALID
    assert "aligned" in pkv.pkv_last_error() or "num_blocks" in pkv.pkv_last_error()


def _decode(**kw):
    a = dict(dtype=BF16, q=FAKE, qs=16 * 128, kc=FAKE, vc=FAKE, bt=FAKE, mb=16, ctx=FAKE,
             maxctx=4096, batch=4, hq=16, hkv=8, d=128, bs=256, nblk=64, scale=0.088,
             splits=0, out=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    lib = pkv.load_library()
    return lib.pkv_paged_decode(a["dtype"], a["q"], a["qs"], a["kc"], a["vc"], a["bt"], a["mb"],
                                a["ctx"], a["maxctx"], a["batch"], a["hq"], a["hkv"], a["d"],
                                a["bs"], a["nblk"], a["scale"], a["splits"], a["out"], a["ws"],
                                a["wsb"], None)


def _step(**kw):
    a = dict(dtype=BF16, q=FAKE, qs=16 * 128, kn=FAKE, ks=8 * 128, vn=FAKE, vs=8 * 128,
             slots=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, mb=16, ctx=FAKE, maxctx=4096, batch=4, hq=16,
             hkv=8, d=128, bs=256, nblk=64, scale=0.088, splits=0, out=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    lib = pkv.load_library()
    return lib.pkv_paged_decode_step(a["dtype"], a["q"], a["qs"], a["kn"], a["ks"], a["vn"],
                                     a["vs"], a["slots"], a["kc"], a["vc"], a["bt"], a["mb"],
                                     a["ctx"], a["maxctx"], a["batch"], a["hq"], a["hkv"], a["d"],
                                     a["bs"], a["nblk"], a["scale"], a["splits"], a["out"], a["ws"],
                                     a["wsb"], None)


def test_decode_step_errors():
    assert _step(batch=0) == OK
    assert _step(kn=None) == INVALID
    assert _step(vn=None) == INVALID
    assert _step(slots=None) == INVALID
    assert _step(kn=FAKE + 8) == INVALID      # misaligned
    assert _step(ks=8 * 128 - 8) == INVALID   # stride below a row
    assert _step(vs=8 * 128 + 3) == INVALID   # stride not a whole 16-byte chunk
    assert _step(nblk=0) == INVALID
    assert _step(hq=24, batch=0) == OK  # group of 3: served (nothing to do)
    assert _step(ws=None, wsb=0) == WORKSPACE
    assert "k_new" in (_step(kn=None) and pkv.pkv_last_error())


def test_noalloc_step_rejects_plans_beyond_its_scratch():
    """The no-allocation decode step refuses a plan whose partials exceed the
    fixed scratch, and a non-finite scale, before any HIP call."""
    lib = pkv.load_library()

    def call(batch, maxctx, splits):
        return lib.pkv_paged_decode_step_noalloc(
            BF16, FAKE, 32 * 128, FAKE, 8 * 128, FAKE, 8 * 128, FAKE, FAKE, FAKE, FAKE,
            maxctx // 256, FAKE, maxctx, batch, 32, 8, 128, 256, 1 << 20, 0.088, splits, FAKE,
            None)

    need = pkv.pkv_paged_decode_workspace_bytes(4096, 32, 8, 128, 32768, 256, 0)
    assert need > pkv.PKV_NOALLOC_SCRATCH_BYTES
    assert call(4096, 32768, 0) == WORKSPACE
    assert "scratch" in pkv.pkv_last_error()
    assert call(0, 32768, 0) == OK  # empty batch: nothing to do
    for bad in (float("nan"), float("inf")):
        assert lib.pkv_paged_decode_step_noalloc(
            BF16, FAKE, 32 * 128, FAKE, 8 * 128, FAKE, 8 * 128, FAKE, FAKE, FAKE, FAKE, 16, FAKE,
            4096, 16, 32, 8, 128, 256, 1 << 20, bad, 0, FAKE, None) == INVALID


def test_decode_errors():
    assert _decode(batch=0) == OK
    assert _decode(batch=-1) == INVALID
    assert _decode(hq=12) == INVALID  # 12 % 8
    assert _decode(hq=24, batch=0) == OK  # group of 3: served (nothing to do)
    assert _decode(hq=0) == INVALID
    assert _decode(d=256) == UNSUPPORTED
    assert _decode(bs=48) == UNSUPPORTED
    assert _decode(bs=128) == INVALID  # supported, but 4096 > 16 table columns * 128
    assert _decode(maxctx=16 * 256 + 1) == INVALID  # beyond the table
    assert _decode(q=None) == INVALID
    assert _decode(out=FAKE + 8) == INVALID
    assert _decode(qs=100) == INVALID
    for bad in (float("nan"), float("inf"), float("-inf")):
        assert _decode(scale=bad) == INVALID
        assert _step(scale=bad) == INVALID
    assert "finite" in pkv.pkv_last_error()
    assert _decode(batch=0, scale=float("inf")) == OK  # no work: nothing is checked further
    assert _decode(splits=-2) == INVALID
    assert _decode(ws=None, wsb=0) == WORKSPACE
    need = pkv.pkv_paged_decode_workspace_bytes(4, 16, 8, 128, 4096, 256, 0)
    assert need > 0
    assert _decode(wsb=need - 4) == WORKSPACE


def test_decode_split_plan():
    # a multiple of 64 keys per split, consistent with the workspace size
    for batch, hq, hkv, maxctx, splits in [(64, 16, 8, 4096, 0), (256, 32, 8, 8192, 0),
                                           (16, 32, 8, 32768, 0), (4, 16, 8, 511, 0),
                                           (4, 16, 8, 511, 3), (3, 8, 2, 5000, 7), (2, 4, 2, 0, 0)]:
        S = pkv.pkv_paged_decode_split_tokens(batch, hq, hkv, 128, maxctx, 256, splits)
        assert S > 0 and S % 64 == 0 and S <= 16384
        assert S <= 256 or S % 256 == 0
        ns = max(1, -(-maxctx // S))
        ws = pkv.pkv_paged_decode_workspace_bytes(batch, hq, hkv, 128, maxctx, 256, splits)
        assert ws == (0 if ns == 1 else batch * hq * ns * 130 * 4)
        if splits and maxctx <= 16384:
            assert ns <= splits
    assert pkv.pkv_paged_decode_split_tokens(4, 16, 8, 128, 4096, 256, 1) >= 4096
    assert pkv.pkv_paged_decode_split_tokens(4, 16, 8, 128, 32768, 256, 1) == 16384
    assert pkv.pkv_paged_decode_workspace_bytes(4, 16, 8, 64, 4096, 256, 0) == 0  # unsupported
    assert pkv.pkv_paged_decode_workspace_bytes(4, 16, 8, 128, 4096, 48, 0) == 0  # unsupported
    # a split's block-table entries fit one register: at most 64 blocks when
    # splits are aligned to the blocks, 62 otherwise
    assert pkv.pkv_paged_decode_split_tokens(4, 16, 8, 128, 32768, 16, 1) == 1024
    assert pkv.pkv_paged_decode_split_tokens(4, 16, 8, 128, 32768, 32, 1) == 2048
    assert pkv.pkv_paged_decode_split_tokens(4, 16, 8, 128, 32768, 64, 1) == 4096
    assert pkv.pkv_paged_decode_split_tokens(4, 16, 8, 128, 65536, 512, 1) == 31744
    assert pkv.pkv_paged_decode_split_tokens(4, 16, 8, 128, 65536, 1024, 1) == 63488


def _prefill(**kw):
    a = dict(dtype=BF16, q=FAKE, qs=32 * 128, kc=FAKE, vc=FAKE, cu=FAKE, maxq=100, ctx=FAKE,
             maxctx=612, bt=FAKE, mb=4, batch=2, hq=32, hkv=8, d=128, bs=256, nblk=8,
             scale=0.088, causal=1, out=FAKE, ws=FAKE, wsb=64)
    a.update(kw)
    lib = pkv.load_library()
    return lib.pkv_paged_prefill_varlen(a["dtype"], a["q"], a["qs"], a["kc"], a["vc"], a["cu"],
                                        a["maxq"], a["ctx"], a["maxctx"], a["bt"], a["mb"],
                                        a["batch"], a["hq"], a["hkv"], a["d"], a["bs"], a["nblk"],
                                        a["scale"], a["causal"], a["out"], a["ws"], a["wsb"], None)


def test_prefill_errors():
    assert _prefill(batch=0) == OK
    assert _prefill(maxq=0) == OK
    assert _prefill(causal=0) == INVALID
    assert _prefill(dtype=FP32) == UNSUPPORTED
    assert _prefill(hq=24, batch=0) == OK  # group of 3: served (nothing to do)
    assert _prefill(d=64) == UNSUPPORTED
    assert _prefill(maxctx=5 * 256) == INVALID
    assert _prefill(cu=None) == INVALID
    assert _prefill(q=FAKE + 4) == INVALID
    assert _prefill(batch=-3) == INVALID
    assert "causal" in (_prefill(causal=2) and pkv.pkv_last_error())
    # any finite scale is taken (negative and zero ones included); a
    # non-finite one is refused
    for bad in (float("nan"), float("inf"), float("-inf")):
        assert _prefill(scale=bad) == INVALID
    assert "finite" in pkv.pkv_last_error()


def _prefill_contig(**kw):
    a = dict(dtype=BF16, q=FAKE, qs=32 * 128, k=FAKE, ks=8 * 128, v=FAKE, vs=8 * 128, cuq=FAKE,
             cuk=FAKE, maxq=100, batch=2, hq=32, hkv=8, d=128, scale=0.088, causal=1, out=FAKE,
             ws=FAKE, wsb=64)
    a.update(kw)
    lib = pkv.load_library()
    return lib.pkv_prefill_varlen(a["dtype"], a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"],
                                  a["cuq"], a["cuk"], a["maxq"], a["batch"], a["hq"], a["hkv"],
                                  a["d"], a["scale"], a["causal"], a["out"], a["ws"], a["wsb"],
                                  None)


def test_prefill_contiguous_errors():
    assert _prefill_contig(batch=0) == OK
    assert _prefill_contig(maxq=0) == OK
    assert _prefill_contig(causal=0) == INVALID
    assert _prefill_contig(dtype=FP32) == UNSUPPORTED
    assert _prefill_contig(hq=24, batch=0) == OK  # group of 3: served
    assert _prefill_contig(cuk=None) == INVALID
    assert _prefill_contig(k=FAKE + 2) == INVALID
    assert _prefill_contig(ks=8 * 128 - 8) == INVALID
    assert _prefill_contig(ws=None) == WORKSPACE
    assert "cu_seqlens_k" in (_prefill_contig(cuk=None) and pkv.pkv_last_error())
    for bad in (float("nan"), float("inf"), float("-inf")):
        assert _prefill_contig(scale=bad) == INVALID


def test_prefill_workspace():
    need = pkv.pkv_paged_prefill_workspace_bytes()
    assert 4 <= need <= 256 and need % 4 == 0
    assert _prefill(ws=None) == WORKSPACE
    assert _prefill(ws=FAKE + 2) == WORKSPACE
    assert _prefill(wsb=need - 4) == WORKSPACE
    assert "workspace" in pkv.pkv_last_error()
    # an empty problem needs no workspace
    assert _prefill(batch=0, ws=None, wsb=0) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 8, 128, dtype=torch.bfloat16)
    c = torch.zeros(2, 8, 256, 128, dtype=torch.bfloat16)
    s = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        pkv.pkv_kv_store(x, x, c, c, s)


def _merge(**kw):
    a = dict(dtype=BF16, ctx=FAKE, maxctx=4096, batch=4, hq=16, hkv=8, d=128, bs=256, splits=4,
             out=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    lib = pkv.load_library()
    return lib.pkv_paged_decode_merge(a["dtype"], a["ctx"], a["maxctx"], a["batch"], a["hq"],
                                      a["hkv"], a["d"], a["bs"], a["splits"], a["out"], a["ws"],
                                      a["wsb"], None)


def test_merge_errors():
    assert _merge(batch=0) == OK
    assert _merge(ctx=None) == INVALID
    assert _merge(out=None) == INVALID
    assert _merge(ws=None, wsb=0) == WORKSPACE
    assert _merge(d=64) == UNSUPPORTED
    assert _merge(hq=24, batch=0) == OK  # group of 3: served
    assert _merge(splits=-1) == INVALID
    assert _merge(dtype=9) == INVALID


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libpkv.so every entry point raises: there is no fallback path."""
    monkeypatch.setattr(pkv, "_LIB", None)
    monkeypatch.setattr(pkv, "lib_path", lambda: str(tmp_path / "libpkv.so"))
    with pytest.raises(RuntimeError, match="missing"):
        pkv.load_library()
    with pytest.raises(RuntimeError, match="missing"):
        pkv.pkv_kv_block_bytes(BF16, 8, 128, 256)
    with pytest.raises(RuntimeError, match="missing"):
        pkv.pkv_paged_decode_workspace_bytes(64, 16, 8, 128, 4096, 256, 0)
