"""GPU: the fused decode step (store + decode in one call) against the two
separate calls, bitwise, and replayed from a captured HIP graph.

Every decode workload here satisfies the decode-step invariant: each row's
slot is -1 or the slot of its last position, in a block no other sequence
reads (the generators place new tokens that way, and shared prefix blocks
never hold a last position)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_325_amd as pkv
from tests.gpu_helpers import announce, attend, check_inputs, store, to_device
from workloads import build, config, small_specs

pytestmark = pytest.mark.gpu

DECODE_SMALL = [s for s in small_specs() if s.mode == "decode"]


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _step(d, num_splits=0, out=None, workspace=None):
    w = d.w
    return pkv.pkv_paged_decode_step(d.q, d.k, d.v, d.slot_mapping, d.k_cache, d.v_cache,
                                     d.block_tables, d.context_lens, w.max_context_len, w.scale,
                                     out=out, workspace=workspace, num_splits=num_splits)


def _compare(w, num_splits):
    ref = to_device(w)
    check_inputs(ref)
    announce(f"{w.spec.name}: store then decode (num_splits={num_splits})")
    store(ref)
    out_ref = attend(ref, num_splits=num_splits)
    fused = to_device(w)
    announce(f"{w.spec.name}: fused decode step (num_splits={num_splits})")
    out = _step(fused, num_splits)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(out_ref)), "outputs differ"
    assert torch.equal(_bits(fused.k_cache), _bits(ref.k_cache)), "k_cache differs"
    assert torch.equal(_bits(fused.v_cache), _bits(ref.v_cache)), "v_cache differs"


@pytest.mark.parametrize("num_splits", [0, 3])
@pytest.mark.parametrize("spec", DECODE_SMALL, ids=[s.name for s in DECODE_SMALL])
def test_step_equals_store_then_decode_small(spec, num_splits):
    _compare(build(spec), num_splits)


@pytest.mark.parametrize("index", [1, 2, 5])
def test_step_equals_store_then_decode_full(index):
    _compare(config(index), 0)


def test_step_replayed_from_graph():
    """Capture one step in a HIP graph (through torch's graph capture) and
    replay it on fresh inputs three times, with eager work in between; every
    replay must equal the eager step bitwise."""
    spec = next(s for s in DECODE_SMALL if s.name == "dec-bf16-g2-ragged")
    w = build(spec)
    d = to_device(w)
    check_inputs(d)
    kc0, vc0 = d.k_cache.clone(), d.v_cache.clone()
    out = torch.empty_like(d.q)
    need = pkv.pkv_paged_decode_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, 128,
                                                w.max_context_len, 256, 0)
    ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device="cuda")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        announce("graph warm-up step")
        _step(d, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    announce("graph capture")
    with torch.cuda.graph(graph):
        _step(d, out=out, workspace=ws)
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(3250)
    for rep in range(3):
        qkv = torch.randn(d.qkv.shape, generator=gen).to(d.qkv.dtype)
        d.qkv.copy_(qkv.to("cuda"))
        d.k_cache.copy_(kc0)
        d.v_cache.copy_(vc0)
        announce(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        got, got_k, got_v = out.clone(), d.k_cache.clone(), d.v_cache.clone()

        e = to_device(w)
        e.qkv.copy_(qkv.to("cuda"))
        announce(f"eager step {rep}")
        want = _step(e)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(want)), f"replay {rep}: outputs differ"
        assert torch.equal(_bits(got_k), _bits(e.k_cache)), f"replay {rep}: k_cache differs"
        assert torch.equal(_bits(got_v), _bits(e.v_cache)), f"replay {rep}: v_cache differs"


def test_graph_bucket_replays_with_padding():
    """One decode step captured for a batch bucket of 8 sequences and a fixed
    split plan (max_context_len 2048), then replayed for real batches of 8,
    5, 1 and 3 sequences of other lengths: the metadata buffers are rewritten
    in place and the unused rows padded with slot -1 and context 0.  Every
    replay equals the eager step on the same buffers bitwise, padded rows are
    zero and leave the caches untouched, and the real rows match the oracle."""
    from tests.gpu_helpers import MAX_ABS, MEAN_ABS, errors
    from tests.oracle_helpers import expected, to_numpy_out
    from workloads import Spec

    bucket, cap, B, pool = 8, 2048, 256, 64
    cols = cap // B
    hq, hkv, D = 8, 2, 128
    cases = []
    rng = np.random.default_rng(3251)
    for r in (8, 5, 1, 3):
        ctx = [int(x) for x in rng.integers(1, cap, size=r, endpoint=True)]
        w = build(Spec(f"bucket-r{r}", "decode", "bf16", hq, hkv, ctx, [1] * r,
                       int(rng.integers(1 << 30)), pool_blocks=pool))
        assert w.block_tables.shape[1] <= cols and w.num_blocks == pool
        cases.append(w)

    def fill(dst, w):
        """Copy workload w into the bucket-sized buffers, padding rows r.."""
        r = w.batch
        dst["qkv"].zero_()
        dst["qkv"][:r].copy_(w.qkv.to("cuda"))
        dst["slot"].fill_(-1)
        dst["slot"][:r].copy_(torch.from_numpy(w.slot_mapping.astype(np.int32)))
        dst["ctx"].zero_()
        dst["ctx"][:r].copy_(torch.from_numpy(w.context_lens.astype(np.int32)))
        dst["bt"].fill_(-1)
        bt = torch.from_numpy(w.block_tables.astype(np.int32))
        dst["bt"][:r, : bt.shape[1]].copy_(bt)
        dst["kc"].copy_(w.k_cache.to("cuda"))
        dst["vc"].copy_(w.v_cache.to("cuda"))

    def buffers():
        w0 = cases[0]
        return {"qkv": torch.empty((bucket,) + tuple(w0.qkv.shape[1:]), dtype=w0.qkv.dtype, device="cuda"),
                "slot": torch.empty(bucket, dtype=torch.int32, device="cuda"),
                "ctx": torch.empty(bucket, dtype=torch.int32, device="cuda"),
                "bt": torch.empty((bucket, cols), dtype=torch.int32, device="cuda"),
                "kc": torch.empty_like(w0.k_cache, device="cuda"),
                "vc": torch.empty_like(w0.v_cache, device="cuda"),
                "out": torch.empty((bucket, hq, D), dtype=w0.qkv.dtype, device="cuda")}

    need = pkv.pkv_paged_decode_workspace_bytes(bucket, hq, hkv, D, cap, B, 0)

    def step(buf, ws):
        q, k, v = buf["qkv"][:, :hq], buf["qkv"][:, hq:hq + hkv], buf["qkv"][:, hq + hkv:]
        return pkv.pkv_paged_decode_step(q, k, v, buf["slot"], buf["kc"], buf["vc"], buf["bt"],
                                         buf["ctx"], cap, cases[0].scale, out=buf["out"],
                                         workspace=ws)

    g_buf = buffers()
    g_ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device="cuda")
    fill(g_buf, cases[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        announce("bucket graph: warm-up step")
        step(g_buf, g_ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    announce("bucket graph: capture")
    with torch.cuda.graph(graph):
        step(g_buf, g_ws)
    torch.cuda.synchronize()

    e_buf = buffers()
    e_ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device="cuda")
    for w in cases:
        r = w.batch
        fill(g_buf, w)
        kc0, vc0 = g_buf["kc"].clone(), g_buf["vc"].clone()
        torch.cuda.synchronize()
        announce(f"bucket graph: replay with {r} real rows")
        graph.replay()
        torch.cuda.synchronize()
        fill(e_buf, w)
        announce(f"bucket graph: eager step with {r} real rows")
        step(e_buf, e_ws)
        torch.cuda.synchronize()
        for key in ("out", "kc", "vc"):
            assert torch.equal(_bits(g_buf[key]), _bits(e_buf[key])), f"r={r}: {key} differs"
        assert not _bits(g_buf["out"][r:]).any(), f"r={r}: padded rows not zero"
        # only the real rows' slots were written
        changed = (_bits(g_buf["kc"]) != _bits(kc0)).any(dim=-1).nonzero()
        written = {int(p) * B + int(o) for p, _, o in changed.tolist()}
        assert written <= {int(s) for s in w.slot_mapping if s >= 0}, f"r={r}: stray cache writes"
        got = to_numpy_out(g_buf["out"][:r])
        mx, mean = errors(got, expected(w))
        assert mx <= MAX_ABS and mean <= MEAN_ABS, f"r={r}: max {mx:.3e} mean {mean:.3e}"
