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
