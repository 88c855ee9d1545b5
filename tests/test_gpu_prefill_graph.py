"""GPU: a prefill step (store, then the paged varlen prefill, then the same
prefill over contiguous k/v) captured in a HIP graph through torch's graph
capture and replayed on fresh inputs.  The prefill's work-queue counters
live in a caller workspace that every call leaves zero, so the captured
kernels need no memset node; each replay must equal the eager step bitwise
and leave the workspace zero, with eager prefills on the same workspace
between the replays."""

import numpy as np
import pytest
import torch

import paged_kv_cache_325_amd as pkv
from tests.gpu_helpers import announce, check_inputs, store, to_device
from workloads import build, small_specs

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16)


def _contiguous_keys(d):
    """Each sequence's context rows from the cache, as [total_k, Hkv, D]
    (index tensors built on the host), and cu_seqlens_k."""
    w = d.w
    blk, row = [], []
    for b in range(w.batch):
        j = np.arange(int(w.context_lens[b]))
        blk.append(w.block_tables[b][j // w.block_size])
        row.append(j % w.block_size)
    blk = torch.from_numpy(np.concatenate(blk).astype(np.int64)).cuda()
    row = torch.from_numpy(np.concatenate(row).astype(np.int64)).cuda()
    cu_k = np.concatenate([[0], np.cumsum(w.context_lens)]).astype(np.int32)
    return blk, row, torch.from_numpy(cu_k).cuda()


def _step(d, out_paged, out_contig, kbuf, vbuf, idx, cu_k, ws):
    """store; paged prefill; gather the context rows; contiguous prefill."""
    w = d.w
    store(d)
    pkv.pkv_paged_prefill_varlen(d.q, d.k_cache, d.v_cache, d.cu_seqlens_q, w.max_seqlen_q,
                                 d.context_lens, w.max_context_len, d.block_tables, w.scale,
                                 out=out_paged, workspace=ws)
    blk, row = idx
    kbuf.copy_(d.k_cache[blk, :, row, :])
    vbuf.copy_(d.v_cache[blk, :, row, :])
    pkv.pkv_prefill_varlen(d.q, kbuf, vbuf, d.cu_seqlens_q, cu_k, w.max_seqlen_q, w.scale,
                           out=out_contig, workspace=ws)


def test_prefill_step_replayed_from_graph():
    spec = next(s for s in small_specs() if s.name == "pre-bf16-g4")
    w = build(spec)
    d = to_device(w)
    check_inputs(d)
    kc0, vc0 = d.k_cache.clone(), d.v_cache.clone()
    blk, row, cu_k = _contiguous_keys(d)
    total_k = int(cu_k[-1].item())
    kbuf = torch.empty((total_k, w.num_kv_heads, 128), dtype=d.q.dtype, device="cuda")
    vbuf = torch.empty_like(kbuf)
    out_p, out_c = torch.empty_like(d.q), torch.empty_like(d.q)
    ws = torch.zeros(max(pkv.pkv_paged_prefill_workspace_bytes() // 4, 1), dtype=torch.int32,
                     device="cuda")
    args = (d, out_p, out_c, kbuf, vbuf, (blk, row), cu_k, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        announce("prefill graph: warm-up step")
        _step(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    announce("prefill graph: capture")
    with torch.cuda.graph(graph):
        _step(*args)
    torch.cuda.synchronize()
    assert int(ws.abs().sum().item()) == 0

    gen = torch.Generator().manual_seed(3251)
    for rep in range(3):
        qkv = torch.randn(d.qkv.shape, generator=gen).to(d.qkv.dtype)
        d.qkv.copy_(qkv.to("cuda"))
        d.k_cache.copy_(kc0)
        d.v_cache.copy_(vc0)
        out_p.zero_()
        out_c.zero_()
        announce(f"prefill graph: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert int(ws.abs().sum().item()) == 0, f"replay {rep}: queue counters not reset"
        got_p, got_c = out_p.clone(), out_c.clone()
        got_k, got_v = d.k_cache.clone(), d.v_cache.clone()

        # the eager step on fresh buffers, sharing the graph's workspace
        e = to_device(w)
        e.qkv.copy_(qkv.to("cuda"))
        ep, ec = torch.empty_like(e.q), torch.empty_like(e.q)
        kb2, vb2 = torch.empty_like(kbuf), torch.empty_like(vbuf)
        announce(f"prefill graph: eager step {rep}")
        _step(e, ep, ec, kb2, vb2, (blk, row), cu_k, ws)
        torch.cuda.synchronize()
        assert int(ws.abs().sum().item()) == 0
        assert torch.equal(_bits(got_p), _bits(ep)), f"replay {rep}: paged outputs differ"
        assert torch.equal(_bits(got_c), _bits(ec)), f"replay {rep}: contiguous outputs differ"
        assert torch.equal(_bits(got_p), _bits(got_c)), f"replay {rep}: paths differ"
        assert torch.equal(_bits(got_k), _bits(e.k_cache)), f"replay {rep}: k_cache differs"
        assert torch.equal(_bits(got_v), _bits(e.v_cache)), f"replay {rep}: v_cache differs"
