"""GPU: varlen causal prefill over contiguous k/v (no cache), against the
paged prefill on the same keys (bitwise: same kernel, only the tile source
differs) and against the fp64 oracle."""

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_325_amd as pkv
from oracle import ref
from tests.gpu_helpers import announce, assert_close, attend, check_inputs, store, to_device
from tests.oracle_helpers import expected
from workloads import Spec, bits_view, build, config, small_specs

pytestmark = pytest.mark.gpu

PREFILL_SMALL = [s for s in small_specs() if s.mode == "prefill"]


def _contiguous_keys(d):
    """The cache rows of every sequence's context, gathered into contiguous
    [total_k, Hkv, D] tensors (after the store), and cu_seqlens_k."""
    w = d.w
    blk, row = [], []
    for b in range(w.batch):
        n = int(w.context_lens[b])
        j = np.arange(n)
        blk.append(w.block_tables[b][j // w.block_size])
        row.append(j % w.block_size)
    blk = torch.from_numpy(np.concatenate(blk).astype(np.int64)).cuda()
    row = torch.from_numpy(np.concatenate(row).astype(np.int64)).cuda()
    k = d.k_cache[blk, :, row, :].contiguous()
    v = d.v_cache[blk, :, row, :].contiguous()
    cu_k = np.concatenate([[0], np.cumsum(w.context_lens)]).astype(np.int32)
    return k, v, torch.from_numpy(cu_k).cuda()


def _both_paths(w):
    d = to_device(w)
    check_inputs(d)
    store(d)
    announce(f"{w.spec.name}: paged prefill")
    paged = attend(d)
    k, v, cu_k = _contiguous_keys(d)
    announce(f"{w.spec.name}: contiguous prefill")
    contig = pkv.pkv_prefill_varlen(d.q, k, v, d.cu_seqlens_q, cu_k, w.max_seqlen_q, w.scale)
    torch.cuda.synchronize()
    return paged, contig


@pytest.mark.parametrize("spec", PREFILL_SMALL, ids=[s.name for s in PREFILL_SMALL])
def test_contiguous_equals_paged_small(spec):
    w = build(spec)
    paged, contig = _both_paths(w)
    assert torch.equal(paged.view(torch.int16), contig.view(torch.int16))
    assert_close(contig.double().cpu().numpy(), expected(w), spec.name)


@pytest.mark.parametrize("scale", [-0.25, 0.0])
def test_contiguous_any_finite_scale(scale):
    """Negative and zero scales through the contiguous tile source too."""
    spec = dataclasses.replace(PREFILL_SMALL[0], scale=scale,
                               name=f"{PREFILL_SMALL[0].name}-scale{scale:+.2f}")
    w = build(spec)
    paged, contig = _both_paths(w)
    assert torch.equal(paged.view(torch.int16), contig.view(torch.int16))
    assert_close(contig.double().cpu().numpy(), expected(w), spec.name)


def test_contiguous_equals_paged_full_prefill_workload():
    paged, contig = _both_paths(config(3))
    assert torch.equal(paged.view(torch.int16), contig.view(torch.int16))


def test_contiguous_fresh_qkv_views():
    """No prefix hit: keys are this step's own k, v -- strided views of the
    fused qkv buffer -- checked against the contiguous oracle."""
    spec = Spec("pre-fresh", "prefill", "bf16", 8, 2, [1, 63, 200, 517], [1, 63, 200, 517], 7311)
    w = build(spec)
    d = to_device(w)
    announce("fresh-qkv contiguous prefill")
    out = pkv.pkv_prefill_varlen(d.q, d.k, d.v, d.cu_seqlens_q, d.cu_seqlens_q, w.max_seqlen_q,
                                 w.scale)
    torch.cuda.synchronize()
    q64 = ref.widen(bits_view(w.q.contiguous()), "bf16")
    k64 = ref.widen(bits_view(w.k.contiguous()), "bf16")
    v64 = ref.widen(bits_view(w.v.contiguous()), "bf16")
    want = ref.prefill_contiguous(q64, k64, v64, w.cu_seqlens_q, w.cu_seqlens_q, w.scale)
    assert_close(out.double().cpu().numpy(), want, "fresh qkv")


def test_contiguous_fewer_keys_than_queries():
    """Bottom-right causal with n_k < n_q: the first n_q - n_k queries see no
    key and are zero."""
    gen = torch.Generator().manual_seed(99)
    nq, nk = [70, 5, 129], [6, 5, 300]
    cu_q = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(nk)]).astype(np.int32)
    q = torch.randn((cu_q[-1], 8, 128), generator=gen).to(torch.bfloat16)
    k = torch.randn((cu_k[-1], 2, 128), generator=gen).to(torch.bfloat16)
    v = torch.randn((cu_k[-1], 2, 128), generator=gen).to(torch.bfloat16)
    scale = 128 ** -0.5
    announce("contiguous prefill, fewer keys than queries")
    out = pkv.pkv_prefill_varlen(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(cu_q).cuda(),
                                 torch.from_numpy(cu_k).cuda(), max(nq), scale)
    torch.cuda.synchronize()
    want = ref.prefill_contiguous(ref.widen(bits_view(q), "bf16"), ref.widen(bits_view(k), "bf16"),
                                  ref.widen(bits_view(v), "bf16"), cu_q, cu_k, scale)
    got = out.double().cpu().numpy()
    assert np.all(got[: nq[0] - nk[0]] == 0.0)
    assert_close(got, want, "n_k < n_q")
