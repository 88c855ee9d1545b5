"""Glue between seeded workloads and the CPU oracle (test code only)."""

from __future__ import annotations

import numpy as np
import torch

from oracle import ref
from workloads import Workload, bits_view


def stored_bits(w: Workload):
    """Oracle store applied to the workload: post-store cache bit patterns."""
    kb = bits_view(w.k.contiguous())
    vb = bits_view(w.v.contiguous())
    return ref.kv_store(kb, vb, bits_view(w.k_cache), bits_view(w.v_cache),
                        w.slot_mapping, w.block_size)


def q64(w: Workload) -> np.ndarray:
    return ref.widen(bits_view(w.q.contiguous()), w.dtype)


def expected(w: Workload):
    """Oracle output of the whole step (store, then attention) in fp64."""
    kcb, vcb = stored_bits(w)
    kc, vc = ref.widen(kcb, w.dtype), ref.widen(vcb, w.dtype)
    q = q64(w)
    if w.spec.mode == "decode":
        return ref.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale)
    return ref.prefill(q, kc, vc, w.cu_seqlens_q, w.context_lens, w.block_tables, w.scale)


def sequence_view(w: Workload, kcb: np.ndarray, vcb: np.ndarray, b: int):
    """fp64 mini-cache holding only sequence b's blocks, and its remapped
    table row; lets the oracle check one sequence of a very large pool."""
    n = int(w.context_lens[b])
    nb = ref.num_blocks(n, w.block_size)
    ids = w.block_tables[b, :nb].astype(np.int64)
    kc = ref.widen(kcb[ids], w.dtype)
    vc = ref.widen(vcb[ids], w.dtype)
    return kc, vc, np.arange(nb, dtype=np.int32)


def to_numpy_out(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()
