"""Run a seeded workload through the HIP library (test code only)."""

from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import paged_kv_cache_325_amd as pkv
from workloads import Workload

# spec tolerance against the fp64 oracle (bf16 or fp32 inputs, fp32 accumulation)
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


@dataclasses.dataclass
class DeviceWorkload:
    w: Workload
    qkv: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    slot_mapping: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    cu_seqlens_q: torch.Tensor

    @property
    def q(self):
        return self.qkv[:, : self.w.num_q_heads]

    @property
    def k(self):
        h = self.w.num_q_heads
        return self.qkv[:, h : h + self.w.num_kv_heads]

    @property
    def v(self):
        h = self.w.num_q_heads + self.w.num_kv_heads
        return self.qkv[:, h : h + self.w.num_kv_heads]


def announce(msg: str) -> None:
    """Name the case before each GPU step, so a fault can be attributed."""
    sys.stdout.write(f"[gpu] {msg}\n")
    sys.stdout.flush()


def to_device(w: Workload, device: str = "cuda") -> DeviceWorkload:
    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    return DeviceWorkload(
        w=w,
        qkv=w.qkv.to(device),
        k_cache=w.k_cache.to(device),
        v_cache=w.v_cache.to(device),
        slot_mapping=i32(w.slot_mapping),
        block_tables=i32(w.block_tables),
        context_lens=i32(w.context_lens),
        cu_seqlens_q=i32(w.cu_seqlens_q),
    )


def check_inputs(d: DeviceWorkload) -> None:
    """Host-side shape checks of what the kernels will index (done on the
    CPU copies before any launch)."""
    w = d.w
    B = w.block_size
    nb_needed = -(-w.context_lens.astype(np.int64) // B)
    assert (nb_needed <= w.block_tables.shape[1]).all()
    for b in range(w.batch):
        row = w.block_tables[b, : nb_needed[b]]
        assert ((row >= 0) & (row < w.num_blocks)).all()
    s = w.slot_mapping
    assert ((s == -1) | ((s >= 0) & (s < w.num_blocks * B))).all()
    assert w.max_context_len <= w.block_tables.shape[1] * B


def store(d: DeviceWorkload, stream=None) -> None:
    pkv.pkv_kv_store(d.k, d.v, d.k_cache, d.v_cache, d.slot_mapping, stream=stream)


def attend(d: DeviceWorkload, num_splits: int = 0, out=None, workspace=None, stream=None):
    w = d.w
    if w.spec.mode == "decode":
        return pkv.pkv_paged_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                    w.max_context_len, w.scale, out=out, workspace=workspace,
                                    num_splits=num_splits, stream=stream)
    return pkv.pkv_paged_prefill_varlen(d.q, d.k_cache, d.v_cache, d.cu_seqlens_q, w.max_seqlen_q,
                                        d.context_lens, w.max_context_len, d.block_tables,
                                        w.scale, out=out, stream=stream)


def errors(got: np.ndarray, want: np.ndarray):
    diff = np.abs(got.astype(np.float64) - want)
    return float(diff.max()) if diff.size else 0.0, float(diff.mean()) if diff.size else 0.0


def assert_close(got: np.ndarray, want: np.ndarray, what: str = "") -> None:
    assert np.isfinite(got).all(), f"{what}: non-finite values in the GPU result"
    mx, mean = errors(got, want)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max-abs {mx:.3g}, mean-abs {mean:.3g}"
