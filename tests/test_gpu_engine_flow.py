"""The library end to end as an engine would drive it: the C block manager
admits, grows, preempts and finishes seeded requests (shared prefixes, so
prefix-cache hits, and a pool small enough to force preemption); its
metadata feeds pkv_kv_store + pkv_paged_prefill_varlen for each prefill step
and pkv_paged_decode_step for each decode step on the GPU.  The CPU oracle
runs the same stream with its own block manager, store and attention.  Every
step's attention output is compared with the tolerance of the parity tests,
and at the end the two caches must be bit-identical."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_325_amd as pkv
from oracle import ref
from tests.bm_scenario import LibAdapter, OracleAdapter, as_plain, run_stream
from tests.gpu_helpers import announce, assert_close
from workloads import bits_view
from workloads.requests import request_stream

pytestmark = pytest.mark.gpu

HQ, HKV, D = 16, 8, 128


def _bf16(rng, *shape):
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)


class Flow:
    def __init__(self, seed: int, num_blocks: int, block_size: int):
        B = self.B = block_size
        self.rng = np.random.default_rng(seed + 1000)
        self.scale = 1.0 / np.sqrt(D)
        kc = _bf16(self.rng, num_blocks, HKV, B, D)
        vc = _bf16(self.rng, num_blocks, HKV, B, D)
        self.kc_gpu, self.vc_gpu = kc.cuda(), vc.cuda()
        self.kc_bits, self.vc_bits = bits_view(kc), bits_view(vc)
        self.num_blocks = num_blocks
        self.steps = 0

    def _store_oracle(self, k, v, slots):
        self.kc_bits, self.vc_bits = ref.kv_store(bits_view(k), bits_view(v), self.kc_bits,
                                                  self.vc_bits, np.asarray(slots), self.B)
        return ref.widen(self.kc_bits, "bf16"), ref.widen(self.vc_bits, "bf16")

    def _check_meta(self, meta):
        tables = np.asarray(meta["block_tables"])
        ctx = np.diff(meta["cu_seqlens_k"]) if "cu_seqlens_k" in meta else meta["context_lens"]
        for row, n in zip(tables, np.asarray(ctx)):
            nb = -(-int(n) // self.B)
            assert ((row[:nb] >= 0) & (row[:nb] < self.num_blocks)).all()
        s = np.asarray(meta["slot_mapping"])
        assert ((s >= 0) & (s < self.num_blocks * self.B)).all()

    def __call__(self, kind, batch, adapters):
        ora, lib = adapters
        width = max(len(lib.table(s)) for s in batch)
        self.steps += 1
        if kind == "prefill":
            m = lib.prefill_meta(batch, width)
            assert as_plain(m) == as_plain(ora.prefill_meta(batch, width))
            self._check_meta(m)
            n = int(m["cu_seqlens_q"][-1])
            q, k, v = _bf16(self.rng, n, HQ, D), _bf16(self.rng, n, HKV, D), \
                _bf16(self.rng, n, HKV, D)
            ctx = np.diff(m["cu_seqlens_k"]).astype(np.int32)
            announce(f"engine flow step {self.steps}: prefill of {len(batch)} seqs, {n} tokens")
            i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
            pkv.pkv_kv_store(k.cuda(), v.cuda(), self.kc_gpu, self.vc_gpu,
                             i32(m["slot_mapping"]))
            out = pkv.pkv_paged_prefill_varlen(
                q.cuda(), self.kc_gpu, self.vc_gpu, i32(m["cu_seqlens_q"]), m["max_seqlen_q"],
                i32(ctx), m["max_seqlen_k"], i32(m["block_tables"]), self.scale)
            kc, vc = self._store_oracle(k, v, m["slot_mapping"])
            want = ref.prefill(ref.widen(bits_view(q), "bf16"), kc, vc, m["cu_seqlens_q"], ctx,
                               m["block_tables"], self.scale)
        else:
            m = lib.decode_meta(batch, width)
            assert as_plain(m) == as_plain(ora.decode_meta(batch, width))
            self._check_meta(m)
            b = len(batch)
            q, k, v = _bf16(self.rng, b, HQ, D), _bf16(self.rng, b, HKV, D), \
                _bf16(self.rng, b, HKV, D)
            announce(f"engine flow step {self.steps}: decode of {b} seqs, "
                     f"max context {m['max_context_len']}")
            i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
            out = pkv.pkv_paged_decode_step(
                q.cuda(), k.cuda(), v.cuda(), i32(m["slot_mapping"]), self.kc_gpu, self.vc_gpu,
                i32(m["block_tables"]), i32(m["context_lens"]), m["max_context_len"], self.scale)
            kc, vc = self._store_oracle(k, v, m["slot_mapping"])
            want = ref.decode(ref.widen(bits_view(q), "bf16"), kc, vc, m["block_tables"],
                              m["context_lens"], self.scale)
        torch.cuda.synchronize()
        assert_close(out.to(torch.float64).cpu().numpy(), want, f"{kind} step {self.steps}")


# (seed, block size, pool blocks, whether the stream must preempt): pools of
# 1 024-2 048 tokens for 8 requests of up to ~1 100 tokens, so admission
# waits, decode growth preempts, and re-admitted requests hit their own
# freed, still-registered prefix blocks; the 256-token blocks of the pages
# and three other block sizes of the kernels
FLOWS = [(5, 256, 6, True), (6, 256, 6, True), (12, 16, 64, True), (9, 32, 48, True),
         (11, 512, 4, False)]


@pytest.mark.parametrize("seed,B,num_blocks,preempts", FLOWS,
                         ids=[f"seed{f[0]}-B{f[1]}" for f in FLOWS])
def test_engine_flow_matches_oracle(seed, B, num_blocks, preempts):
    reqs = request_stream(seed, 8, B, vocab=3, max_prefix_blocks=max(1, 256 // B),
                          max_suffix=300, max_decode=400)
    flow = Flow(seed, num_blocks, B)
    adapters = [OracleAdapter(num_blocks, B), LibAdapter(num_blocks, B)]
    stats = run_stream(adapters, reqs, seed, num_blocks, max_running=4, on_step=flow)
    torch.cuda.synchronize()
    assert np.array_equal(bits_view(flow.kc_gpu.cpu()), flow.kc_bits)
    assert np.array_equal(bits_view(flow.vc_gpu.cpu()), flow.vc_bits)
    assert stats["finished"] == len(reqs) and stats["cached_tokens"] > 0
    assert stats["freed_hits"] > 0
    if preempts:
        assert stats["preemptions"] > 0
    announce(f"engine flow seed {seed} block size {B}: {stats}")
