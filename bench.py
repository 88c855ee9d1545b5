"""Benchmark of the paged KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle S] [--workload 4]
                    [--no-extra] [--no-cpu] [--cpu-budget S] [--copy-calibration]

One step = the whole per-layer hot path over one batch of the workload: the
store of this step's K/V tokens into the cache, then attention over the cache,
inputs already resident in HBM.  For decode workloads the headline step is the
one call ``pkv_paged_decode_step`` (the store fused into the decode kernel,
bitwise equal to the two calls); the same step as ``pkv_kv_store`` then
``pkv_paged_decode`` is timed too and reported under ``separate_calls``, with a
per-kernel breakdown.  The prefill workload's step is ``pkv_kv_store`` then
``pkv_paged_prefill_varlen``.  Before every step (warm-up and timed) a 1 GiB buffer
is *read* (a row-wise max) to evict the 256 MB MALL, so every step reads the
KV cache from HBM.  The eviction reads rather than writes: a write would leave
up to 256 MB of dirty lines whose write-back would then be charged to the
measured step.  Before the warm-up steps the step runs back to back for
``--settle`` seconds (default 1) so that the GPU has left its idle clocks.
Every launch is timed with HIP events recorded on the stream the kernels run
on, which excludes the eviction; figures are medians over the timed steps.
The timed region (K steps) is bracketed by device synchronisation.

The headline line is the largest workload, the 256-sequence bf16 decode
layer (context lengths U[1024, 8192], 32 q / 8 kv heads, 4.8 GB of K/V).
``value`` is the step's algorithmic bytes (stored K/V rows read and written,
the context's K and V, q and out) per second.  ``roofline`` covers the
dominant kernel, the decode split kernel: its algorithmic bytes per launch
over its mean event-timed duration (the figure rocprofv3's average is
compared with), against the 8 TB/s HBM peak.  ``headline`` and ``extra``
give every workload's times and the fraction of its roofline each part
reaches (decode: the partials kernel, partials + merge, the fused step, and
for the prefix-shared workload the same on unique bytes; prefill: against
the 2.5 PFLOP/s dense bf16 MFMA peak).  ``cpu_baseline`` times the CPU oracle
as it stands on the host's cores (the headline workload, and every other one
under ``per_workload``), bounded to ``--cpu-budget`` seconds of work each,
with the core count and the sample stated.  ``extra`` also holds a 28-layer
decode step (one fused step per layer, each layer with its own cache)
launched eagerly and replayed from one captured graph
(``decode-step-28-layers``; the 4-sequence fp32 workload, batches of 1, 4
and 16 of the 64-sequence workload's sequences, and all 64), the 64-sequence
decode and the prefill with cache blocks of 16, 32, 64 and 1024 tokens
(``block-size-study``: attention time and fragmentation), the 256-sequence
and long-context decode and the prefill at one GPU's share of 8-way tensor
parallelism (4 query heads, 1 kv head; ``tp8-per-rank``), and the host time
of the block manager (C++ through the binding) for one decode step of 256
sequences and one prefill admission of 8 prompts; the oracle's time for the
same appears under ``cpu_baseline.block_manager``.
Prints exactly one JSON line on stdout.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
FLUSH_BYTES = 1 << 30

METRIC = "paged decode KV GB/s (% HBM peak) + tokens/s; prefill TFLOP/s (% MFMA peak)"


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


class Device:
    """Workload tensors on the GPU (the generator's CPU tensors, copied)."""

    def __init__(self, w, torch):
        import numpy as np

        self.w = w
        dev = "cuda"

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

        self.qkv = w.qkv.to(dev)
        self.k_cache = w.k_cache.to(dev)
        self.v_cache = w.v_cache.to(dev)
        self.slot_mapping = i32(w.slot_mapping)
        self.block_tables = i32(w.block_tables)
        self.context_lens = i32(w.context_lens)
        self.cu_seqlens_q = i32(w.cu_seqlens_q)
        hq, hkv = w.num_q_heads, w.num_kv_heads
        self.q = self.qkv[:, :hq]
        self.k = self.qkv[:, hq : hq + hkv]
        self.v = self.qkv[:, hq + hkv : hq + 2 * hkv]
        self.out = torch.empty((w.num_tokens, hq, w.head_dim), dtype=w.torch_dtype, device=dev)
        self.workspace = None
        if w.spec.mode == "decode":
            import paged_kv_cache_325_amd as pkv

            need = pkv.pkv_paged_decode_workspace_bytes(w.batch, hq, hkv, w.head_dim,
                                                        w.max_context_len, w.block_size, 0)
            if need:
                self.workspace = torch.zeros(need // 4, dtype=torch.float32, device=dev)

    def check(self):
        """Host-side check of every index the kernels will follow."""
        import numpy as np

        w = self.w
        B = w.block_size
        nb = -(-w.context_lens.astype(np.int64) // B)
        assert (nb <= w.block_tables.shape[1]).all()
        for b in range(w.batch):
            row = w.block_tables[b, : nb[b]]
            assert ((row >= 0) & (row < w.num_blocks)).all()
        s = w.slot_mapping
        assert ((s == -1) | ((s >= 0) & (s < w.num_blocks * B))).all()

    def store(self):
        import paged_kv_cache_325_amd as pkv

        pkv.pkv_kv_store(self.k, self.v, self.k_cache, self.v_cache, self.slot_mapping)

    def attend_parts(self):
        """The attention call as its kernel launches, in order: decode is the
        split-K partials kernel then the merge kernel; prefill is one kernel."""
        import paged_kv_cache_325_amd as pkv

        w = self.w
        if w.spec.mode == "decode":
            def partials():
                pkv.pkv_paged_decode_partials(self.q, self.k_cache, self.v_cache,
                                              self.block_tables, self.context_lens,
                                              w.max_context_len, w.scale, out=self.out,
                                              workspace=self.workspace)

            def merge():
                pkv.pkv_paged_decode_merge(self.context_lens, w.max_context_len, w.num_q_heads,
                                           w.num_kv_heads, w.block_size, self.out,
                                           self.workspace)

            return [partials, merge]

        def prefill():
            pkv.pkv_paged_prefill_varlen(self.q, self.k_cache, self.v_cache, self.cu_seqlens_q,
                                         w.max_seqlen_q, self.context_lens, w.max_context_len,
                                         self.block_tables, w.scale, out=self.out)

        return [prefill]

    def attend(self):
        for part in self.attend_parts():
            part()


def make_flush(torch):
    """A read-only MALL eviction: row-wise max over a 1 GiB buffer."""
    buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda").view(4096, -1)
    return lambda: torch.amax(buf, dim=1)


def time_steps(d: Device, steps: int, warmup: int, torch, settle_s: float = 0.0):
    """Per-step event times in ms, MALL evicted before each step: the store,
    then each attention launch (decode: partials, merge; prefill: one).

    Before the warm-up steps the step runs back to back for ``settle_s``
    seconds: an idle GPU takes a while to reach its steady clocks, and a few
    warm-up steps do not cover that ramp."""
    flush = make_flush(torch)
    stream = torch.cuda.current_stream()
    parts = d.attend_parts()
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            flush()
            d.store()
            for p in parts:
                p()
        torch.cuda.synchronize()
    for i in range(warmup):
        flush()
        d.store()
        for p in parts:
            p()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + len(parts))]
           for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        flush()
        evs[i][0].record(stream)
        d.store()
        evs[i][1].record(stream)
        for j, p in enumerate(parts):
            p()
            evs[i][2 + j].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    store_ms = [e[0].elapsed_time(e[1]) for e in evs]
    part_ms = [[e[1 + j].elapsed_time(e[2 + j]) for e in evs] for j in range(len(parts))]
    del flush
    return store_ms, part_ms, wall


def mean(x):
    return sum(x) / len(x)


def median(x):
    y = sorted(x)
    n = len(y)
    return y[n // 2] if n % 2 else 0.5 * (y[n // 2 - 1] + y[n // 2])


def time_fused_step(d: Device, steps: int, warmup: int, torch):
    """The decode step as one call (pkv_paged_decode_step: store fused into
    the decode): ``warmup`` untimed steps, then exactly ``steps`` timed ones
    between device synchronisations, MALL evicted before each step as in
    time_steps.  Returns (median event-timed ms, wall seconds of the timed
    region, median ms of the same step replayed from a captured graph)."""
    import paged_kv_cache_325_amd as pkv

    w = d.w

    def step():
        pkv.pkv_paged_decode_step(d.q, d.k, d.v, d.slot_mapping, d.k_cache, d.v_cache,
                                  d.block_tables, d.context_lens, w.max_context_len, w.scale,
                                  out=d.out, workspace=d.workspace)

    flush = make_flush(torch)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(max(warmup, 1)):
            flush()
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        t0 = time.perf_counter()
        for e0, e1 in evs:
            flush()
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return median([e0.elapsed_time(e1) for e0, e1 in evs]), wall

    eager_ms, wall = timed(step)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    graph_ms, _ = timed(graph.replay)
    del flush
    return eager_ms, wall, graph_ms


def time_prefix_decode(d: Device, steps: int, warmup: int, torch):
    """The shared-prefix decode of a workload whose tables share leading
    blocks: the plan is built on the host from the host tables and lengths
    (metadata, outside the timed region), then pkv_paged_decode_prefix (the
    attention: split kernel with the plan's MFMA workgroups, and the merge)
    and pkv_paged_decode_step_prefix (with the fused store) are each timed
    ``steps`` times, MALL evicted before each, medians in ms.  None if the
    plan shares nothing."""
    import paged_kv_cache_325_amd as pkv

    w = d.w
    S = pkv.pkv_paged_decode_split_tokens(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                          w.max_context_len, w.block_size, 0)
    plan, items = pkv.pkv_decode_prefix_plan(w.block_tables, w.context_lens, w.num_q_heads,
                                             w.num_kv_heads, w.block_size, S)
    if items == 0:
        return None
    plan = plan.cuda()

    def attn():
        pkv.pkv_paged_decode_prefix(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                    w.max_context_len, w.scale, plan, items, out=d.out,
                                    workspace=d.workspace)

    def step():
        pkv.pkv_paged_decode_step_prefix(d.q, d.k, d.v, d.slot_mapping, d.k_cache, d.v_cache,
                                         d.block_tables, d.context_lens, w.max_context_len,
                                         w.scale, plan, items, out=d.out, workspace=d.workspace)

    flush = make_flush(torch)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(max(warmup, 1)):
            flush()
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for e0, e1 in evs:
            flush()
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return median([e0.elapsed_time(e1) for e0, e1 in evs])

    d.store()
    out = {"items": items, "split_tokens": S, "attn_ms": timed(attn), "step_ms": timed(step)}
    del flush
    return out


def prefix_sharing_study(torch, steps: int = 10, warmup: int = 3) -> dict:
    """Where the shared-prefix decode pays: 64 sequences of 7000-9000 keys
    (32 / 8 heads, bf16, 256-token blocks) whose first 6144 keys are shared
    in groups of 4, i.e. 2.3x fewer distinct K/V bytes than logical ones.
    The plain decode and the shared-prefix decode (attention calls), median
    event-timed ms, MALL evicted before each."""
    import numpy as np

    import paged_kv_cache_325_amd as pkv
    from workloads import Spec, build

    rng = np.random.default_rng(325_600)
    ctx = rng.integers(7000, 9000, size=64, endpoint=True).tolist()
    w = build(Spec("decode-bf16-b64-ctx7000-9000-shared6144-groups4-h32-8", "decode", "bf16", 32,
                   8, ctx, [1] * 64, 325_601, share_group=[b // 4 for b in range(64)],
                   shared_blocks=[24] * 64))
    d = Device(w, torch)
    d.check()
    d.store()
    flush = make_flush(torch)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            flush()
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for e0, e1 in evs:
            flush()
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return median([e0.elapsed_time(e1) for e0, e1 in evs])

    plain_ms = timed(lambda: pkv.pkv_paged_decode(d.q, d.k_cache, d.v_cache, d.block_tables,
                                                  d.context_lens, w.max_context_len, w.scale,
                                                  out=d.out, workspace=d.workspace))
    pre = time_prefix_decode(d, steps, warmup, torch)
    uniq = w.unique_kv_bytes() + w.qo_bytes()
    logical = w.logical_kv_bytes() + w.qo_bytes()
    res = {"workload": w.spec.name, "logical_bytes": logical, "unique_bytes": uniq,
           "plain_decode_ms": round(plain_ms, 4),
           "plain_unique_hbm_frac": round(uniq / (plain_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "prefix_items": pre["items"], "prefix_decode_ms": round(pre["attn_ms"], 4),
           "prefix_unique_hbm_frac": round(uniq / (pre["attn_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                           4),
           "prefix_fused_step_ms": round(pre["step_ms"], 4)}
    del d, flush
    torch.cuda.empty_cache()
    return res


def decode_batch_bucket(nb: int):
    """The first ``nb`` sequences of the 64-sequence decode workload (same
    lengths, seed and head counts): the batch of one graph bucket."""
    from workloads import Spec, build, config_specs

    spec, _ = config_specs(2)
    ctx = spec.context_lens[:nb]
    return build(Spec(f"decode-bf16-b{nb}-ctx512-4096-h16-8", "decode", "bf16", spec.num_q_heads,
                      spec.num_kv_heads, ctx, [1] * nb, spec.seed))


def time_layer_stack(torch, w, layers: int = 28, reps: int = 20) -> dict:
    """A model's decode step is one pkv_paged_decode_step per layer: the
    step of ``layers`` layers (each with its own K/V cache, the same batch)
    launched eagerly and replayed from one captured HIP graph, mean
    event-timed microseconds per layer.  At small batch the eager step is
    launch-bound and the graph removes the per-launch overhead (the pages
    capture the decode step in graphs for this reason)."""
    import paged_kv_cache_325_amd as pkv

    d = Device(w, torch)
    caches = [(d.k_cache.clone(), d.v_cache.clone()) for _ in range(layers)]

    def step_all():
        for kc, vc in caches:
            pkv.pkv_paged_decode_step(d.q, d.k, d.v, d.slot_mapping, kc, vc, d.block_tables,
                                      d.context_lens, w.max_context_len, w.scale, out=d.out,
                                      workspace=d.workspace)

    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return median([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e3 / layers

    eager_us = timed(step_all)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step_all()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_all()
    torch.cuda.synchronize()
    graph_us = timed(graph.replay)
    del graph, caches, d
    torch.cuda.empty_cache()
    return {"workload": w.spec.name, "layers": layers, "eager_us_per_layer": round(eager_us, 2),
            "graph_us_per_layer": round(graph_us, 2)}


# HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE runs (KiB per
# dispatch, scaled by the same counters on a plain 256 MiB device copy), with
# the sha256 of the kernel source they were taken on: once the source
# changes, the figure no longer describes the kernel and is reported as null.
TRAFFIC = {
    ("decode_split_kernel", "decode-bf16-b256-ctx1024-8192-h32-8"): {
        "bytes": 4844618811, "source": "decode.hip",
        "sha256": "b64697fe84a19af58d02c3e4a18983fbb38da73e634959b6f57779efacce1407"},
    ("decode_split_kernel", "decode-bf16-b64-ctx512-4096-h16-8"): {
        "bytes": 545483092, "source": "decode.hip",
        "sha256": "b64697fe84a19af58d02c3e4a18983fbb38da73e634959b6f57779efacce1407"},
    ("decode_split_kernel", "decode-bf16-b16-lognormal8192-shared4096-h32-8"): {
        "bytes": 616375385, "source": "decode.hip",
        "sha256": "b64697fe84a19af58d02c3e4a18983fbb38da73e634959b6f57779efacce1407"},
    ("decode_split_kernel", "decode-fp32-4seq"): {
        "bytes": 9229930, "source": "decode.hip",
        "sha256": "b64697fe84a19af58d02c3e4a18983fbb38da73e634959b6f57779efacce1407"},
    ("prefill_kernel", "prefill-bf16-8seq-L1024-4096-prefix512-h32-8"): {
        "bytes": 2074232850, "source": "prefill.hip",
        "sha256": "d6349ec4a18e79c3d90a65b94067f1dc170db6e80ffbbb8c5952a5a2f1cd7029"},
}


def traffic_for(kernel: str, workload: str):
    import hashlib

    rec = TRAFFIC.get((kernel, workload))
    if rec is None:
        return None
    src = os.path.join(ROOT, "paged_kv_cache_325_amd", "csrc", rec["source"])
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["sha256"]:
            return None
    return rec["bytes"]


def time_contiguous_prefill(d: Device, steps: int, torch, settle_s: float = 0.5):
    """pkv_prefill_varlen (keys from contiguous rows, no block table) on the
    same keys as the paged prefill: every context row gathered once from the
    cache (after the store) into [total_k, Hkv, D].  Mean event-timed ms,
    MALL evicted before each launch, after ``settle_s`` seconds of
    back-to-back launches (the gather leaves the GPU idle long enough for its
    clocks to drop)."""
    import numpy as np

    import paged_kv_cache_325_amd as pkv

    w = d.w
    blk, row = [], []
    for b in range(w.batch):
        j = np.arange(int(w.context_lens[b]))
        blk.append(w.block_tables[b][j // w.block_size])
        row.append(j % w.block_size)
    blk = torch.from_numpy(np.concatenate(blk).astype(np.int64)).cuda()
    row = torch.from_numpy(np.concatenate(row).astype(np.int64)).cuda()
    d.store()
    k = d.k_cache[blk, :, row, :].contiguous()
    v = d.v_cache[blk, :, row, :].contiguous()
    cu_k = torch.from_numpy(
        np.concatenate([[0], np.cumsum(w.context_lens)]).astype(np.int32)).cuda()
    out = torch.empty_like(d.out)

    def run():
        pkv.pkv_prefill_varlen(d.q, k, v, d.cu_seqlens_q, cu_k, w.max_seqlen_q, w.scale, out=out)

    flush = make_flush(torch)
    stream = torch.cuda.current_stream()
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            run()
        torch.cuda.synchronize()
    for _ in range(3):
        flush()
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        flush()
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    del flush, k, v
    return median([e0.elapsed_time(e1) for e0, e1 in evs])


def measure(w, steps: int, warmup: int, torch, settle_s: float):
    """Event-timed store, attention launches and (decode) fused step of one
    workload, MALL evicted before every step; medians over the timed steps,
    plus the mean duration of the roofline kernel (the one rocprofv3's
    average is compared with)."""
    d = Device(w, torch)
    d.check()
    store_ms, part_ms, wall = time_steps(d, steps, warmup, torch, settle_s)
    attn_ms = [sum(x) for x in zip(*part_ms)]
    step_ms = [a + b for a, b in zip(store_ms, attn_ms)]
    r = {
        "w": w,
        "store_ms": median(store_ms),
        "attn_ms": median(attn_ms),
        "part_ms": [median(p) for p in part_ms],
        "part_mean_ms": [mean(p) for p in part_ms],
        "step_ms": median(step_ms),
        "wall_s": wall,
    }
    kv = w.logical_kv_bytes()
    if w.spec.mode == "decode":
        (r["fused_step_ms"], r["fused_wall_s"],
         r["fused_step_graph_ms"]) = time_fused_step(d, steps, warmup, torch)
        if w.dtype == "bf16" and w.spec.share_group:
            r["prefix"] = time_prefix_decode(d, steps, warmup, torch)
        attn_bytes = kv + w.qo_bytes()
        r["attn_bytes"] = attn_bytes
        r["unique_attn_bytes"] = w.unique_kv_bytes() + w.qo_bytes()
        r["attn_gbs"] = attn_bytes / (r["attn_ms"] * 1e-3) / 1e9
        r["unique_gbs"] = r["unique_attn_bytes"] / (r["attn_ms"] * 1e-3) / 1e9
        # the partials kernel reads every context K/V row and q
        r["split_bytes"] = kv + w.qo_bytes() // 2
        r["split_gbs"] = r["split_bytes"] / (r["part_mean_ms"][0] * 1e-3) / 1e9
    else:
        r["flops"] = w.prefill_flops()
        r["tflops"] = r["flops"] / (r["attn_ms"] * 1e-3) / 1e12
        r["tflops_mean"] = r["flops"] / (r["part_mean_ms"][0] * 1e-3) / 1e12
        r["contiguous_ms"] = time_contiguous_prefill(d, max(5, steps // 2), torch)
        r["contiguous_tflops"] = r["flops"] / (r["contiguous_ms"] * 1e-3) / 1e12
        # prefill reads each unique cached K/V byte at least once
        r["attn_bytes"] = w.unique_kv_bytes() + w.qo_bytes()
    r["step_bytes"] = w.store_bytes() + r["attn_bytes"]
    r["step_gbs"] = r["step_bytes"] / (r["step_ms"] * 1e-3) / 1e9
    if "fused_step_ms" in r:
        r["fused_step_gbs"] = r["step_bytes"] / (r["fused_step_ms"] * 1e-3) / 1e9
    r["store_gbs"] = w.store_bytes() / (r["store_ms"] * 1e-3) / 1e9 if r["store_ms"] > 0 else None
    del d
    torch.cuda.empty_cache()
    return r


def summary(r) -> dict:
    """Per-workload line of ``extra``: times (medians) and the fraction of
    the roofline each part reaches."""
    w = r["w"]
    e = {"step_ms": round(r["step_ms"], 4), "store_ms": round(r["store_ms"], 4),
         "attn_ms": round(r["attn_ms"], 4)}
    if w.spec.mode == "prefill":
        e.update(hbm_traffic_bytes=traffic_for("prefill_kernel", w.spec.name))
        e.update(prefill_tflops=round(r["tflops"], 1),
                 mfma_frac=round(r["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                 prefill_tokens_per_s=round(w.num_tokens / (r["attn_ms"] * 1e-3), 1),
                 contiguous_kv_ms=round(r["contiguous_ms"], 4),
                 contiguous_kv_tflops=round(r["contiguous_tflops"], 1),
                 contiguous_kv_mfma_frac=round(r["contiguous_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4))
        return e
    e.update(partials_hbm_traffic_bytes=traffic_for("decode_split_kernel", w.spec.name))
    e.update(decode_gbs=round(r["attn_gbs"], 1),
             decode_hbm_frac=round(r["attn_gbs"] / HBM_PEAK_GBS, 4),
             partials_ms=round(r["part_ms"][0], 4),
             partials_hbm_frac=round(r["split_bytes"] / (r["part_ms"][0] * 1e-3) / 1e9
                                     / HBM_PEAK_GBS, 4),
             merge_ms=round(r["part_ms"][1], 4) if len(r["part_ms"]) > 1 else None,
             decode_tokens_per_s=round(w.batch / (r["attn_ms"] * 1e-3), 1),
             fused_step_ms=round(r["fused_step_ms"], 4),
             fused_step_gbs=round(r["fused_step_gbs"], 1),
             fused_step_hbm_frac=round(r["fused_step_gbs"] / HBM_PEAK_GBS, 4),
             fused_step_graph_ms=round(r["fused_step_graph_ms"], 4))
    if r["unique_attn_bytes"] != r["attn_bytes"]:
        e.update(decode_unique_gbs=round(r["unique_gbs"], 1),
                 decode_unique_hbm_frac=round(r["unique_gbs"] / HBM_PEAK_GBS, 4))
    pre = r.get("prefix")
    if pre:
        ub = r["unique_attn_bytes"]
        e.update(prefix_plan_items=pre["items"], prefix_decode_ms=round(pre["attn_ms"], 4),
                 prefix_decode_unique_gbs=round(ub / (pre["attn_ms"] * 1e-3) / 1e9, 1),
                 prefix_decode_unique_hbm_frac=round(ub / (pre["attn_ms"] * 1e-3) / 1e9
                                                     / HBM_PEAK_GBS, 4),
                 prefix_fused_step_ms=round(pre["step_ms"], 4))
    return e


def host_cores() -> int:
    """CPU threads this process may use: its affinity set, capped by
    OMP_NUM_THREADS when that is set (a shared host may grant only a share of
    its cores through it)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    omp = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(omp)) if omp.isdigit() and int(omp) > 0 else n


def cpu_baseline(w, budget_s: float = 8.0, cores: int = 0) -> dict:
    """The CPU oracle, as it stands, on one workload, on ``cores`` host
    threads.  Decode: the oracle's store, then its decode of every sequence,
    sequences spread over a pool of ``cores`` threads (one BLAS thread each;
    the oracle's per-head products are too small for BLAS threads to help),
    whole passes repeated until ``budget_s``.  Prefill: the oracle's store,
    then its prefill one sequence at a time with ``cores`` BLAS threads (the
    products are large), sequences in order until ``budget_s`` -- a sample
    whose size is stated.  Rates use the same algorithmic bytes and flops as
    the GPU figures."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import ref
    from workloads import bits_view

    cores = cores or host_cores()
    kb, vb = bits_view(w.k.contiguous()), bits_view(w.v.contiguous())
    kcb0, vcb0 = bits_view(w.k_cache), bits_view(w.v_cache)
    q = ref.widen(bits_view(w.q.contiguous()), w.dtype)
    t0 = time.perf_counter()
    kcb, vcb = ref.kv_store(kb, vb, kcb0, vcb0, w.slot_mapping, w.block_size)
    store_s = time.perf_counter() - t0

    def decode_one(b):
        n = int(w.context_lens[b])
        ids = w.block_tables[b, : ref.num_blocks(n, w.block_size)]
        kc, vc = ref.widen(kcb[ids], w.dtype), ref.widen(vcb[ids], w.dtype)
        ref.decode(q[b : b + 1], kc, vc, np.arange(len(ids), dtype=np.int32)[None],
                   w.context_lens[b : b + 1], w.scale)

    if w.spec.mode == "decode":
        passes, t1 = 0, time.perf_counter()
        with threadpool_limits(1), ThreadPoolExecutor(cores) as ex:
            while True:
                list(ex.map(decode_one, range(w.batch)))
                passes += 1
                if time.perf_counter() - t1 >= budget_s:
                    break
        dt = time.perf_counter() - t1
        nbytes = w.logical_kv_bytes() + w.qo_bytes()
        total_s = store_s + dt / passes  # one step: the store, then one decode pass
        return {
            "value": round((w.store_bytes() + nbytes) / total_s / 1e9, 4),
            "unit": "GB/s",
            "cores": cores,
            "kind": "oracle",
            "sample": f"whole workload: oracle store ({store_s:.2f} s) + decode of all {w.batch} "
                      f"sequences, {passes} pass(es) in {dt:.1f} s on a pool of {cores} "
                      f"threads, numpy fp64; value = step bytes / (store + one pass)",
            "decode_gbs": round(nbytes / (dt / passes) / 1e9, 4),
            "tokens_per_s": round(passes * w.batch / dt, 2),
        }
    kc, vc = ref.widen(kcb, w.dtype), ref.widen(vcb, w.dtype)
    done, flops, rows, t1 = 0, 0, 0, time.perf_counter()
    with threadpool_limits(cores):
        for b in range(w.batch):
            lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
            ref.prefill(q[lo:hi], kc, vc, np.array([0, hi - lo], dtype=np.int32),
                        w.context_lens[b : b + 1], w.block_tables[b : b + 1], w.scale)
            nk, nq = int(w.context_lens[b]), hi - lo
            flops += 4 * w.head_dim * w.num_q_heads * (nq * (nk - nq + 1) + nq * (nq - 1) // 2)
            rows += nq
            done += 1
            if time.perf_counter() - t1 >= budget_s:
                break
    dt = time.perf_counter() - t1
    return {
        "value": round(flops / dt / 1e9, 3),
        "unit": "GFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"oracle store of the whole workload ({store_s:.2f} s, not in the rate), "
                  f"then prefill of the first {done} of {w.batch} sequences ({rows} of "
                  f"{w.num_tokens} query rows, {flops / w.prefill_flops():.1%} of the flops) "
                  f"in {dt:.1f} s with {cores} BLAS threads, numpy fp64",
        "prefill_tokens_per_s": round(rows / dt, 2),
    }


BLOCK_SIZE_STUDY = (16, 32, 64, 1024)


def time_block_sizes(torch, steps: int = 10, warmup: int = 3) -> dict:
    """Gather efficiency against fragmentation: the 64-sequence decode and
    the prefill workload drawn with other cache block sizes (same lengths,
    same sharing in tokens), attention timed as in time_steps; fragmentation
    = unused share of the rows of the blocks the contexts occupy."""
    import dataclasses

    import numpy as np

    from workloads import build, config_specs

    out = {}
    for index in (2, 3):
        for B in BLOCK_SIZE_STUDY:
            spec, rng = config_specs(index)
            shared = [x * 256 // B for x in spec.shared_blocks] if spec.shared_blocks else None
            w = build(dataclasses.replace(spec, block_size=B, shared_blocks=shared), rng)
            d = Device(w, torch)
            d.check()
            _, part_ms, _ = time_steps(d, steps, warmup, torch, 0.3)
            attn_ms = median([sum(x) for x in zip(*part_ms)])
            blocks = int((-(-w.context_lens.astype(np.int64) // B)).sum())
            e = {"attn_ms": round(attn_ms, 4),
                 "fragmentation": round(1 - float(w.context_lens.sum()) / (blocks * B), 4)}
            if w.spec.mode == "decode":
                e["decode_gbs"] = round((w.logical_kv_bytes() + w.qo_bytes()) /
                                        (attn_ms * 1e-3) / 1e9, 1)
            else:
                e["prefill_tflops"] = round(w.prefill_flops() / (attn_ms * 1e-3) / 1e12, 1)
            out[f"{w.spec.name}@B{B}"] = e
            log(f"block size {B}, workload {index}: {e}")
            del d
            torch.cuda.empty_cache()
    return out


def time_per_rank_shapes(torch, steps: int = 10, warmup: int = 3) -> dict:
    """One GPU's share under 8-way tensor parallelism (heads split over the
    GPUs, 32/8 -> 4 query heads and 1 kv head per GPU; tables, lengths and
    slots replicated): the 256-sequence and the long-context decode and the
    prefill workload drawn with those head counts, attention timed as in
    time_steps."""
    import dataclasses

    from workloads import build, config_specs

    out = {}
    for index in (4, 5, 3):
        spec, rng = config_specs(index)
        w = build(dataclasses.replace(spec, name=f"{spec.name}-tp8-rank", num_q_heads=4,
                                      num_kv_heads=1), rng)
        d = Device(w, torch)
        d.check()
        _, part_ms, _ = time_steps(d, steps, warmup, torch, 0.3)
        attn_ms = median([sum(x) for x in zip(*part_ms)])
        e = {"attn_ms": round(attn_ms, 4)}
        if w.spec.mode == "decode":
            gbs = (w.logical_kv_bytes() + w.qo_bytes()) / (attn_ms * 1e-3) / 1e9
            e.update(decode_gbs=round(gbs, 1), decode_hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                     partials_ms=round(median(part_ms[0]), 4))
        else:
            tf = w.prefill_flops() / (attn_ms * 1e-3) / 1e12
            e.update(prefill_tflops=round(tf, 1), mfma_frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4))
        out[w.spec.name] = e
        log(f"per-rank shape, workload {index}: {e}")
        del d
        torch.cuda.empty_cache()
    return out


# Host block manager: one engine step's bookkeeping at the shapes of the
# 256-sequence decode workload (contexts U[1024, 8192]) and of the prefill
# workload (8 prompts of U[1024, 4096] tokens behind a shared 512-token
# prefix).  Token ids are seeded random ints; they only feed the hash.
BM_BLOCK = 256


def _bm_inputs(seed: int = 325500):
    import numpy as np

    rng = np.random.default_rng(seed)
    decode = [rng.integers(0, 32000, int(n)).astype(np.int32)
              for n in rng.integers(1024, 8193, 256)]
    shared = rng.integers(0, 32000, 512).astype(np.int32)
    prefill = [np.concatenate([shared, rng.integers(0, 32000, int(n) - 512).astype(np.int32)])
               for n in rng.integers(1024, 4097, 8)]
    new_tokens = rng.integers(0, 32000, (4096, 256)).astype(np.int32)
    return decode, prefill, new_tokens


def _bm_pool(prompts, steps):
    return sum(-(-(len(p) + steps) // BM_BLOCK) for p in prompts) + 8


def time_block_manager(steps: int = 1024) -> dict:
    """The library's block manager (C++ behind the C ABI, through the Python
    binding): mean host time of one decode step of 256 sequences
    (pkv_bm_append_tokens + pkv_bm_decode_step, which crosses 256-token
    block boundaries as the sequences grow) and of one prefill admission of
    8 prompts (allocate with prefix hits + pkv_bm_build_prefill)."""
    import numpy as np

    from paged_kv_cache_325_amd.block_manager import BlockManager

    decode, prefill, new_tokens = _bm_inputs()
    m = BlockManager(_bm_pool(decode, steps), BM_BLOCK)
    ids = np.arange(len(decode), dtype=np.int64)
    for i, p in zip(ids, decode):
        m.add_sequence(int(i), p)
        m.allocate(int(i))
    width = max(-(-(len(p) + steps) // BM_BLOCK) for p in decode)
    t0 = time.perf_counter()
    for s in range(steps):
        m.append_tokens(ids, new_tokens[s % len(new_tokens)])
        m.decode_step(ids, width)
    dec_us = (time.perf_counter() - t0) / steps * 1e6
    reps = 50
    t0 = time.perf_counter()
    for r in range(reps):
        pm = BlockManager(_bm_pool(prefill, 0), BM_BLOCK)
        for i, p in enumerate(prefill):
            pm.add_sequence(i, p)
            pm.allocate(i)
        pm.build_prefill(list(range(len(prefill))))
        pm.close()
    pre_us = (time.perf_counter() - t0) / reps * 1e6
    return {"decode_step_us_batch256": round(dec_us, 2), "decode_steps": steps,
            "prefill_admission_us_8_prompts": round(pre_us, 2),
            "what": "host time through the Python binding; decode step = append_tokens + "
                    "decode_step over 256 sequences (may_append + metadata); prefill admission "
                    "= 8 x allocate (chained hashing, 512-token shared prefix hits) + "
                    "build_prefill"}


def block_manager_oracle(steps: int = 64) -> dict:
    """The same two measurements on the plain-Python oracle block manager."""
    from oracle import block_manager as obm

    decode, prefill, new_tokens = _bm_inputs()
    m = obm.BlockManager(_bm_pool(decode, steps), BM_BLOCK)
    seqs = [obm.Sequence(i, p, BM_BLOCK) for i, p in enumerate(decode)]
    for q in seqs:
        m.allocate(q)
    width = max(-(-(len(p) + steps) // BM_BLOCK) for p in decode)
    t0 = time.perf_counter()
    for s in range(steps):
        for q, t in zip(seqs, new_tokens[s]):
            q.append_token(int(t))
            m.may_append(q)
        obm.prepare_decode(seqs, width)
    dec_us = (time.perf_counter() - t0) / steps * 1e6
    reps = 3
    t0 = time.perf_counter()
    for r in range(reps):
        pm = obm.BlockManager(_bm_pool(prefill, 0), BM_BLOCK)
        ps = [obm.Sequence(i, p, BM_BLOCK) for i, p in enumerate(prefill)]
        for q in ps:
            pm.allocate(q)
        obm.prepare_prefill(ps, max(len(q.block_table) for q in ps))
    pre_us = (time.perf_counter() - t0) / reps * 1e6
    return {"decode_step_us_batch256": round(dec_us, 2), "decode_steps": steps,
            "prefill_admission_us_8_prompts": round(pre_us, 2), "cores": 1}


def copy_calibration(torch, nbytes: int = 256 << 20, reps: int = 3) -> None:
    """Plain device copies of a known size: a reference for HBM byte counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of back-to-back untimed steps before the warm-up steps, "
                         "so the GPU reaches its steady clocks")
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle work per workload for the CPU baselines")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain copies of a known size (for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the hot path is "
              "measured on one GPU's share.  Under tensor parallelism each GPU holds "
              "num_kv_heads / tp kv heads and runs the same kernels on them, with no "
              "exchange inside this path", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    import paged_kv_cache_325_amd as pkv
    from workloads import config

    pkv.load_library()  # fails loudly if the HIP library is missing
    if args.copy_calibration:
        copy_calibration(torch)

    workloads = {}

    def workload(i):
        if i not in workloads:
            t = time.perf_counter()
            workloads[i] = config(i)
            log(f"workload {i} ({workloads[i].spec.name}) generated in "
                f"{time.perf_counter() - t:.1f}s")
        return workloads[i]

    head = measure(workload(args.workload), args.steps, args.warmup, torch, args.settle)
    w = head["w"]
    log(f"headline: {summary(head)}")

    extra = {}
    if not args.no_extra:
        for idx in (1, 2, 3, 4, 5):
            if idx == args.workload:
                continue
            r = measure(workload(idx), max(3, args.steps // 2), max(1, args.warmup // 2), torch,
                        args.settle / 2)
            extra[r["w"].spec.name] = summary(r)
            log(f"workload {idx}: {extra[r['w'].spec.name]}")

    if w.spec.mode == "decode":
        roof = {"bound": "hbm", "achieved": round(head["split_gbs"], 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(head["split_gbs"] / HBM_PEAK_GBS, 4),
                "traffic": traffic_for("decode_split_kernel", w.spec.name),
                "kernel": "decode_split_kernel (pkv_paged_decode_partials)",
                "bytes_per_launch": head["split_bytes"],
                "mean_launch_ms": round(head["part_mean_ms"][0], 5),
                "median_launch_ms": round(head["part_ms"][0], 5),
                "merge_kernel_median_ms": round(head["part_ms"][1], 5)}
    else:
        roof = {"bound": "mfma", "achieved": round(head["tflops_mean"], 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(head["tflops_mean"] / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_for("prefill_kernel", w.spec.name),
                "kernel": "prefill_kernel", "flops_per_launch": head["flops"],
                "mean_launch_ms": round(head["part_mean_ms"][0], 5),
                "median_launch_ms": round(head["part_ms"][0], 5)}

    if not args.no_extra:
        log("timing a 28-layer decode step, eager and from a captured graph")
        stacks = [workload(1)] + [decode_batch_bucket(nb) for nb in (1, 4, 16)] + [workload(2)]
        extra["decode-step-28-layers"] = [time_layer_stack(torch, x) for x in stacks]
        log(f"28-layer decode step: {extra['decode-step-28-layers']}")
        log("timing other cache block sizes")
        extra["block-size-study"] = time_block_sizes(torch)
        log("timing one GPU's share of 8-way tensor parallelism")
        extra["tp8-per-rank"] = time_per_rank_shapes(torch)
        log("timing the host block manager")
        extra["block-manager-host"] = time_block_manager()
        log("timing the shared-prefix decode on a heavily shared batch")
        extra["prefix-sharing-study"] = prefix_sharing_study(torch)
        log(f"prefix sharing: {extra['prefix-sharing-study']}")

    cpu = None
    if not args.no_cpu:
        cores = host_cores()
        log(f"timing the CPU oracle on {cores} host threads")
        cpu = cpu_baseline(w, args.cpu_budget, cores)
        log(f"oracle, {w.spec.name}: {cpu}")
        if not args.no_extra:
            per = {}
            for idx in (1, 2, 3, 4, 5):
                if idx != args.workload:
                    x = workload(idx)
                    per[x.spec.name] = cpu_baseline(x, args.cpu_budget, cores)
                    log(f"oracle, {x.spec.name}: {per[x.spec.name]}")
            cpu["per_workload"] = per
            cpu["block_manager"] = block_manager_oracle()

    # The headline step: for decode the library's one-call step
    # (pkv_paged_decode_step, bitwise equal to store-then-decode); the same
    # step as separate calls is reported under "separate_calls".
    fused = "fused_step_ms" in head
    step_ms = head["fused_step_ms"] if fused else head["step_ms"]
    step_gbs = head["fused_step_gbs"] if fused else head["step_gbs"]
    wall_s = head["fused_wall_s"] if fused else head["wall_s"]
    line = {
        "metric": METRIC,
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.spec.name,
            "batch": w.batch,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "sum_context_tokens": int(w.context_lens.sum()),
            "stored_tokens": int((w.slot_mapping >= 0).sum()),
            "seed": w.spec.seed,
        },
        "step_path": ("pkv_paged_decode_step (kv_store fused into the decode)" if fused
                      else "pkv_kv_store + attention call"),
        "step_tokens_per_s": round(w.batch / (step_ms * 1e-3), 1) if fused else None,
        "headline": summary(head),
        "separate_calls": {"step_ms": round(head["step_ms"], 5),
                           "step_gbs": round(head["step_gbs"], 2),
                           "store_ms": round(head["store_ms"], 5)},
        "step_graph_replay_ms": (round(head["fused_step_graph_ms"], 5) if fused else None),
        "timing": "HIP events on the kernels' stream; medians over the timed steps (the "
                  "roofline kernel: mean, as rocprofv3 averages); 1 GiB read-only MALL eviction "
                  "before every step (outside the events); "
                  f"{args.settle:g} s of untimed back-to-back steps before the warm-up",
        "wall_s_timed_region": round(wall_s, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
