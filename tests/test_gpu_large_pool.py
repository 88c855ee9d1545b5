"""GPU: a KV pool larger than 4 GiB per cache (architecture page, "Dynamische
KV-Cache-Allokation": the cache is sized to the GPU's free memory, so block
ids index far past 2^32 bytes).  A small seeded workload is laid out in a
pool of 12 288 bf16 blocks per cache (6 GiB each at 8 kv heads, 3.2 * 10^9
elements, past the int32 element range too), with its blocks placed on both
sides of the 4 GiB byte offset and on the last block of the pool.  The pool is
built on the GPU only: the workload's own blocks are copied to their new
places, every other block holds NaN poison.  The store must be bit-exact and
leave the poison alone; decode, the fused decode step and the paged prefill
must match the oracle on the workload's own (small) cache -- the same logical
K/V."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_325_amd as pkv
from tests.gpu_helpers import announce, assert_close, attend, check_inputs, store, to_device
from tests.oracle_helpers import expected, stored_bits
from workloads import Spec, bits_view, build

pytestmark = pytest.mark.gpu

POOL = 12288  # blocks per cache: 6 GiB at 256 rows x 8 kv heads x 128 dims x 2 bytes
FOUR_GIB_BLOCK = (4 << 30) // (256 * 8 * 128 * 2)  # first block at or past 4 GiB (8192)
POISON = 0x7FC0


def _placement(w, seed: int) -> np.ndarray:
    """New ids for the workload's physical blocks: blocks the tables use get
    the two blocks on either side of the 4 GiB offset and the pool's last
    block first, then distinct random ids below and above the offset."""
    rng = np.random.default_rng(seed)
    n_small = w.num_blocks
    used = rng.permutation(np.unique(w.block_tables[w.block_tables >= 0]))
    assert len(used) >= 3
    must = np.array([FOUR_GIB_BLOCK - 1, FOUR_GIB_BLOCK, POOL - 1])
    low = rng.choice(np.arange(0, FOUR_GIB_BLOCK - 1), size=n_small // 3, replace=False)
    high = rng.choice(np.arange(FOUR_GIB_BLOCK + 1, POOL - 1), size=n_small, replace=False)
    others = rng.permutation(np.setdiff1d(np.concatenate([low, high]), must))[: n_small - 3]
    order = np.concatenate([used, np.setdiff1d(np.arange(n_small), used)])
    place = np.empty(n_small, dtype=np.int64)
    place[order] = np.concatenate([must, others])
    assert len(np.unique(place)) == n_small
    return place


@pytest.fixture(autouse=True)
def _release_pool():
    yield
    torch.cuda.empty_cache()


def _big_pool(d, place: np.ndarray):
    """The device workload re-laid out in a POOL-block cache: block p of the
    small pool becomes block place[p]; tables and slots follow."""
    w = d.w
    shape = (POOL,) + tuple(d.k_cache.shape[1:])
    free = torch.cuda.mem_get_info()[0]
    need = 2 * POOL * int(np.prod(shape[1:])) * 2
    if free < need + (4 << 30):
        pytest.skip(f"needs {need / 2**30:.1f} GiB of free device memory")
    kb = torch.full(shape, POISON, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vb = torch.full(shape, POISON, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    pl = torch.from_numpy(place).cuda()
    kb[pl] = d.k_cache
    vb[pl] = d.v_cache
    bt = w.block_tables.astype(np.int64)
    bt_big = np.where(bt >= 0, place[np.maximum(bt, 0)], -1).astype(np.int32)
    B = w.block_size
    s = w.slot_mapping.astype(np.int64)
    s_big = np.where(s >= 0, place[np.maximum(s, 0) // B] * B + np.maximum(s, 0) % B, -1)
    assert s_big.max() < POOL * B and bt_big.max() < POOL
    big = dataclasses.replace(
        d, k_cache=kb, v_cache=vb,
        block_tables=torch.from_numpy(np.ascontiguousarray(bt_big)).cuda(),
        slot_mapping=torch.from_numpy(s_big.astype(np.int32)).cuda())
    return big, pl


def _small_view(cache: torch.Tensor, pl: torch.Tensor) -> np.ndarray:
    return bits_view(cache[pl].cpu())


def _untouched(cache: torch.Tensor, pl: torch.Tensor) -> bool:
    used = torch.zeros(POOL, dtype=torch.bool, device="cuda")
    used[pl] = True
    # blocks next to used ones (both sides of 4 GiB included) and a sample
    probe = torch.tensor(sorted({0, FOUR_GIB_BLOCK - 2, FOUR_GIB_BLOCK + 1, POOL - 2}
                                | set(range(FOUR_GIB_BLOCK - 64, FOUR_GIB_BLOCK + 64))),
                         device="cuda")
    probe = probe[~used[probe]]
    return bool((cache[probe].view(torch.int16) == POISON).all())


DECODE = Spec("big-pool-decode", "decode", "bf16", 32, 8,
              [4097, 1, 300, 2048, 8000, 513, 256, 6000], [1] * 8, 9401)
PREFILL = Spec("big-pool-prefill", "prefill", "bf16", 32, 8, [2600, 1024 + 300, 700],
               [2600, 300, 700], 9402, share_group=[-1, 0, -1], shared_blocks=[0, 4, 0])


def test_decode_and_store_past_4gib():
    w = build(DECODE)
    d = to_device(w)
    check_inputs(d)
    big, pl = _big_pool(d, _placement(w, 1))
    announce("pool past 4 GiB: store + decode")
    store(big)
    out = attend(big)
    torch.cuda.synchronize()
    kcb, vcb = stored_bits(w)
    assert np.array_equal(_small_view(big.k_cache, pl), kcb)
    assert np.array_equal(_small_view(big.v_cache, pl), vcb)
    assert _untouched(big.k_cache, pl) and _untouched(big.v_cache, pl)
    want = expected(w)
    assert_close(out.double().cpu().numpy(), want, "decode, pool past 4 GiB")
    for splits in (1, 7):
        announce(f"pool past 4 GiB: decode with {splits} splits")
        o = attend(big, num_splits=splits)
        torch.cuda.synchronize()
        assert_close(o.double().cpu().numpy(), want, f"decode, {splits} splits")


def test_fused_step_past_4gib():
    w = build(DECODE)
    d = to_device(w)
    check_inputs(d)
    big, pl = _big_pool(d, _placement(w, 2))
    announce("pool past 4 GiB: fused decode step")
    out = pkv.pkv_paged_decode_step(big.q, big.k, big.v, big.slot_mapping, big.k_cache,
                                    big.v_cache, big.block_tables, big.context_lens,
                                    w.max_context_len, w.scale)
    torch.cuda.synchronize()
    kcb, vcb = stored_bits(w)
    assert np.array_equal(_small_view(big.k_cache, pl), kcb)
    assert np.array_equal(_small_view(big.v_cache, pl), vcb)
    assert_close(out.double().cpu().numpy(), expected(w), "fused step, pool past 4 GiB")


def test_prefill_past_4gib():
    w = build(PREFILL)
    d = to_device(w)
    check_inputs(d)
    big, pl = _big_pool(d, _placement(w, 3))
    announce("pool past 4 GiB: store + paged prefill")
    store(big)
    out = attend(big)
    torch.cuda.synchronize()
    kcb, vcb = stored_bits(w)
    assert np.array_equal(_small_view(big.k_cache, pl), kcb)
    assert_close(out.double().cpu().numpy(), expected(w), "prefill, pool past 4 GiB")
