"""The seeded generators: reproducible, and shaped as the workloads require."""

import numpy as np
import pytest
import torch

from workloads import POISON_BITS, SENTINEL_BITS, bits_view, build, config, config_specs, small_specs


def _check_structure(w):
    B = w.block_size
    # every used table entry is a valid pool index, padding is -1
    for b in range(w.batch):
        nb = (int(w.context_lens[b]) + B - 1) // B
        row = w.block_tables[b]
        assert (row[:nb] >= 0).all() and (row[:nb] < w.num_blocks).all()
        assert (row[nb:] == -1).all()
    # no physical block is used by two sequences unless it is a shared block
    owners = {}
    for b in range(w.batch):
        nb = (int(w.context_lens[b]) + B - 1) // B
        for p in w.block_tables[b, :nb]:
            owners.setdefault(int(p), set()).add(b)
    for p, who in owners.items():
        if len(who) > 1:
            assert p in w.shared_physical
    # slots: distinct, inside the pool, inside the owning sequence's private block
    s = w.slot_mapping[w.slot_mapping >= 0]
    assert len(np.unique(s)) == len(s)
    assert (s < w.num_blocks * B).all()
    for p in (s // B):
        assert int(p) not in w.shared_physical
    # cache cells: sentinel exactly at store targets, poison outside contexts
    kb = bits_view(w.k_cache)
    sent, poison = SENTINEL_BITS[w.dtype], POISON_BITS[w.dtype]
    for slot in s:
        p, o = divmod(int(slot), B)
        assert (kb[p, :, o] == sent).all()
    used = np.zeros((w.num_blocks, B), dtype=bool)
    for b in range(w.batch):
        n = int(w.context_lens[b])
        for j in range(n):
            used[w.block_tables[b, j // B], j % B] = True
    assert (kb.transpose(0, 2, 1, 3)[~used] == poison).all()
    inside = kb.transpose(0, 2, 1, 3)[used]
    assert not ((inside == poison).all(axis=(1, 2))).any()


@pytest.mark.parametrize("spec", small_specs(), ids=lambda s: s.name)
def test_small_specs_structure(spec):
    _check_structure(build(spec))


def test_reproducible():
    a = build(small_specs()[0])
    b = build(small_specs()[0])
    assert torch.equal(a.qkv, b.qkv)
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))
    assert np.array_equal(a.block_tables, b.block_tables)


def test_config1_shape():
    w = config(1)
    assert w.dtype == "fp32" and w.num_blocks == 16
    assert list(w.context_lens) == [17, 256, 300, 511]
    assert (w.block_tables >= 0).sum() == 6
    assert w.num_q_heads == 16 and w.num_kv_heads == 8
    _check_structure(w)


def test_config_structures_without_values():
    # lengths and sharing rules of the larger workloads (structure only)
    s2, _ = config_specs(2)
    assert len(s2.context_lens) == 64 and min(s2.context_lens) >= 512 and max(s2.context_lens) <= 4096
    assert len(s2.skip) == 3
    s3, _ = config_specs(3)
    assert all(1024 <= L <= 4096 for L in s3.context_lens)
    assert [L - n for L, n in zip(s3.context_lens, s3.new_tokens)] == [512] * 8
    s4, _ = config_specs(4)
    assert len(s4.context_lens) == 256 and s4.num_q_heads == 32
    s5, _ = config_specs(5)
    assert all(256 <= c <= 32768 for c in s5.context_lens)
    assert s5.share_group == [b // 4 for b in range(16)]


@pytest.mark.slow
def test_config3_sharing():
    w = config(3)
    _check_structure(w)
    assert len(w.shared_physical) == 2
    assert (w.block_tables[:, :2] == np.array(w.shared_physical)).all()
    assert w.num_tokens == int(sum(w.spec.new_tokens))
