"""numpy fp64 definition of the paged KV-cache hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources, cited by page title and section:

* nano-vllm architecture page ("Architektur im Überblick", repothread.com),
  sections "Dynamische KV-Cache-Allokation" (cache tensor indexed by block,
  row in block, kv head, head dim), "Prefill- und Decode-Vorbereitung" (slot of
  a token = block id * block size + row; positions of uncached tokens run from
  the cached prefix length to the sequence length), "Block-Berechnung und
  Token-Appending" (number of blocks and tokens in the last block),
  "Hash-basiertes Prefix Caching" (prefix blocks are shared whole), and
  "Kern-Designentscheidungen" item 1 (block size 256).
* nano-vllm source study ("Nano-vLLM 源碼學習", hk.pswp.cn), section 2
  "注意力層": the store kernel writes k/v into the cache at slot_mapping, then
  prefill uses varlen attention over the cache and decode uses attention over
  the paged cache with per-sequence context lengths and block tables.
* essay on vLLM and nano-vllm (lshu.cn), section 3.2: logical position ->
  (page index = pos // page size, offset = pos % page size), worked example
  position 25 with page size 16 -> page index 1, offset 9; attention gathers
  K and V from the scattered pages and then computes.

The attention formula itself is softmax(scale * q . k_j) weighted sum of v_j
over the keys a query may see; the pages name the operation (decode and varlen
causal prefill) but not the formula, so the plain textbook definition is used.

Readings where the pages are silent:
  * query head h uses kv head h // (Hq / Hkv) (contiguous GQA groups);
  * the store runs before attention and ``context_lens`` counts the stored
    token; a decode query sits at position ctx - 1;
  * prefill causal alignment is bottom-right: with n_q queries and n_k keys,
    query i is at position n_k - n_q + i and sees keys 0..n_k - n_q + i;
  * ``slot_mapping == -1`` stores nothing;
  * a sequence with no visible keys produces a zero output row;
  * the cache layout of one layer is [num_blocks][num_kv_heads][block_size]
    [head_dim] (row-major), i.e. each (block, kv head) tile is contiguous.

Arrays: values are fp64 numpy arrays already widened from the stored bf16/fp32
bits with :func:`widen`; the store works on raw bit patterns.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# Element widening (exact): bf16 bits are the top half of an fp32.
# ---------------------------------------------------------------------------

def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of raw bf16 (uint16) or fp32 (uint32) bit patterns."""
    if dtype == "bf16":
        u32 = bits.astype(np.uint32) << np.uint32(16)
        return u32.view(np.float32).astype(np.float64)
    if dtype == "fp32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Block arithmetic (architecture page, "Block-Berechnung und Token-Appending";
# essay section 3.2 for the position -> (page, offset) translation).
# ---------------------------------------------------------------------------

def num_blocks(num_tokens: int, block_size: int) -> int:
    """Blocks holding ``num_tokens`` tokens: ceiling division."""
    return (num_tokens + block_size - 1) // block_size


def last_block_tokens(num_tokens: int, block_size: int) -> int:
    """Tokens in the last block of a sequence of ``num_tokens`` (>0) tokens."""
    return num_tokens - (num_blocks(num_tokens, block_size) - 1) * block_size


def locate(position: int, block_size: int) -> Tuple[int, int]:
    """Logical position -> (logical block index, row inside the block)."""
    return position // block_size, position % block_size


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``h`` (contiguous groups of Hq/Hkv heads)."""
    return h // (num_q_heads // num_kv_heads)


def visible_keys(i: int, n_q: int, n_k: int) -> int:
    """Number of keys query ``i`` of ``n_q`` sees among ``n_k`` (bottom-right
    causal alignment: the last query sees every key)."""
    return max(0, min(n_k, n_k - n_q + i + 1))


# ---------------------------------------------------------------------------
# Store (source study section 2, store kernel; architecture page, slot mapping)
# ---------------------------------------------------------------------------

def kv_store(k_bits: np.ndarray, v_bits: np.ndarray, k_cache_bits: np.ndarray,
             v_cache_bits: np.ndarray, slot_mapping: np.ndarray, block_size: int):
    """Return copies of the caches after writing token t's K and V rows (all kv
    heads) into slot ``slot_mapping[t]``; a slot of -1 writes nothing.

    Works on raw bit patterns, so the copy is exact for every value including
    NaN payloads.  k_bits/v_bits: [N, Hkv, D]; caches: [nblk, Hkv, B, D].
    Tokens are applied in order t = 0..N-1.
    """
    kc = k_cache_bits.copy()
    vc = v_cache_bits.copy()
    for t in range(slot_mapping.shape[0]):
        s = int(slot_mapping[t])
        if s == -1:
            continue
        p, o = locate(s, block_size)
        kc[p, :, o, :] = k_bits[t]
        vc[p, :, o, :] = v_bits[t]
    return kc, vc


# ---------------------------------------------------------------------------
# Gather through the block table (essay section 3.2: collect K and V from the
# scattered pages, then compute).
# ---------------------------------------------------------------------------

def gather(cache: np.ndarray, table_row: Sequence[int], n: int) -> np.ndarray:
    """Logical rows 0..n-1 of one sequence: [n, Hkv, D]."""
    B = cache.shape[2]
    nb = num_blocks(n, B)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    tiles = cache[ids]  # [nb, Hkv, B, D]
    rows = tiles.transpose(0, 2, 1, 3).reshape(nb * B, cache.shape[1], cache.shape[3])
    return rows[:n]


def _attend(qvec: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """softmax(scale * keys @ q) @ vals for one query row; returns (out, weights).
    With no keys the output is zero and the weight vector is empty."""
    if keys.shape[0] == 0:
        return np.zeros(vals.shape[1]), np.zeros(0)
    s = scale * (keys @ qvec)
    m = s.max()
    e = np.exp(s - m)
    w = e / e.sum()
    return w @ vals, w


# ---------------------------------------------------------------------------
# Decode (source study section 2: decode attention over the paged cache)
# ---------------------------------------------------------------------------

def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
           return_weights: bool = False):
    """q: [batch, Hq, D] fp64; caches [nblk, Hkv, B, D] fp64 (after the store).
    Returns out [batch, Hq, D] (and weights[b][h] arrays if asked)."""
    batch, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    out = np.zeros((batch, Hq, D))
    weights = [[None] * Hq for _ in range(batch)]
    for b in range(batch):
        n = int(context_lens[b])
        K = gather(k_cache, block_tables[b], n)
        V = gather(v_cache, block_tables[b], n)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[b, h], weights[b][h] = _attend(q[b, h], K[:, g, :], V[:, g, :], scale)
    return (out, weights) if return_weights else out


def decode_partials(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                    block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                    split_tokens: int):
    """Split-K partials: for split s of sequence b (keys s*S .. min(n,(s+1)*S)-1),
    acc = sum_j exp(x_j - m) v_j, m = max_j x_j, l = sum_j exp(x_j - m), with
    x_j = scale * q . k_j (natural-log domain).  Returns a list per sequence of
    (acc [nsplit, Hq, D], m [nsplit, Hq], l [nsplit, Hq])."""
    batch, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    res = []
    for b in range(batch):
        n = int(context_lens[b])
        K = gather(k_cache, block_tables[b], n)
        V = gather(v_cache, block_tables[b], n)
        ns = (n + split_tokens - 1) // split_tokens
        acc = np.zeros((ns, Hq, D))
        m = np.full((ns, Hq), -np.inf)
        l = np.zeros((ns, Hq))
        for s in range(ns):
            lo, hi = s * split_tokens, min(n, (s + 1) * split_tokens)
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                x = scale * (K[lo:hi, g, :] @ q[b, h])
                m[s, h] = x.max()
                e = np.exp(x - m[s, h])
                l[s, h] = e.sum()
                acc[s, h] = e @ V[lo:hi, g, :]
        res.append((acc, m, l))
    return res


def merge_partials(acc: np.ndarray, m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """Combine split partials of one sequence: M = max_s m_s,
    L = sum_s exp(m_s - M) l_s, out = sum_s exp(m_s - M) acc_s / L, summing in
    split order.  acc [ns, Hq, D], m/l [ns, Hq] -> out [Hq, D]."""
    ns, Hq, D = acc.shape
    if ns == 0:
        return np.zeros((Hq, D))
    M = m.max(axis=0)
    L = np.zeros(Hq)
    O = np.zeros((Hq, D))
    for s in range(ns):
        f = np.exp(m[s] - M)
        L += f * l[s]
        O += f[:, None] * acc[s]
    return O / L[:, None]


# ---------------------------------------------------------------------------
# Varlen causal prefill over prefix-cached blocks (source study section 2;
# architecture page, "Prefill- und Decode-Vorbereitung": the uncached tokens
# are positions num_cached_tokens .. seqlen - 1)
# ---------------------------------------------------------------------------

def _prefill_sequence(q: np.ndarray, K: np.ndarray, V: np.ndarray, lo: int, n_q: int, n_k: int,
                      scale: float, out: np.ndarray, wanted) -> None:
    """Rows lo .. lo+n_q-1 of ``out`` for one sequence whose keys are K, V
    ([n_k, Hkv, D]); bottom-right causal.  ``wanted``: None (all rows) or a
    set of global row indices."""
    Hq = q.shape[1]
    Hkv = K.shape[1]
    idx = [i for i in range(n_q) if wanted is None or (lo + i) in wanted]
    if not idx:
        return
    if wanted is not None:
        for i in idx:
            nv = visible_keys(i, n_q, n_k)
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                out[lo + i, h], _ = _attend(q[lo + i, h], K[:nv, g, :], V[:nv, g, :], scale)
        return
    # all rows of the sequence at once, one head at a time
    hi = lo + n_q
    nv = np.array([visible_keys(i, n_q, n_k) for i in range(n_q)])
    mask = np.arange(n_k)[None, :] < nv[:, None]  # [n_q, n_k]
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        S = scale * (q[lo:hi, h, :] @ K[:, g, :].T)
        S = np.where(mask, S, -np.inf)
        m = S.max(axis=1, initial=-np.inf)
        m = np.where(np.isfinite(m), m, 0.0)
        E = np.where(mask, np.exp(S - m[:, None]), 0.0)
        L = E.sum(axis=1)
        with np.errstate(invalid="ignore", divide="ignore"):
            O = (E @ V[:, g, :]) / L[:, None]
        out[lo:hi, h] = np.where((nv > 0)[:, None], O, 0.0)


def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
            cu_seqlens_q: np.ndarray, context_lens: np.ndarray,
            block_tables: np.ndarray, scale: float,
            rows: Optional[Sequence[int]] = None):
    """q: [total_q, Hq, D] fp64 packed by cu_seqlens_q; caches after the store.
    Returns out [total_q, Hq, D]; if ``rows`` is given, only those query rows
    are computed (others stay zero) -- used for sampled checks at full size."""
    total_q, Hq, D = q.shape
    out = np.zeros((total_q, Hq, D))
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(len(context_lens)):
        lo, hi = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n_k = int(context_lens[b])
        if wanted is not None and not any(lo <= r < hi for r in wanted):
            continue
        K = gather(k_cache, block_tables[b], n_k)
        V = gather(v_cache, block_tables[b], n_k)
        _prefill_sequence(q, K, V, lo, hi - lo, n_k, scale, out, wanted)
    return out


def prefill_contiguous(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens_q: np.ndarray,
                       cu_seqlens_k: np.ndarray, scale: float,
                       rows: Optional[Sequence[int]] = None):
    """Varlen causal prefill without a cache (source study section 2: with
    no prefix hit the attention layer attends this step's own k, v): keys of
    sequence b are rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k / v
    ([total_k, Hkv, D] fp64); bottom-right causal as in ``prefill``, so a
    query that sees no key (n_k < n_q) gets zeros."""
    total_q, Hq, D = q.shape
    out = np.zeros((total_q, Hq, D))
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(len(cu_seqlens_q) - 1):
        lo, hi = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        _prefill_sequence(q, k[k0:k1], v[k0:k1], lo, hi - lo, k1 - k0, scale, out, wanted)
    return out
