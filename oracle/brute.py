"""Pure-Python loop versions of paged decode and prefill for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Written independently of ``oracle.ref`` (no shared
helpers) so that it can pin it: every key is fetched cell by cell through the
block table with the page/offset translation of the vLLM essay (lshu.cn,
section 3.2), every dot product and exponential is a scalar loop.

Inputs are nested Python lists (or anything indexable) of floats:
q[b][h][d], cache[p][g][o][d], block_tables[b][i], context_lens[b].
"""

import math


def _key(cache, table, j, g, B):
    page = table[j // B]
    return cache[page][g][j % B]


def scores(qv, cache_k, table, nkeys, g, B, scale):
    """scale * (q . k_j) for keys j = 0 .. nkeys-1 of one sequence, each key
    fetched cell by cell through its page and offset."""
    out = []
    for j in range(nkeys):
        kr = _key(cache_k, table, j, g, B)
        s = 0.0
        for d in range(len(qv)):
            s += qv[d] * kr[d]
        out.append(s * scale)
    return out


def value_row(cache_v, table, j, g, B):
    """V row of logical key j of one sequence (page and offset, as _key)."""
    return _key(cache_v, table, j, g, B)


def _attend_one(qv, cache_k, cache_v, table, nkeys, g, B, scale):
    D = len(qv)
    if nkeys <= 0:
        return [0.0] * D
    scores_ = scores(qv, cache_k, table, nkeys, g, B, scale)
    top = max(scores_)
    ex = [math.exp(s - top) for s in scores_]
    tot = math.fsum(ex)
    out = [0.0] * D
    for j in range(nkeys):
        vr = _key(cache_v, table, j, g, B)
        w = ex[j] / tot
        for d in range(D):
            out[d] += w * vr[d]
    return out


def decode(q, cache_k, cache_v, block_tables, context_lens, scale, num_kv_heads, block_size):
    out = []
    for b in range(len(context_lens)):
        hq = len(q[b])
        group = hq // num_kv_heads
        row = []
        for h in range(hq):
            row.append(_attend_one(q[b][h], cache_k, cache_v, block_tables[b],
                                   context_lens[b], h // group, block_size, scale))
        out.append(row)
    return out


def prefill(q, cache_k, cache_v, cu_seqlens_q, context_lens, block_tables, scale,
            num_kv_heads, block_size):
    out = [None] * len(q)
    for b in range(len(context_lens)):
        start, stop = cu_seqlens_q[b], cu_seqlens_q[b + 1]
        n_q, n_k = stop - start, context_lens[b]
        for i in range(n_q):
            pos = n_k - n_q + i  # position of this query in its sequence
            hq = len(q[start + i])
            group = hq // num_kv_heads
            out[start + i] = [
                _attend_one(q[start + i][h], cache_k, cache_v, block_tables[b],
                            pos + 1, h // group, block_size, scale)
                for h in range(hq)
            ]
    return out


def prefill_contiguous(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, num_kv_heads):
    """Keys of sequence b are rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of
    k[t][g][d] / v[t][g][d]; query i of n_q sees keys 0 .. n_k - n_q + i."""
    out = [None] * len(q)
    for b in range(len(cu_seqlens_q) - 1):
        qs, qe = cu_seqlens_q[b], cu_seqlens_q[b + 1]
        ks, ke = cu_seqlens_k[b], cu_seqlens_k[b + 1]
        n_q, n_k = qe - qs, ke - ks
        for i in range(n_q):
            row = []
            for h in range(len(q[qs + i])):
                g = h // (len(q[qs + i]) // num_kv_heads)
                qv = q[qs + i][h]
                D = len(qv)
                nkeys = min(n_k, n_k - n_q + i + 1)
                if nkeys <= 0:
                    row.append([0.0] * D)
                    continue
                scores = []
                for j in range(nkeys):
                    acc = 0.0
                    for d in range(D):
                        acc += qv[d] * k[ks + j][g][d]
                    scores.append(acc * scale)
                top = max(scores)
                ex = [math.exp(x - top) for x in scores]
                tot = math.fsum(ex)
                o = [0.0] * D
                for j in range(nkeys):
                    for d in range(D):
                        o[d] += ex[j] / tot * v[ks + j][g][d]
                row.append(o)
            out[qs + i] = row
    return out
