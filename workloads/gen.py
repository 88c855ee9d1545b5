"""Seeded generators for the five paged-attention workloads and for small
parity cases.

What is drawn, and in which order (the order fixes the values for a seed):

1. Structure, with ``numpy.random.default_rng(seed)``: sequence lengths (by the
   per-workload functions below), the indices of stores that are skipped
   (``slot = -1``), then one permutation of the physical block pool.
2. Values, with ``torch.Generator().manual_seed(seed)`` on the CPU: the fused
   ``qkv`` rows of this step's tokens, then, for every physical block in the
   order it was handed out, its K rows and then its V rows.  Values are N(0, 1)
   fp32, rounded to bf16 (round to nearest even) for bf16 workloads.

The physical pool is handed out like a block manager would (nano-vllm
architecture page, "Block Manager und KV-Cache-Verwaltung"): shared prefix
blocks of each sharing group first, then every sequence's private blocks in
sequence order.  A sequence's logical block ``i`` is ``block_tables[b][i]``;
unused table columns hold -1.  Only whole blocks are shared, and the block
that receives a store is always private.

Cache contents before the store:
  * cells inside a context that are not written this step: random values;
  * cells a store will write: ``SENTINEL_BITS`` (a NaN with a payload), so a
    missed store is visible;
  * every other cell: ``POISON_BITS`` (a quiet NaN), so a kernel that reads
    past a context, or multiplies a masked row by zero instead of leaving it
    out, produces NaN.

Nothing here performs the store or any attention arithmetic.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

BLOCK_SIZE = 256
HEAD_DIM = 128

POISON_BITS = {"bf16": 0x7FC0, "fp32": 0x7FC00000}
SENTINEL_BITS = {"bf16": 0xFFE5, "fp32": 0xFFE5A5A5}

_TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}
_INT_DTYPE = {"bf16": torch.int16, "fp32": torch.int32}
_NP_UINT = {"bf16": np.uint16, "fp32": np.uint32}


def _as_signed(bits: int, width: int) -> int:
    return bits - (1 << width) if bits >= (1 << (width - 1)) else bits


def bits_view(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU bf16/fp32 tensor as a uint16/uint32 array."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(f"unsupported dtype {t.dtype}")


@dataclasses.dataclass
class Spec:
    name: str
    mode: str  # "decode" or "prefill"
    dtype: str  # "fp32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    context_lens: List[int]  # keys per sequence, including this step's tokens
    new_tokens: List[int]  # tokens stored this step, at the end of each context
    seed: int
    skip: List[int] = dataclasses.field(default_factory=list)  # new-token indices with slot -1
    share_group: Optional[List[int]] = None  # sharing group per sequence (-1: none)
    shared_blocks: Optional[List[int]] = None  # leading blocks taken from the group
    pool_blocks: Optional[int] = None
    pool_factor: float = 1.25
    head_dim: int = HEAD_DIM
    block_size: int = BLOCK_SIZE
    scale: Optional[float] = None
    q_scale: float = 1.0  # >1 sharpens the softmax
    pad_columns: int = 0  # extra -1 columns in block_tables


@dataclasses.dataclass
class Workload:
    spec: Spec
    qkv: torch.Tensor  # [N, Hq + 2 Hkv, D], CPU
    k_cache: torch.Tensor  # [num_blocks, Hkv, B, D], CPU, before the store
    v_cache: torch.Tensor
    slot_mapping: np.ndarray  # int32 [N]
    block_tables: np.ndarray  # int32 [batch, max_blocks], -1 padded
    context_lens: np.ndarray  # int32 [batch]
    cu_seqlens_q: np.ndarray  # int32 [batch + 1]
    shared_physical: List[int]  # physical ids of shared blocks
    scale: float

    # -- convenient views -------------------------------------------------
    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.spec.dtype]

    @property
    def batch(self) -> int:
        return len(self.spec.context_lens)

    @property
    def num_q_heads(self) -> int:
        return self.spec.num_q_heads

    @property
    def num_kv_heads(self) -> int:
        return self.spec.num_kv_heads

    @property
    def head_dim(self) -> int:
        return self.spec.head_dim

    @property
    def block_size(self) -> int:
        return self.spec.block_size

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.qkv.shape[0])

    @property
    def q(self) -> torch.Tensor:
        return self.qkv[:, : self.num_q_heads]

    @property
    def k(self) -> torch.Tensor:
        h = self.num_q_heads
        return self.qkv[:, h : h + self.num_kv_heads]

    @property
    def v(self) -> torch.Tensor:
        h = self.num_q_heads + self.num_kv_heads
        return self.qkv[:, h : h + self.num_kv_heads]

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0

    @property
    def max_seqlen_q(self) -> int:
        if self.batch == 0:
            return 0
        return int(np.diff(self.cu_seqlens_q).max())

    # -- algorithmic sizes (what the method must move or compute) ---------
    def elem_bytes(self) -> int:
        return 2 if self.spec.dtype == "bf16" else 4

    def kv_token_bytes(self) -> int:
        """K+V bytes of one token across all kv heads (one layer)."""
        return 2 * self.num_kv_heads * self.head_dim * self.elem_bytes()

    def logical_kv_bytes(self) -> int:
        return int(self.context_lens.astype(np.int64).sum()) * self.kv_token_bytes()

    def unique_kv_bytes(self) -> int:
        """K+V bytes of distinct (physical block, row) cells read by attention."""
        seen = {}
        B = self.block_size
        for b in range(self.batch):
            n = int(self.context_lens[b])
            for i in range((n + B - 1) // B):
                p = int(self.block_tables[b, i])
                rows = min(B, n - i * B)
                seen[p] = max(seen.get(p, 0), rows)
        return sum(seen.values()) * self.kv_token_bytes()

    def qo_bytes(self) -> int:
        """Bytes of q read plus attention output written."""
        return 2 * self.num_tokens * self.num_q_heads * self.head_dim * self.elem_bytes()

    def store_bytes(self) -> int:
        """Bytes the slot scatter reads plus writes (skipped tokens move nothing)."""
        stored = int((self.slot_mapping >= 0).sum())
        return 2 * stored * self.kv_token_bytes()

    def prefill_flops(self) -> int:
        """4·D flops per unmasked (query, key) pair per query head."""
        total = 0
        for b in range(self.batch):
            nq = int(self.cu_seqlens_q[b + 1] - self.cu_seqlens_q[b])
            nk = int(self.context_lens[b])
            off = nk - nq
            # query i sees keys 0..off+i
            total += nq * (off + 1) + nq * (nq - 1) // 2
        return 4 * self.head_dim * self.num_q_heads * total


def _fill_bits(shape, bits: int, dtype: str) -> torch.Tensor:
    width = 16 if dtype == "bf16" else 32
    return torch.full(shape, _as_signed(bits, width), dtype=_INT_DTYPE[dtype])


def build(spec: Spec, rng: Optional[np.random.Generator] = None) -> Workload:
    """Draw one workload.  ``rng`` continues the structure stream of a caller
    that already drew lengths from it; otherwise one is made from the seed."""
    if rng is None:
        rng = np.random.default_rng(spec.seed)
    B, D = spec.block_size, spec.head_dim
    Hq, Hkv = spec.num_q_heads, spec.num_kv_heads
    batch = len(spec.context_lens)
    ctx = [int(c) for c in spec.context_lens]
    new = [int(n) for n in spec.new_tokens]
    assert len(new) == batch
    groups = spec.share_group or [-1] * batch
    shared = spec.shared_blocks or [0] * batch
    nblk = [(c + B - 1) // B for c in ctx]
    for b in range(batch):
        assert 0 <= new[b] <= ctx[b], "new tokens must lie inside the context"
        assert shared[b] * B <= ctx[b] - new[b], "stored rows may not fall in shared blocks"
        assert shared[b] <= nblk[b]

    group_ids = sorted({g for g in groups if g >= 0})
    group_need = {g: max(shared[b] for b in range(batch) if groups[b] == g) for g in group_ids}
    needed = sum(group_need.values()) + sum(nblk[b] - (shared[b] if groups[b] >= 0 else 0) for b in range(batch))
    pool = spec.pool_blocks if spec.pool_blocks is not None else int(math.ceil(spec.pool_factor * needed))
    assert pool >= needed
    perm = rng.permutation(pool).astype(np.int64) if pool else np.zeros(0, np.int64)

    cursor = 0
    handout: List[int] = []
    group_blocks = {}
    for g in group_ids:
        group_blocks[g] = [int(x) for x in perm[cursor : cursor + group_need[g]]]
        handout += group_blocks[g]
        cursor += group_need[g]
    max_blocks = (max(nblk) if batch else 0) + spec.pad_columns
    block_tables = np.full((batch, max(max_blocks, 1)), -1, dtype=np.int32)
    for b in range(batch):
        row = []
        if groups[b] >= 0:
            row += group_blocks[groups[b]][: shared[b]]
        priv = nblk[b] - len(row)
        mine = [int(x) for x in perm[cursor : cursor + priv]]
        cursor += priv
        handout += mine
        row += mine
        block_tables[b, : len(row)] = row
    shared_physical = [p for g in group_ids for p in group_blocks[g]]

    # rows of each physical block that hold context data
    valid = {}
    for b in range(batch):
        for i in range(nblk[b]):
            p = int(block_tables[b, i])
            valid[p] = max(valid.get(p, 0), min(B, ctx[b] - i * B))

    # slots of this step's tokens.  A decode step has one row per sequence;
    # a decode row with new_tokens == 0 is a padding row (slot -1).
    decode = spec.mode == "decode"
    if decode:
        assert all(n in (0, 1) for n in new)
    rows_per_seq = [1] * batch if decode else new
    n_tok = sum(rows_per_seq)
    slot_mapping = np.zeros(n_tok, dtype=np.int32)
    skip = set(int(s) for s in spec.skip)
    t = 0
    targets = []
    for b in range(batch):
        if decode and new[b] == 0:
            slot_mapping[t] = -1
            t += 1
            continue
        for pos in range(ctx[b] - new[b], ctx[b]):
            if t in skip:
                slot_mapping[t] = -1
            else:
                p = int(block_tables[b, pos // B])
                slot_mapping[t] = p * B + pos % B
                targets.append((p, pos % B))
            t += 1

    # values
    gen = torch.Generator().manual_seed(spec.seed)
    tdt = _TORCH_DTYPE[spec.dtype]
    qkv32 = torch.randn((n_tok, Hq + 2 * Hkv, D), generator=gen, dtype=torch.float32)
    if spec.q_scale != 1.0:
        qkv32[:, :Hq] *= spec.q_scale
    qkv = qkv32.to(tdt)

    kc = _fill_bits((pool, Hkv, B, D), POISON_BITS[spec.dtype], spec.dtype)
    vc = _fill_bits((pool, Hkv, B, D), POISON_BITS[spec.dtype], spec.dtype)
    idt = _INT_DTYPE[spec.dtype]
    for p in handout:
        rows = valid.get(p, 0)
        if rows <= 0:
            continue
        kv = torch.randn((2, Hkv, rows, D), generator=gen, dtype=torch.float32).to(tdt)
        kc[p, :, :rows] = kv[0].view(idt)
        vc[p, :, :rows] = kv[1].view(idt)
    sent = _as_signed(SENTINEL_BITS[spec.dtype], 16 if spec.dtype == "bf16" else 32)
    for p, o in targets:
        kc[p, :, o] = sent
        vc[p, :, o] = sent

    cu = np.zeros(batch + 1, dtype=np.int32)
    cu[1:] = np.cumsum(rows_per_seq)
    scale = spec.scale if spec.scale is not None else 1.0 / math.sqrt(D)
    return Workload(
        spec=spec,
        qkv=qkv,
        k_cache=kc.view(tdt),
        v_cache=vc.view(tdt),
        slot_mapping=slot_mapping,
        block_tables=block_tables,
        context_lens=np.asarray(ctx, dtype=np.int32),
        cu_seqlens_q=cu,
        shared_physical=shared_physical,
        scale=float(scale),
    )


# ---------------------------------------------------------------------------
# The five workloads (sizes, head counts and distributions as specified for
# this hot path; seeds 325001..325005).
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "decode-fp32-4seq",
    2: "decode-bf16-b64-ctx512-4096-h16-8",
    3: "prefill-bf16-8seq-L1024-4096-prefix512-h32-8",
    4: "decode-bf16-b256-ctx1024-8192-h32-8",
    5: "decode-bf16-b16-lognormal8192-shared4096-h32-8",
}


def config_specs(index: int):
    """(Spec, rng) for workload ``index`` in 1..5; the rng has already drawn
    the lengths and skip indices and continues with the block permutation."""
    seed = 325_000 + index
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[index]
    if index == 1:
        ctx = [17, 256, 300, 511]
        spec = Spec(name, "decode", "fp32", 16, 8, ctx, [1] * 4, seed, pool_blocks=16)
    elif index == 2:
        ctx = rng.integers(512, 4096, size=64, endpoint=True).tolist()
        skip = sorted(rng.choice(64, size=round(0.05 * 64), replace=False).tolist())
        spec = Spec(name, "decode", "bf16", 16, 8, ctx, [1] * 64, seed, skip=skip)
    elif index == 3:
        L = rng.integers(1024, 4096, size=8, endpoint=True).tolist()
        spec = Spec(
            name, "prefill", "bf16", 32, 8, L, [x - 512 for x in L], seed,
            share_group=[0] * 8, shared_blocks=[2] * 8,
        )
    elif index == 4:
        ctx = rng.integers(1024, 8192, size=256, endpoint=True).tolist()
        spec = Spec(name, "decode", "bf16", 32, 8, ctx, [1] * 256, seed)
    elif index == 5:
        raw = rng.lognormal(mean=math.log(8192), sigma=0.8, size=16)
        ctx = np.clip(np.round(raw), 256, 32768).astype(int).tolist()
        groups = [b // 4 for b in range(16)]
        shared = [min(16, (c - 1) // BLOCK_SIZE) for c in ctx]
        spec = Spec(
            name, "decode", "bf16", 32, 8, ctx, [1] * 16, seed,
            share_group=groups, shared_blocks=shared,
        )
    else:
        raise ValueError(index)
    return spec, rng


def config(index: int) -> Workload:
    spec, rng = config_specs(index)
    return build(spec, rng)


def small_specs():
    """Parity cases the oracle finishes in seconds: several 64-token chunks,
    several blocks, ragged tails, GQA 1/2/3/4/5/6/8/12, fp32 and bf16, contexts of 1,
    an empty context, prefill sequences without query rows, shared prefixes,
    skipped stores and extra padding."""
    out = []
    out.append(Spec("dec-bf16-g2-ragged", "decode", "bf16", 4, 2,
                    [1, 2, 63, 64, 65, 255, 256, 257, 511, 700, 1025, 2049], [1] * 12, 9001,
                    skip=[3], pad_columns=2))
    out.append(Spec("dec-bf16-g4-long", "decode", "bf16", 8, 2,
                    [3000, 1, 4097, 129, 5000, 256], [1] * 6, 9002))
    out.append(Spec("dec-fp32-g2", "decode", "fp32", 4, 2, [5, 300, 777, 1], [1] * 4, 9003))
    out.append(Spec("dec-bf16-g1", "decode", "bf16", 2, 2, [100, 1500], [1] * 2, 9004))
    out.append(Spec("dec-bf16-g8", "decode", "bf16", 8, 1, [999, 3], [1] * 2, 9005))
    out.append(Spec("dec-bf16-shared", "decode", "bf16", 8, 2, [1300, 700, 1025, 257], [1] * 4, 9006,
                    share_group=[0, 0, 1, 1], shared_blocks=[4, 2, 4, 1]))
    out.append(Spec("dec-bf16-peaked", "decode", "bf16", 8, 2, [2000, 517, 64], [1] * 3, 9007, q_scale=6.0))
    out.append(Spec("dec-bf16-empty-ctx", "decode", "bf16", 4, 2, [0, 33, 0], [0, 1, 0], 9008))
    # GQA groups that are not 1, 2, 4 or 8: a masked head in the workgroup
    # (3 of 4, 5 of 8), a partial second chunk (12 = 8 + 4), fp32 with 6 of 8
    out.append(Spec("dec-bf16-g3", "decode", "bf16", 6, 2, [1000, 65, 1], [1] * 3, 9009))
    out.append(Spec("dec-bf16-g5", "decode", "bf16", 10, 2, [2100, 300], [1] * 2, 9010))
    out.append(Spec("dec-bf16-g12", "decode", "bf16", 12, 1, [700, 1500], [1] * 2, 9011))
    out.append(Spec("dec-fp32-g6", "decode", "fp32", 6, 1, [400, 33], [1] * 2, 9012))
    out.append(Spec("pre-bf16-g4", "prefill", "bf16", 8, 2, [300, 512 + 37, 256 + 1, 1024 + 700],
                    [300, 37, 1, 700], 9101, share_group=[-1, 0, 0, 0], shared_blocks=[0, 2, 1, 4]))
    out.append(Spec("pre-bf16-g2", "prefill", "bf16", 4, 2, [63, 64, 65, 129, 600],
                    [63, 64, 65, 129, 88], 9102))
    out.append(Spec("pre-bf16-g8", "prefill", "bf16", 8, 1, [200, 777], [200, 500], 9103))
    out.append(Spec("pre-bf16-peaked", "prefill", "bf16", 8, 2, [900, 300], [400, 300], 9104, q_scale=6.0))
    # odd and non-multiple-of-4 groups: 1 head x 256 positions per work
    # item (3, 5), 2 heads x 128 positions (6)
    out.append(Spec("pre-bf16-g3", "prefill", "bf16", 6, 2, [300, 700], [300, 450], 9106))
    out.append(Spec("pre-bf16-g5", "prefill", "bf16", 5, 1, [520, 129], [400, 129], 9107))
    out.append(Spec("pre-bf16-g6", "prefill", "bf16", 12, 2, [333, 640], [333, 200], 9108))
    # sequences with cached context but no query rows this step, first and
    # in the middle, beside a single-row and a short fresh prompt
    out.append(Spec("pre-bf16-zero-rows", "prefill", "bf16", 8, 2, [300, 5, 700, 256],
                    [0, 5, 0, 1], 9105))
    return out
