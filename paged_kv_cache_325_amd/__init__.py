"""Python binding of libpkv (paged KV-cache attention for gfx950).

Argument marshalling only: every function here takes torch tensors that live
on the GPU, checks their shapes, and passes raw pointers, sizes and the
current HIP stream to the C ABI declared in ``include/pkv.h``.  All work runs
in the library's HIP kernels; there is no CPU fallback.  If ``libpkv.so`` is
missing or a tensor is not on the GPU, the call raises.

Names follow the C ABI: ``pkv_kv_store``, ``pkv_paged_decode`` (and its two
halves ``pkv_paged_decode_partials`` / ``pkv_paged_decode_merge``),
``pkv_paged_decode_step`` (store fused into decode), ``pkv_paged_decode_step_noalloc``
(the same without a workspace), ``pkv_decode_prefix_plan`` /
``pkv_decode_prefix_plan_words`` (host planner of the shared-prefix decode),
``pkv_paged_decode_prefix`` and ``pkv_paged_decode_step_prefix`` (decode with
that plan), ``pkv_paged_decode_workspace_bytes``,
``pkv_paged_decode_split_tokens``, ``pkv_paged_prefill_workspace_bytes``,
``pkv_paged_prefill_varlen``, ``pkv_prefill_varlen`` (contiguous k/v, no cache),
``pkv_kv_block_bytes``, ``pkv_check_metadata``, ``pkv_last_error``.

Debug mode: with the environment variable ``PKV_CHECK_METADATA`` set to a
value other than ``0``, every call first copies its metadata (slots, block
tables, context lengths, query offsets) to the host and checks its ranges
with ``pkv_check_metadata`` (a synchronising copy: not for graph capture or
timing); out-of-range entries then raise instead of being undefined.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PKV_OK", "PKV_ERR_INVALID", "PKV_ERR_UNSUPPORTED", "PKV_ERR_WORKSPACE", "PKV_ERR_HIP",
    "PKV_FP32", "PKV_BF16", "PkvError", "lib_path", "load_library",
    "pkv_kv_store", "pkv_paged_decode", "pkv_paged_decode_partials", "pkv_paged_decode_merge",
    "pkv_paged_decode_step", "pkv_paged_decode_step_noalloc", "PKV_NOALLOC_SCRATCH_BYTES",
    "pkv_decode_prefix_plan_words", "pkv_decode_prefix_plan", "pkv_paged_decode_prefix",
    "pkv_paged_decode_step_prefix",
    "pkv_paged_decode_workspace_bytes",
    "pkv_paged_decode_split_tokens", "pkv_paged_prefill_varlen",
    "pkv_paged_prefill_workspace_bytes", "pkv_prefill_varlen", "pkv_kv_block_bytes",
    "pkv_check_metadata", "pkv_last_error",
]

PKV_OK, PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP = range(5)
PKV_FP32, PKV_BF16 = 0, 1
PKV_NOALLOC_SCRATCH_BYTES = 32 << 20  # include/pkv.h

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pkv status {status}: {message}")
        self.status = status


def lib_path() -> str:
    return os.path.join(_HERE, "libpkv.so")


def load_library() -> ctypes.CDLL:
    """Load libpkv.so once and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -m paged_kv_cache_325_amd.build)")
    lib = ctypes.CDLL(path)
    c_i32, c_i64, c_p, c_f = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.pkv_kv_store.restype = c_i32
    lib.pkv_kv_store.argtypes = [c_i32, c_p, c_i64, c_p, c_i64, c_p, c_p, c_p, c_i32, c_i32,
                                 c_i32, c_i32, c_i64, c_p]
    lib.pkv_paged_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pkv_paged_decode_workspace_bytes.argtypes = [c_i32] * 7
    lib.pkv_paged_decode_split_tokens.restype = c_i32
    lib.pkv_paged_decode_split_tokens.argtypes = [c_i32] * 7
    for fn in (lib.pkv_paged_decode, lib.pkv_paged_decode_partials):
        fn.restype = c_i32
        fn.argtypes = [c_i32, c_p, c_i64, c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i32,
                       c_i32, c_i32, c_i64, c_f, c_i32, c_p, c_p, ctypes.c_size_t, c_p]
    lib.pkv_paged_decode_step.restype = c_i32
    lib.pkv_paged_decode_step.argtypes = [c_i32, c_p, c_i64, c_p, c_i64, c_p, c_i64, c_p, c_p, c_p,
                                          c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                          c_i64, c_f, c_i32, c_p, c_p, ctypes.c_size_t, c_p]
    lib.pkv_paged_decode_step_noalloc.restype = c_i32
    lib.pkv_paged_decode_step_noalloc.argtypes = [c_i32, c_p, c_i64, c_p, c_i64, c_p, c_i64, c_p,
                                                  c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32,
                                                  c_i32, c_i32, c_i32, c_i64, c_f, c_i32, c_p,
                                                  c_p]
    lib.pkv_decode_prefix_plan_words.restype = c_i64
    lib.pkv_decode_prefix_plan_words.argtypes = [c_i32, c_i32, c_i32]
    lib.pkv_decode_prefix_plan.restype = c_i32
    lib.pkv_decode_prefix_plan.argtypes = [c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_p,
                                           c_i64, c_p, c_p]
    lib.pkv_paged_decode_prefix.restype = c_i32
    lib.pkv_paged_decode_prefix.argtypes = [c_i32, c_p, c_i64, c_p, c_p, c_p, c_i32, c_p, c_i32,
                                            c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, c_f, c_i32,
                                            c_p, c_i32, c_p, c_p, ctypes.c_size_t, c_p]
    lib.pkv_paged_decode_step_prefix.restype = c_i32
    lib.pkv_paged_decode_step_prefix.argtypes = [c_i32, c_p, c_i64, c_p, c_i64, c_p, c_i64, c_p,
                                                 c_p, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32,
                                                 c_i32, c_i32, c_i32, c_i64, c_f, c_i32, c_p,
                                                 c_i32, c_p, c_p, ctypes.c_size_t, c_p]
    lib.pkv_paged_decode_merge.restype = c_i32
    lib.pkv_paged_decode_merge.argtypes = [c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                           c_i32, c_p, c_p, ctypes.c_size_t, c_p]
    lib.pkv_paged_prefill_varlen.restype = c_i32
    lib.pkv_paged_prefill_varlen.argtypes = [c_i32, c_p, c_i64, c_p, c_p, c_p, c_i32, c_p, c_i32,
                                             c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                             c_i64, c_f, c_i32, c_p, c_p, ctypes.c_size_t, c_p]
    lib.pkv_prefill_varlen.restype = c_i32
    lib.pkv_prefill_varlen.argtypes = [c_i32, c_p, c_i64, c_p, c_i64, c_p, c_i64, c_p, c_p, c_i32,
                                       c_i32, c_i32, c_i32, c_i32, c_f, c_i32, c_p, c_p,
                                       ctypes.c_size_t, c_p]
    lib.pkv_paged_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.pkv_paged_prefill_workspace_bytes.argtypes = []
    lib.pkv_check_metadata.restype = c_i32
    lib.pkv_check_metadata.argtypes = [c_p, c_i32, c_p, c_i32, c_p, c_p, c_i32, c_i32, c_i32,
                                       c_i32, c_i32, c_i64]
    lib.pkv_kv_block_bytes.restype = c_i64
    lib.pkv_kv_block_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32]
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    _LIB = lib
    return lib


def pkv_last_error() -> str:
    return load_library().pkv_last_error().decode()


def _check(status: int) -> None:
    if status != PKV_OK:
        raise PkvError(status, pkv_last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _gpu(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor on the GPU")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _rows(t: torch.Tensor, name: str, heads: int, dim: int) -> int:
    """Token stride of a [tokens, heads, dim] tensor whose heads/dims are dense."""
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != dim:
        raise ValueError(f"{name} must be [tokens, {heads}, {dim}], got {tuple(t.shape)}")
    if t.stride(2) != 1 or t.stride(1) != dim:
        raise ValueError(f"{name} must have dense heads and dims (strides (*, {dim}, 1))")
    return t.stride(0)


def _cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor):
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must both be [num_blocks, num_kv_heads, block_size, head_dim]")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache dtypes differ")
    return tuple(int(x) for x in k_cache.shape)


def _int32(t: torch.Tensor, name: str) -> None:
    _gpu(t, name)
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor")


def pkv_kv_block_bytes(dtype: int, num_kv_heads: int, head_dim: int, block_size: int) -> int:
    return int(load_library().pkv_kv_block_bytes(dtype, num_kv_heads, head_dim, block_size))


def pkv_check_metadata(slot_mapping=None, block_tables=None, context_lens=None,
                       cu_seqlens_q=None, *, max_context_len: int = 0, max_seqlen_q: int = 0,
                       total_q: int = -1, block_size: int = 256, num_blocks: int = 0) -> None:
    """Range-check one step's metadata on the host (tensors on any device,
    or array-likes; copied as int32).  Raises PkvError(PKV_ERR_INVALID)
    naming the first bad entry; see pkv_check_metadata in include/pkv.h."""
    def host(a):
        if a is None:
            return None
        t = a.detach() if isinstance(a, torch.Tensor) else torch.as_tensor(a)
        return t.to("cpu", torch.int32).contiguous()
    sm, bt, cl, cu = host(slot_mapping), host(block_tables), host(context_lens), host(cu_seqlens_q)
    if cl is not None:
        batch = cl.numel()
    elif cu is not None:
        batch = max(cu.numel() - 1, 0)
    else:
        batch = 0 if bt is None else int(bt.shape[0])
    max_blocks = 0
    if bt is not None:
        if bt.dim() != 2 or bt.shape[0] != batch:
            raise ValueError("block_tables must be [batch, max_blocks]")
        max_blocks = int(bt.shape[1])
    if cu is not None and cu.numel() != batch + 1:
        raise ValueError("cu_seqlens_q must be [batch + 1]")
    _check(load_library().pkv_check_metadata(
        None if sm is None else sm.data_ptr(), 0 if sm is None else sm.numel(),
        None if bt is None else bt.data_ptr(), max_blocks,
        None if cl is None else cl.data_ptr(), None if cu is None else cu.data_ptr(), batch,
        int(max_context_len), int(max_seqlen_q), int(total_q), int(block_size), int(num_blocks)))


def _debug_check(**kw) -> None:
    """pkv_check_metadata(**kw) in debug mode (PKV_CHECK_METADATA set, not 0)."""
    if os.environ.get("PKV_CHECK_METADATA", "0") not in ("", "0"):
        pkv_check_metadata(**kw)


def pkv_kv_store(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 slot_mapping: torch.Tensor, stream=None) -> None:
    """Scatter k/v rows ([N, Hkv, D], token stride free) into the caches."""
    lib = load_library()
    for t, n in ((k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _gpu(t, n)
    _int32(slot_mapping, "slot_mapping")
    nblk, hkv, bs, d = _cache_dims(k_cache, v_cache)
    if k.dtype != k_cache.dtype or v.dtype != k_cache.dtype:
        raise ValueError("k, v and caches must share a dtype")
    ks = _rows(k, "k", hkv, d)
    vs = _rows(v, "v", hkv, d)
    n = k.shape[0]
    if v.shape[0] != n or slot_mapping.numel() != n:
        raise ValueError("k, v and slot_mapping disagree on the number of tokens")
    _debug_check(slot_mapping=slot_mapping, block_size=bs, num_blocks=nblk)
    _check(lib.pkv_kv_store(_dtype_code(k), _ptr(k), ks, _ptr(v), vs, _ptr(k_cache), _ptr(v_cache),
                            _ptr(slot_mapping), n, hkv, d, bs, nblk, _stream(stream)))


def pkv_paged_decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int,
                                     head_dim: int, max_context_len: int, block_size: int,
                                     num_splits: int = 0) -> int:
    return int(load_library().pkv_paged_decode_workspace_bytes(
        batch, num_q_heads, num_kv_heads, head_dim, max_context_len, block_size, num_splits))


def pkv_paged_decode_split_tokens(batch: int, num_q_heads: int, num_kv_heads: int,
                                  head_dim: int, max_context_len: int, block_size: int,
                                  num_splits: int = 0) -> int:
    return int(load_library().pkv_paged_decode_split_tokens(
        batch, num_q_heads, num_kv_heads, head_dim, max_context_len, block_size, num_splits))


def _decode_call(fn_name, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                 scale, out, workspace, num_splits, stream, plan=None):
    lib = load_library()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _gpu(t, n)
    _int32(block_tables, "block_tables")
    _int32(context_lens, "context_lens")
    nblk, hkv, bs, d = _cache_dims(k_cache, v_cache)
    if q.dtype != k_cache.dtype:
        raise ValueError("q and caches must share a dtype")
    if q.dim() != 3:
        raise ValueError("q must be [batch, num_q_heads, head_dim]")
    batch, hq = int(q.shape[0]), int(q.shape[1])
    qs = _rows(q, "q", hq, d)
    if block_tables.dim() != 2 or block_tables.shape[0] != batch or context_lens.numel() != batch:
        raise ValueError("block_tables must be [batch, max_blocks] and context_lens [batch]")
    max_blocks = int(block_tables.shape[1])
    if out is None:
        out = torch.empty((batch, hq, d), dtype=q.dtype, device=q.device)
    _gpu(out, "out")
    if out.shape != (batch, hq, d) or not out.is_contiguous() or out.dtype != q.dtype:
        raise ValueError("out must be a contiguous [batch, Hq, D] tensor of q's dtype")
    need = pkv_paged_decode_workspace_bytes(batch, hq, hkv, d, max_context_len, bs, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _debug_check(block_tables=block_tables, context_lens=context_lens,
                 max_context_len=max_context_len, block_size=bs, num_blocks=nblk)
    _check(getattr(lib, fn_name)(
        _dtype_code(q), _ptr(q), qs, _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), max_blocks,
        _ptr(context_lens), int(max_context_len), batch, hq, hkv, d, bs, nblk, float(scale),
        int(num_splits), *([] if plan is None else list(plan)), _ptr(out), _ptr(workspace),
        ws_bytes, _stream(stream)))
    return out, workspace


def _plan_args(prefix_plan: Optional[torch.Tensor], prefix_items: int):
    """Pointer and item count of a device plan (None: no plan)."""
    if prefix_plan is None:
        if prefix_items:
            raise ValueError("prefix_items > 0 needs a prefix_plan")
        return (None, 0)
    _int32(prefix_plan, "prefix_plan")
    return (_ptr(prefix_plan), int(prefix_items))


def pkv_decode_prefix_plan_words(batch: int, max_context_len: int, split_tokens: int) -> int:
    return int(load_library().pkv_decode_prefix_plan_words(batch, max_context_len, split_tokens))


def pkv_decode_prefix_plan(block_tables, context_lens, num_q_heads: int, num_kv_heads: int,
                           block_size: int, split_tokens: int):
    """Host planner of the shared-prefix decode (include/pkv.h): from the HOST
    block tables [batch, max_blocks] and context lengths [batch] (int32, torch
    CPU tensors or numpy arrays), returns (plan, items): the plan as an int32
    CPU tensor (copy it to the GPU for the decode) and its number of items."""
    lib = load_library()
    bt = torch.as_tensor(block_tables).to(torch.int32).contiguous()
    cl = torch.as_tensor(context_lens).to(torch.int32).contiguous()
    if bt.is_cuda or cl.is_cuda:
        raise ValueError("the planner reads host copies of the tables and context lengths")
    if bt.dim() != 2 or cl.dim() != 1 or bt.shape[0] != cl.shape[0]:
        raise ValueError("block_tables must be [batch, max_blocks] and context_lens [batch]")
    batch, max_blocks = int(bt.shape[0]), int(bt.shape[1])
    max_ctx = int(cl.max()) if batch else 0
    cap = pkv_decode_prefix_plan_words(batch, max(max_ctx, 0), split_tokens)
    if cap < 0:
        raise ValueError("bad batch or split_tokens")
    buf = torch.empty(cap, dtype=torch.int32)
    items, words = ctypes.c_int32(0), ctypes.c_int64(0)
    _check(lib.pkv_decode_prefix_plan(bt.data_ptr(), max_blocks, cl.data_ptr(), batch,
                                      num_q_heads, num_kv_heads, block_size, split_tokens,
                                      buf.data_ptr(), cap, ctypes.byref(items),
                                      ctypes.byref(words)))
    return buf[: words.value].clone(), int(items.value)


def pkv_paged_decode_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor,
                            max_context_len: int, scale: float,
                            prefix_plan: Optional[torch.Tensor], prefix_items: int,
                            out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, num_splits: int = 0,
                            stream=None) -> torch.Tensor:
    """pkv_paged_decode with a shared-prefix plan (a device int32 tensor from
    pkv_decode_prefix_plan for the same tables, lengths and split length)."""
    return _decode_call("pkv_paged_decode_prefix", q, k_cache, v_cache, block_tables,
                        context_lens, max_context_len, scale, out, workspace, num_splits, stream,
                        plan=_plan_args(prefix_plan, prefix_items))[0]


def pkv_paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     block_tables: torch.Tensor, context_lens: torch.Tensor,
                     max_context_len: int, scale: float, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, num_splits: int = 0,
                     stream=None) -> torch.Tensor:
    """Paged decode: q [batch, Hq, D] (token stride free) -> out [batch, Hq, D].

    ``max_context_len`` is a host integer >= every context length (it sets the
    split plan without a device-to-host read).  ``workspace`` is allocated
    with torch if not given."""
    return _decode_call("pkv_paged_decode", q, k_cache, v_cache, block_tables, context_lens,
                        max_context_len, scale, out, workspace, num_splits, stream)[0]


def _step_args(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens,
               out, max_context_len):
    """Checked pointers and sizes of a decode step (shared by both forms)."""
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _gpu(t, n)
    for t, n in ((slot_mapping, "slot_mapping"), (block_tables, "block_tables"),
                 (context_lens, "context_lens")):
        _int32(t, n)
    nblk, hkv, bs, d = _cache_dims(k_cache, v_cache)
    if q.dtype != k_cache.dtype or k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise ValueError("q, k_new, v_new and caches must share a dtype")
    if q.dim() != 3:
        raise ValueError("q must be [batch, num_q_heads, head_dim]")
    batch, hq = int(q.shape[0]), int(q.shape[1])
    qs = _rows(q, "q", hq, d)
    ks = _rows(k_new, "k_new", hkv, d)
    vs = _rows(v_new, "v_new", hkv, d)
    if (k_new.shape[0] != batch or v_new.shape[0] != batch or slot_mapping.numel() != batch
            or context_lens.numel() != batch or block_tables.dim() != 2
            or block_tables.shape[0] != batch):
        raise ValueError("q, k_new, v_new, slot_mapping, context_lens and block_tables must "
                         "agree on the batch")
    _gpu(out, "out")
    if out.shape != (batch, hq, d) or not out.is_contiguous() or out.dtype != q.dtype:
        raise ValueError("out must be a contiguous [batch, Hq, D] tensor of q's dtype")
    _debug_check(slot_mapping=slot_mapping, block_tables=block_tables, context_lens=context_lens,
                 max_context_len=max_context_len, block_size=bs, num_blocks=nblk)
    return (batch, hq, hkv, d, bs, nblk,
            [_dtype_code(q), _ptr(q), qs, _ptr(k_new), ks, _ptr(v_new), vs, _ptr(slot_mapping),
             _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), int(block_tables.shape[1]),
             _ptr(context_lens)])


def pkv_paged_decode_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                          slot_mapping: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_tables: torch.Tensor, context_lens: torch.Tensor,
                          max_context_len: int, scale: float, out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, num_splits: int = 0,
                          stream=None) -> torch.Tensor:
    """One decode step: store k_new/v_new ([batch, Hkv, D]) at slot_mapping
    and decode q ([batch, Hq, D]) over the cache, in one call (see
    pkv_paged_decode_step in include/pkv.h for the decode-step invariant)."""
    lib = load_library()
    if out is None:
        _gpu(q, "q")
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    batch, hq, hkv, d, bs, nblk, head = _step_args(q, k_new, v_new, slot_mapping, k_cache,
                                                   v_cache, block_tables, context_lens, out,
                                                   max_context_len)
    need = pkv_paged_decode_workspace_bytes(batch, hq, hkv, d, max_context_len, bs, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_decode_step(
        *head, int(max_context_len), batch, hq, hkv, d, bs, nblk, float(scale),
        int(num_splits), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def pkv_paged_decode_step_prefix(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                 slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                                 v_cache: torch.Tensor, block_tables: torch.Tensor,
                                 context_lens: torch.Tensor, max_context_len: int, scale: float,
                                 prefix_plan: Optional[torch.Tensor], prefix_items: int,
                                 out: Optional[torch.Tensor] = None,
                                 workspace: Optional[torch.Tensor] = None, num_splits: int = 0,
                                 stream=None) -> torch.Tensor:
    """pkv_paged_decode_step with a shared-prefix plan (see
    pkv_paged_decode_prefix)."""
    lib = load_library()
    if out is None:
        _gpu(q, "q")
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    batch, hq, hkv, d, bs, nblk, head = _step_args(q, k_new, v_new, slot_mapping, k_cache,
                                                   v_cache, block_tables, context_lens, out,
                                                   max_context_len)
    need = pkv_paged_decode_workspace_bytes(batch, hq, hkv, d, max_context_len, bs, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_decode_step_prefix(
        *head, int(max_context_len), batch, hq, hkv, d, bs, nblk, float(scale),
        int(num_splits), *_plan_args(prefix_plan, prefix_items), _ptr(out), _ptr(workspace),
        ws_bytes, _stream(stream)))
    return out


def pkv_paged_decode_step_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                  slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                                  v_cache: torch.Tensor, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, max_context_len: int, scale: float,
                                  out: torch.Tensor, num_splits: int = 0,
                                  stream=None) -> torch.Tensor:
    """pkv_paged_decode_step without a workspace, allocating nothing: the
    split-K partials go to the library's fixed per-GPU scratch of
    PKV_NOALLOC_SCRATCH_BYTES.  ``out`` must be given.  Calls that overlap on
    one GPU race on the scratch."""
    lib = load_library()
    batch, hq, hkv, d, bs, nblk, head = _step_args(q, k_new, v_new, slot_mapping, k_cache,
                                                   v_cache, block_tables, context_lens, out,
                                                   max_context_len)
    _check(lib.pkv_paged_decode_step_noalloc(
        *head, int(max_context_len), batch, hq, hkv, d, bs, nblk, float(scale),
        int(num_splits), _ptr(out), _stream(stream)))
    return out


def pkv_paged_decode_partials(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                              scale, out=None, workspace=None, num_splits=0, stream=None):
    """First half of pkv_paged_decode: returns (out, workspace); out holds the
    rows of single-split sequences, workspace the split-K partials."""
    return _decode_call("pkv_paged_decode_partials", q, k_cache, v_cache, block_tables,
                        context_lens, max_context_len, scale, out, workspace, num_splits, stream)


def pkv_paged_decode_merge(context_lens: torch.Tensor, max_context_len: int, num_q_heads: int,
                           num_kv_heads: int, block_size: int, out: torch.Tensor,
                           workspace: Optional[torch.Tensor], num_splits: int = 0,
                           stream=None) -> torch.Tensor:
    """Second half of pkv_paged_decode: merge the partials in ``workspace``
    into the rows of ``out`` [batch, Hq, D] whose sequences were split.

    ``max_context_len``, ``block_size`` and ``num_splits`` must be those of
    the partials call: together with the head counts they fix the split plan
    (a split never spans more than 64 cache blocks, so the plan depends on
    the block size)."""
    lib = load_library()
    _int32(context_lens, "context_lens")
    _gpu(out, "out")
    batch = int(context_lens.numel())
    if out.dim() != 3 or out.shape[0] != batch or out.shape[1] != num_q_heads or not out.is_contiguous():
        raise ValueError("out must be a contiguous [batch, num_q_heads, head_dim] tensor")
    d = int(out.shape[2])
    if workspace is not None:
        _gpu(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_decode_merge(_dtype_code(out), _ptr(context_lens), int(max_context_len),
                                      batch, int(num_q_heads), int(num_kv_heads), d,
                                      int(block_size), int(num_splits), _ptr(out),
                                      _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def pkv_paged_prefill_varlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             cu_seqlens_q: torch.Tensor, max_seqlen_q: int,
                             context_lens: torch.Tensor, max_context_len: int,
                             block_tables: torch.Tensor, scale: float,
                             out: Optional[torch.Tensor] = None, causal: int = 1,
                             workspace: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """Varlen causal prefill: q [total_q, Hq, D] bf16 -> out [total_q, Hq, D].

    ``workspace`` holds the kernel's work-queue counters: zero-filled before
    its first use, left zero by every call.  Without one, a zero-filled
    workspace kept per (device, stream) is used, so calls on one stream never
    share counters with calls running concurrently on another."""
    lib = load_library()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _gpu(t, n)
    _int32(cu_seqlens_q, "cu_seqlens_q")
    _int32(context_lens, "context_lens")
    _int32(block_tables, "block_tables")
    nblk, hkv, bs, d = _cache_dims(k_cache, v_cache)
    if q.dtype != k_cache.dtype:
        raise ValueError("q and caches must share a dtype")
    if q.dim() != 3:
        raise ValueError("q must be [total_q, num_q_heads, head_dim]")
    total, hq = int(q.shape[0]), int(q.shape[1])
    qs = _rows(q, "q", hq, d)
    batch = int(context_lens.numel())
    if cu_seqlens_q.numel() != batch + 1 or block_tables.dim() != 2 or block_tables.shape[0] != batch:
        raise ValueError("cu_seqlens_q must be [batch+1] and block_tables [batch, max_blocks]")
    if out is None:
        out = torch.empty((total, hq, d), dtype=q.dtype, device=q.device)
    _gpu(out, "out")
    if out.shape != (total, hq, d) or not out.is_contiguous() or out.dtype != q.dtype:
        raise ValueError("out must be a contiguous [total_q, Hq, D] tensor of q's dtype")
    st = _stream(stream)
    if workspace is None:
        workspace = _prefill_workspace(q.device, st)
    _gpu(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    _debug_check(block_tables=block_tables, context_lens=context_lens, cu_seqlens_q=cu_seqlens_q,
                 max_context_len=max_context_len, max_seqlen_q=max_seqlen_q, total_q=total,
                 block_size=bs, num_blocks=nblk)
    _check(lib.pkv_paged_prefill_varlen(_dtype_code(q), _ptr(q), qs, _ptr(k_cache), _ptr(v_cache),
                                        _ptr(cu_seqlens_q), int(max_seqlen_q), _ptr(context_lens),
                                        int(max_context_len), _ptr(block_tables),
                                        int(block_tables.shape[1]), batch, hq, hkv, d, bs, nblk,
                                        float(scale), int(causal), _ptr(out), _ptr(workspace),
                                        ws_bytes, st))
    return out


def pkv_prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
                       scale: float, out: Optional[torch.Tensor] = None, causal: int = 1,
                       workspace: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Varlen causal prefill over contiguous k/v (no cache): q [total_q, Hq, D],
    k/v [total_k, Hkv, D] (token strides free) -> out [total_q, Hq, D]."""
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _gpu(t, n)
    _int32(cu_seqlens_q, "cu_seqlens_q")
    _int32(cu_seqlens_k, "cu_seqlens_k")
    if q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("q, k and v must share a dtype")
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [total_q, Hq, D] and k, v [total_k, Hkv, D]")
    total, hq, d = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    hkv = int(k.shape[1])
    qs = _rows(q, "q", hq, d)
    ks = _rows(k, "k", hkv, d)
    vs = _rows(v, "v", hkv, d)
    batch = int(cu_seqlens_q.numel()) - 1
    if batch < 0 or cu_seqlens_k.numel() != batch + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [batch + 1]")
    if out is None:
        out = torch.empty((total, hq, d), dtype=q.dtype, device=q.device)
    _gpu(out, "out")
    if out.shape != (total, hq, d) or not out.is_contiguous() or out.dtype != q.dtype:
        raise ValueError("out must be a contiguous [total_q, Hq, D] tensor of q's dtype")
    st = _stream(stream)
    if workspace is None:
        workspace = _prefill_workspace(q.device, st)
    _gpu(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    # query offsets against q's rows, key offsets against k's rows
    _debug_check(cu_seqlens_q=cu_seqlens_q, max_seqlen_q=max_seqlen_q, total_q=total)
    _debug_check(cu_seqlens_q=cu_seqlens_k, max_seqlen_q=int(k.shape[0]), total_q=int(k.shape[0]))
    _check(lib.pkv_prefill_varlen(_dtype_code(q), _ptr(q), qs, _ptr(k), ks, _ptr(v), vs,
                                  _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(max_seqlen_q), batch,
                                  hq, hkv, d, float(scale), int(causal), _ptr(out),
                                  _ptr(workspace), ws_bytes, st))
    return out


_PREFILL_WS = {}


def pkv_paged_prefill_workspace_bytes() -> int:
    return int(load_library().pkv_paged_prefill_workspace_bytes())


def _prefill_workspace(device, stream_handle) -> torch.Tensor:
    key = (device.index, stream_handle)
    ws = _PREFILL_WS.get(key)
    if ws is None:
        n = (pkv_paged_prefill_workspace_bytes() + 3) // 4
        ws = torch.zeros(n, dtype=torch.int32, device=device)
        _PREFILL_WS[key] = ws
    return ws
