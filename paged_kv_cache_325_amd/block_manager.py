"""Python binding of the host block manager in libpkv (``include/pkv_block_manager.h``).

Argument marshalling only: each method of :class:`BlockManager` calls the C
function of the same name (``allocate`` -> ``pkv_bm_allocate``, ...) on the
library's handle and converts host arrays with numpy.  All bookkeeping runs in
the library's C++ code; nothing here touches the GPU.
"""

from __future__ import annotations

import ctypes

import numpy as np

from . import PKV_OK, PkvError, load_library, pkv_last_error

__all__ = ["BlockManager", "pkv_block_hash"]

_c_i32, _c_i64, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
_P_I32 = ctypes.POINTER(ctypes.c_int32)
_P_I64 = ctypes.POINTER(ctypes.c_int64)
_declared = False


def _lib():
    global _declared
    lib = load_library()
    if _declared:
        return lib
    sigs = {
        "pkv_block_hash": (_c_i64, [_c_p, _c_i32, _c_i64]),
        "pkv_bm_create": (_c_i32, [_c_i32, _c_i32, ctypes.POINTER(_c_p)]),
        "pkv_bm_destroy": (None, [_c_p]),
        "pkv_bm_add_sequence": (_c_i32, [_c_p, _c_i64, _c_p, _c_i32]),
        "pkv_bm_append_token": (_c_i32, [_c_p, _c_i64, _c_i32]),
        "pkv_bm_remove_sequence": (_c_i32, [_c_p, _c_i64]),
        "pkv_bm_can_allocate": (_c_i32, [_c_p, _c_i64, _P_I32]),
        "pkv_bm_allocate": (_c_i32, [_c_p, _c_i64]),
        "pkv_bm_deallocate": (_c_i32, [_c_p, _c_i64]),
        "pkv_bm_can_append": (_c_i32, [_c_p, _c_i64, _P_I32]),
        "pkv_bm_may_append": (_c_i32, [_c_p, _c_i64]),
        "pkv_bm_num_free_blocks": (_c_i32, [_c_p]),
        "pkv_bm_sequence": (_c_i32, [_c_p, _c_i64, _P_I32, _P_I32, _P_I32]),
        "pkv_bm_block_table": (_c_i32, [_c_p, _c_i64, _c_p, _c_i32]),
        "pkv_bm_block": (_c_i32, [_c_p, _c_i32, _P_I32, _P_I64, _P_I32]),
        "pkv_bm_free_blocks": (_c_i32, [_c_p, _c_p, _c_i32]),
        "pkv_bm_prefill_sizes": (_c_i32, [_c_p, _c_p, _c_i32, _P_I32, _P_I32]),
        "pkv_bm_build_prefill": (_c_i32, [_c_p, _c_p, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_i32,
                                          _c_p, _c_p, _c_p, _P_I32, _P_I32]),
        "pkv_bm_build_decode": (_c_i32, [_c_p, _c_p, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p,
                                         _c_p, _P_I32]),
        "pkv_bm_append_tokens": (_c_i32, [_c_p, _c_p, _c_i32, _c_p]),
        "pkv_bm_decode_step": (_c_i32, [_c_p, _c_p, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p,
                                        _c_p, _P_I32]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _declared = True
    return lib


def _check(status: int) -> None:
    if status != PKV_OK:
        raise PkvError(status, pkv_last_error())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data if a.size else None


def pkv_block_hash(token_ids, prefix: int = -1) -> int:
    """The library's chained block hash of token_ids on ``prefix``."""
    t = _i32(token_ids)
    return int(_lib().pkv_block_hash(_ptr(t), t.size, prefix))


class BlockManager:
    """Handle on a C block manager (pkv_bm_create / pkv_bm_destroy)."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = _lib()
        h = _c_p()
        _check(self._lib.pkv_bm_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    # sequences
    def add_sequence(self, seq_id: int, token_ids) -> None:
        t = _i32(token_ids)
        _check(self._lib.pkv_bm_add_sequence(self._h, seq_id, _ptr(t), t.size))

    def append_token(self, seq_id: int, token_id: int) -> None:
        _check(self._lib.pkv_bm_append_token(self._h, seq_id, int(token_id)))

    def remove_sequence(self, seq_id: int) -> None:
        _check(self._lib.pkv_bm_remove_sequence(self._h, seq_id))

    # block manager operations
    def can_allocate(self, seq_id: int) -> bool:
        out = ctypes.c_int32()
        _check(self._lib.pkv_bm_can_allocate(self._h, seq_id, ctypes.byref(out)))
        return bool(out.value)

    def allocate(self, seq_id: int) -> None:
        _check(self._lib.pkv_bm_allocate(self._h, seq_id))

    def deallocate(self, seq_id: int) -> None:
        _check(self._lib.pkv_bm_deallocate(self._h, seq_id))

    def can_append(self, seq_id: int) -> bool:
        out = ctypes.c_int32()
        _check(self._lib.pkv_bm_can_append(self._h, seq_id, ctypes.byref(out)))
        return bool(out.value)

    def may_append(self, seq_id: int) -> None:
        _check(self._lib.pkv_bm_may_append(self._h, seq_id))

    # queries
    def num_free_blocks(self) -> int:
        return int(self._lib.pkv_bm_num_free_blocks(self._h))

    def sequence(self, seq_id: int):
        """(num_tokens, num_cached_tokens, num_table_blocks)."""
        n, c, t = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pkv_bm_sequence(self._h, seq_id, ctypes.byref(n), ctypes.byref(c),
                                         ctypes.byref(t)))
        return n.value, c.value, t.value

    def block_table(self, seq_id: int) -> list:
        n = self.sequence(seq_id)[2]
        out = np.empty(n, np.int32)
        _check(self._lib.pkv_bm_block_table(self._h, seq_id, _ptr(out), n))
        return out.tolist()

    def block(self, block_id: int):
        """(ref_count, hash, num_tokens) of one block."""
        r, h, n = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
        _check(self._lib.pkv_bm_block(self._h, block_id, ctypes.byref(r), ctypes.byref(h),
                                      ctypes.byref(n)))
        return r.value, h.value, n.value

    def free_blocks(self) -> list:
        n = self.num_free_blocks()
        out = np.empty(n, np.int32)
        _check(self._lib.pkv_bm_free_blocks(self._h, _ptr(out), n))
        return out.tolist()

    # step metadata
    def build_prefill(self, seq_ids, width: int | None = None) -> dict:
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        ntok, mt = ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pkv_bm_prefill_sizes(self._h, _ptr(ids), ids.size, ctypes.byref(ntok),
                                              ctypes.byref(mt)))
        width = mt.value if width is None else width
        n = ntok.value
        input_ids, positions, slots = (np.empty(n, np.int32) for _ in range(3))
        cu_q, cu_k = np.empty(ids.size + 1, np.int32), np.empty(ids.size + 1, np.int32)
        tables = np.empty((ids.size, width), np.int32)
        mq, mk = ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pkv_bm_build_prefill(
            self._h, _ptr(ids), ids.size, width, _ptr(input_ids), _ptr(positions), _ptr(slots), n,
            _ptr(cu_q), _ptr(cu_k), _ptr(tables), ctypes.byref(mq), ctypes.byref(mk)))
        return {"input_ids": input_ids, "positions": positions, "slot_mapping": slots,
                "cu_seqlens_q": cu_q, "cu_seqlens_k": cu_k, "max_seqlen_q": mq.value,
                "max_seqlen_k": mk.value, "block_tables": tables}

    def build_decode(self, seq_ids, width: int | None = None) -> dict:
        return self._decode(self._lib.pkv_bm_build_decode, seq_ids, width)

    # batch forms of one engine step
    def append_tokens(self, seq_ids, token_ids) -> None:
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        t = _i32(token_ids)
        if t.size != ids.size:
            raise ValueError("one token per sequence")
        _check(self._lib.pkv_bm_append_tokens(self._h, _ptr(ids), ids.size, _ptr(t)))

    def decode_step(self, seq_ids, width: int) -> dict:
        """may_append for each sequence, then build_decode (pkv_bm_decode_step)."""
        return self._decode(self._lib.pkv_bm_decode_step, seq_ids, width)

    def _decode(self, fn, seq_ids, width):
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        if width is None:
            width = max((self.sequence(int(i))[2] for i in ids), default=0)
        n = ids.size
        input_ids, positions, slots, ctx = (np.empty(n, np.int32) for _ in range(4))
        tables = np.empty((n, width), np.int32)
        mk = ctypes.c_int32()
        _check(fn(self._h, _ptr(ids), n, width, _ptr(input_ids), _ptr(positions), _ptr(slots),
                  _ptr(ctx), _ptr(tables), ctypes.byref(mk)))
        return {"input_ids": input_ids, "positions": positions, "slot_mapping": slots,
                "context_lens": ctx, "max_context_len": mk.value, "block_tables": tables}
