"""Python binding of the host block allocator of libpkv (``include/pkv_blocks.h``).

Argument marshalling only: the pool, the per-type managers and the two-phase
``allocate_slots`` are the C++ ones behind the C ABI.  Tables come back as numpy
int32 arrays, ready to be copied to the device for the attention entry points.
"""
from __future__ import annotations

import ctypes
from typing import Iterable, Sequence

import numpy as np

from . import PkvError, load

ATTN_FULL, ATTN_SLIDING = 0, 1

# Every symbol include/pkv_blocks.h declares.
EXPORTS = ("pkv_pool_create", "pkv_pool_destroy", "pkv_pool_num_free", "pkv_pool_get_new_blocks",
           "pkv_pool_free_blocks", "pkv_kvm_create", "pkv_kvm_destroy", "pkv_kvm_allocate_slots",
           "pkv_kvm_free", "pkv_kvm_get_block_ids", "pkv_kvm_num_free_blocks", "pkv_kvm_format_usage",
           "pkv_kvm_prepare_block_table", "pkv_block_num_fixed", "pkv_block_num_full", "pkv_block_num_budget")


class AttnGroup(ctypes.Structure):
    _fields_ = [("attn_type", ctypes.c_int32), ("num_blocks", ctypes.c_int32), ("sliding_window", ctypes.c_int32)]


_typed = False


def _lib():
    global _typed
    lib = load()
    if not _typed:
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        pi32, pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
        sig = {
            "pkv_pool_create": [i32, ctypes.POINTER(P)],
            "pkv_pool_num_free": [P, pi32],
            "pkv_pool_get_new_blocks": [P, i32, P],
            "pkv_pool_free_blocks": [P, P, i32],
            "pkv_kvm_create": [ctypes.POINTER(AttnGroup), i32, i32, i32, ctypes.POINTER(P)],
            "pkv_kvm_allocate_slots": [P, i64, i32, i32, i32, pi32],
            "pkv_kvm_free": [P, i64],
            "pkv_kvm_get_block_ids": [P, i64, i32, P, i32, pi32],
            "pkv_kvm_num_free_blocks": [P, i32, pi32],
            "pkv_kvm_format_usage": [P, ctypes.c_char_p, sz],
            "pkv_kvm_prepare_block_table": [P, i32, P, i32, i32, P],
            "pkv_block_num_fixed": [i32, i32, i32, i32, pi64],
            "pkv_block_num_full": [i32, i32, i32, pi64],
            "pkv_block_num_budget": [i64, i64, i64, i32, pi64],
        }
        for name, args in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        lib.pkv_pool_destroy.argtypes = [P]
        lib.pkv_pool_destroy.restype = None
        lib.pkv_kvm_destroy.argtypes = [P]
        lib.pkv_kvm_destroy.restype = None
        _typed = True
    return lib


def _check(status: int):
    if status != 0:
        raise PkvError(status, _lib().pkv_last_error().decode())


def _ids(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class BlockPool:
    """Block ids 0..num_blocks-1; 0 is the null block; FIFO issue, tail return."""

    def __init__(self, num_blocks: int):
        h = ctypes.c_void_p()
        _check(_lib().pkv_pool_create(num_blocks, ctypes.byref(h)))
        self._h = h

    def __del__(self):
        if getattr(self, "_h", None):
            _lib().pkv_pool_destroy(self._h)
            self._h = None

    def num_free(self) -> int:
        n = ctypes.c_int32()
        _check(_lib().pkv_pool_num_free(self._h, ctypes.byref(n)))
        return n.value

    def get_new_blocks(self, n: int) -> list:
        out = np.zeros(max(n, 1), dtype=np.int32)
        _check(_lib().pkv_pool_get_new_blocks(self._h, n, out.ctypes.data))
        return out[:n].tolist()

    def free_blocks(self, ids: Iterable[int]) -> None:
        a = _ids(list(ids))
        _check(_lib().pkv_pool_free_blocks(self._h, a.ctypes.data if a.size else None, a.size))


class KVCacheManager:
    """Request-level manager over one pool per attention group.

    groups: (attn_type, num_blocks, sliding_window) per group (ATTN_FULL / ATTN_SLIDING)."""

    def __init__(self, groups: Sequence[tuple], block_size: int, max_model_len: int):
        arr = (AttnGroup * len(groups))(*[AttnGroup(int(t), int(n), int(w)) for t, n, w in groups])
        h = ctypes.c_void_p()
        _check(_lib().pkv_kvm_create(arr, len(groups), block_size, max_model_len, ctypes.byref(h)))
        self._h = h
        self.num_groups = len(groups)
        self.block_size = block_size
        self.max_model_len = max_model_len

    def __del__(self):
        if getattr(self, "_h", None):
            _lib().pkv_kvm_destroy(self._h)
            self._h = None

    def allocate_slots(self, request_id: int, computed_tokens: int, num_new_tokens: int,
                       lookahead_tokens: int = 0) -> bool:
        ok = ctypes.c_int32()
        _check(_lib().pkv_kvm_allocate_slots(self._h, request_id, computed_tokens, num_new_tokens,
                                             lookahead_tokens, ctypes.byref(ok)))
        return bool(ok.value)

    def free(self, request_id: int) -> None:
        _check(_lib().pkv_kvm_free(self._h, request_id))

    def get_block_ids(self, request_id: int, group: int = 0) -> list:
        n = ctypes.c_int32()
        _check(_lib().pkv_kvm_get_block_ids(self._h, request_id, group, None, 0, ctypes.byref(n)))
        out = np.zeros(max(n.value, 1), dtype=np.int32)
        _check(_lib().pkv_kvm_get_block_ids(self._h, request_id, group, out.ctypes.data, n.value, ctypes.byref(n)))
        return out[:n.value].tolist()

    def num_free_blocks(self, group: int = 0) -> int:
        n = ctypes.c_int32()
        _check(_lib().pkv_kvm_num_free_blocks(self._h, group, ctypes.byref(n)))
        return n.value

    def format_usage(self) -> str:
        buf = ctypes.create_string_buffer(64 * self.num_groups + 16)
        _check(_lib().pkv_kvm_format_usage(self._h, buf, len(buf)))
        return buf.value.decode()

    def prepare_block_table(self, group: int, request_ids: Sequence[int], max_blocks_per_seq: int) -> np.ndarray:
        ids = np.ascontiguousarray(np.asarray(request_ids, dtype=np.int64))
        table = np.zeros((len(ids), max_blocks_per_seq), dtype=np.int32)
        _check(_lib().pkv_kvm_prepare_block_table(self._h, group, ids.ctypes.data if ids.size else None, len(ids),
                                                  max_blocks_per_seq, table.ctypes.data if ids.size else None))
        return table


def block_num_fixed(max_concurrency: int, sliding_window: int, next_n: int, block_size: int) -> int:
    n = ctypes.c_int64()
    _check(_lib().pkv_block_num_fixed(max_concurrency, sliding_window, next_n, block_size, ctypes.byref(n)))
    return n.value


def block_num_full(max_len: int, max_concurrency: int, block_size: int) -> int:
    n = ctypes.c_int64()
    _check(_lib().pkv_block_num_full(max_len, max_concurrency, block_size, ctypes.byref(n)))
    return n.value


def block_num_budget(budget_bytes: int, fixed_bytes: int, per_token_bytes: int, block_size: int) -> int:
    n = ctypes.c_int64()
    _check(_lib().pkv_block_num_budget(budget_bytes, fixed_bytes, per_token_bytes, block_size, ctypes.byref(n)))
    return n.value
