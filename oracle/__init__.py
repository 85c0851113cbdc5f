"""CPU oracle for attention over a paged KV cache (ctypes binding of pkv_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never calls it and never falls back to it; the two share no code.

Arrays are numpy: float32 for f32 data, uint16 raw bits for bf16 data, float64
for dequantized int8 caches, int32 for indices.  Results are float64.  What each function computes, and the page each
step follows, is written in the header comment of ``pkv_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2

_ERRORS = {-1: "invalid argument", -2: "index out of range", -3: "out of memory"}


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE double arithmetic)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class _Cache(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("k_rope_cache", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("k_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_lib = None


def load(path: str = _LIB_PATH):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is not None and path == _LIB_PATH:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.or_max_threads.restype = ctypes.c_int
    lib.or_resolve_slots.argtypes = [P, i32, i32, i32, i32, P, P, i32, P]
    lib.or_cache_write.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, i32, P]
    lib.or_paged_decode.argtypes = [ctypes.POINTER(_Cache), i32, i32, i32, ctypes.c_double, i32,
                                    P, P, P, P, P, i32, P, P, i32]
    lib.or_paged_prefill.argtypes = [ctypes.POINTER(_Cache), i32, i32, i32, ctypes.c_double, i32,
                                     P, P, i32, P, P, P, P, i32, P, P, i32]
    for f in (lib.or_resolve_slots, lib.or_cache_write, lib.or_paged_decode, lib.or_paged_prefill):
        f.restype = ctypes.c_int
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported element array dtype {a.dtype}")


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def max_threads(lib=None) -> int:
    return int((lib or load()).or_max_threads())


def resolve_slots(block_table, block_size, num_blocks, batch_idx, pos, lib=None) -> np.ndarray:
    """slot = block_table[b, pos // block_size] * block_size + pos % block_size."""
    lib = lib or load()
    bt = _i32(block_table)
    bi, ps = _i32(batch_idx).ravel(), _i32(pos).ravel()
    out = np.empty(bi.size, dtype=np.int32)
    _check(lib.or_resolve_slots(_ptr(bt), bt.shape[0], bt.shape[1], block_size, num_blocks,
                                _ptr(bi), _ptr(ps), bi.size, _ptr(out)), "resolve_slots")
    return out


def cache_write(cache: np.ndarray, slot_mapping, rows: np.ndarray, lib=None) -> None:
    """In place: cache viewed as [num_slots, row] gets rows[t] at slot_mapping[t] (slot < 0 skips)."""
    lib = lib or load()
    assert cache.flags.c_contiguous and rows.flags.c_contiguous and cache.dtype == rows.dtype
    sm = _i32(slot_mapping).ravel()
    n = sm.size
    if n == 0:
        return
    row_bytes = rows.nbytes // n
    num_slots = cache.nbytes // row_bytes
    _check(lib.or_cache_write(_ptr(cache), num_slots, row_bytes, _ptr(sm), n, _ptr(rows)), "cache_write")


def _cache_struct(k_cache, v_cache, k_rope_cache):
    """k_cache [NB, bs, Hkv, Dk]; v_cache [NB, bs, Hkv, Dv]; k_rope_cache [NB, bs, Hkv, R] or None."""
    dt = _dtype_code(k_cache)
    assert _dtype_code(v_cache) == dt
    nb, bs, hkv, dk = k_cache.shape
    assert v_cache.shape[:3] == (nb, bs, hkv)
    rd = 0
    if k_rope_cache is not None:
        assert _dtype_code(k_rope_cache) == dt and k_rope_cache.shape[:3] == (nb, bs, hkv)
        rd = k_rope_cache.shape[3]
    for a in (k_cache, v_cache, k_rope_cache):
        assert a is None or a.flags.c_contiguous
    return _Cache(_ptr(k_cache), _ptr(v_cache), _ptr(k_rope_cache), nb, bs, hkv, dk,
                  v_cache.shape[3], rd, dt)


def paged_decode(q, k_cache, v_cache, block_table, seq_lens, scale, window=0, q_rope=None,
                 k_rope_cache=None, units=None, want_probs=False, nthreads=0, lib=None):
    """q [B, H, Dk] -> out [B, H, Dv] float64 (and probs [B, H, max_keys] if asked)."""
    lib = lib or load()
    c = _cache_struct(k_cache, v_cache, k_rope_cache)
    B, H, _ = q.shape
    assert q.flags.c_contiguous and _dtype_code(q) == c.dtype
    if q_rope is not None:
        assert q_rope.flags.c_contiguous and _dtype_code(q_rope) == c.dtype
    bt, sl = _i32(block_table), _i32(seq_lens)
    u = None if units is None else _i32(units).ravel()
    out = np.zeros((B, H, c.v_dim), dtype=np.float64)
    max_keys = bt.shape[1] * c.block_size
    probs = np.zeros((B, H, max_keys), dtype=np.float64) if want_probs else None
    _check(lib.or_paged_decode(ctypes.byref(c), B, H, bt.shape[1], float(scale), int(window),
                               _ptr(q), _ptr(q_rope), _ptr(bt), _ptr(sl), _ptr(u),
                               0 if u is None else u.size, _ptr(out), _ptr(probs), int(nthreads)),
           "paged_decode")
    return (out, probs) if want_probs else out


def paged_prefill(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_kv, scale, window=0,
                  q_rope=None, k_rope_cache=None, units=None, want_probs=False, nthreads=0, lib=None):
    """q TND [T, H, Dk] -> out [T, H, Dv] float64 (and probs [T, H, max_keys] if asked)."""
    lib = lib or load()
    c = _cache_struct(k_cache, v_cache, k_rope_cache)
    T, H, _ = q.shape
    assert q.flags.c_contiguous and _dtype_code(q) == c.dtype
    bt, cu, sl = _i32(block_table), _i32(cu_seqlens_q), _i32(seq_lens_kv)
    u = None if units is None else _i32(units).ravel()
    out = np.zeros((T, H, c.v_dim), dtype=np.float64)
    max_keys = bt.shape[1] * c.block_size
    probs = np.zeros((T, H, max_keys), dtype=np.float64) if want_probs else None
    _check(lib.or_paged_prefill(ctypes.byref(c), bt.shape[0], H, bt.shape[1], float(scale),
                                int(window), _ptr(q), _ptr(q_rope), T, _ptr(bt), _ptr(cu), _ptr(sl),
                                _ptr(u), 0 if u is None else u.size, _ptr(out), _ptr(probs),
                                int(nthreads)), "paged_prefill")
    return (out, probs) if want_probs else out
