"""Python binding of libpkv, the gfx950 paged-KV-cache attention library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
of ``include/pkv.h``.  The functions take torch tensors that already live on
the GPU, pass their device pointers and the current HIP stream, and raise
``PkvError`` on a non-OK status.  There is no fallback: if ``libpkv.so`` is
missing, ``load()`` raises.

Names follow the C ABI: ``pkv_resolve_slots``, ``kv_cache_write``,
``kv_rmsnorm_rope_cache``, ``paged_attn_decode``, ``paged_attn_prefill`` (+ their
``*_workspace`` sizes).

``set_check_indices(True)`` turns on host-side bounds checks of the device index
arrays (``checks.py``): each call then copies block_table / seq_lens /
cu_seqlens_q / slot_mapping to the host and raises ``PkvError`` naming the first
entry a kernel would read out of bounds, before launching anything.  It
synchronises, so it is a debugging mode (and cannot run under graph capture).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_F32, PKV_BF16, PKV_INT8 = 0, 1, 2
PKV_ROPE_HALF, PKV_ROPE_INTERLEAVED = 0, 1
STATUS = {0: "PKV_OK", 1: "PKV_ERR_INVALID_ARG", 2: "PKV_ERR_UNSUPPORTED", 3: "PKV_ERR_WORKSPACE",
          4: "PKV_ERR_HIP"}

# Every symbol include/pkv.h declares.
EXPORTS = ("pkv_resolve_slots", "paged_resolve_slots", "kv_cache_write", "kv_cache_write_at", "kv_rmsnorm_rope_cache",
           "paged_attn_decode_workspace",
           "paged_attn_decode", "paged_attn_decode_append", "paged_attn_decode_noalloc",
           "paged_attn_decode_noalloc_capacity",
           "paged_attn_prefill_workspace", "paged_attn_prefill", "pkv_last_error", "pkv_version")


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class PagedCacheDesc(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("k_rope_cache", ctypes.c_void_p), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class AttnParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("scale", ctypes.c_float),
                ("window", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("split_tokens", ctypes.c_int32)]


_lib = None
_check_indices = False


def set_check_indices(on: bool) -> None:
    """Turn the host-side index checks of every entry point on or off (off by default)."""
    global _check_indices
    _check_indices = bool(on)


def check_indices_enabled() -> bool:
    return _check_indices


def _run_check(fn, *args, **kw) -> None:
    from . import checks
    try:
        fn(*args, **kw)
    except checks.IndexCheckError as e:
        raise PkvError(1, f"index check: {e}") from None


def load(path: str = LIB_PATH):
    """Load libpkv.so (built by ``python -m paged_kv_cache_80_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m paged_kv_cache_80_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pc, pp = ctypes.POINTER(PagedCacheDesc), ctypes.POINTER(AttnParams)
    lib.pkv_resolve_slots.argtypes = [P, i32, i32, i32, P, P, i32, P, P]
    lib.paged_resolve_slots.argtypes = [P, i32, i32, P, P, i32, P, P]
    lib.kv_cache_write.argtypes = [P, i32, P, P, P, pc, P]
    lib.kv_cache_write_at.argtypes = [P, i32, P, P, i32, P, P, P, pc, P, P]
    lib.kv_rmsnorm_rope_cache.argtypes = [P, P, P, P, P, i32, ctypes.c_float, i32, pc, P, P, P]
    lib.paged_attn_decode_workspace.argtypes = [pp, pc]
    lib.paged_attn_decode_workspace.restype = sz
    lib.paged_attn_decode.argtypes = [P, P, pc, P, P, pp, P, P, sz, P]
    lib.paged_attn_decode_append.argtypes = [P, P, P, P, P, pc, P, P, pp, P, P, sz, P]
    lib.paged_attn_decode_noalloc.argtypes = [P, P, pc, P, P, pp, P, P]
    lib.paged_attn_decode_noalloc_capacity.argtypes = []
    lib.paged_attn_decode_noalloc_capacity.restype = sz
    lib.paged_attn_prefill_workspace.argtypes = [pp, pc, i32]
    lib.paged_attn_prefill_workspace.restype = sz
    lib.paged_attn_prefill.argtypes = [P, P, pc, P, P, P, i32, i32, pp, P, P, sz, P]
    for f in (lib.pkv_resolve_slots, lib.paged_resolve_slots, lib.kv_cache_write, lib.kv_cache_write_at,
              lib.kv_rmsnorm_rope_cache, lib.paged_attn_decode,
              lib.paged_attn_decode_noalloc, lib.paged_attn_prefill):
        f.restype = ctypes.c_int
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise PkvError(status, load().pkv_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.int8:
        return PKV_INT8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _i32(t: torch.Tensor) -> torch.Tensor:
    if t.dtype != torch.int32:
        raise TypeError(f"index tensors must be int32, got {t.dtype}")
    return t


def _check_elems(cache: "PagedKVCache", *ts) -> None:
    """q / k / v / q_rope take the cache dtype; an int8 cache takes bf16 ones."""
    want = torch.bfloat16 if cache.k_cache.dtype == torch.int8 else cache.k_cache.dtype
    for t in ts:
        if t is not None and t.dtype != want:
            raise TypeError(f"expected {want} rows for a {cache.k_cache.dtype} cache, got {t.dtype}")


def _expect(t: Optional[torch.Tensor], shape: tuple, name: str) -> None:
    """The kernels read exactly these extents through plain pointers: a smaller tensor would be
    read past its end, so a mismatch is refused here."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream) -> Optional[int]:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


@dataclasses.dataclass
class PagedKVCache:
    """One layer's paged cache: k_cache, v_cache [num_blocks, block_size, H_kv, D].

    MLA: k_cache is the latent (cache_nope), v_cache is None (the value is the
    latent itself) and k_rope_cache [num_blocks, block_size, 1, 64] holds the
    rotary part.  INT8: k_cache / v_cache are int8 codes and k_scale / v_scale
    float32 [num_blocks, H_kv, block_size] scales."""
    k_cache: torch.Tensor
    v_cache: Optional[torch.Tensor] = None
    k_rope_cache: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None

    def desc(self) -> PagedCacheDesc:
        k = self.k_cache
        nb, bs, hkv, d = k.shape
        v = k if self.v_cache is None else self.v_cache
        if v.shape != k.shape or v.dtype != k.dtype:
            raise ValueError("v_cache must match k_cache in shape and dtype")
        rd = 0 if self.k_rope_cache is None else self.k_rope_cache.shape[3]
        for sc in (self.k_scale, self.v_scale):
            if sc is not None and (sc.dtype != torch.float32 or tuple(sc.shape) != (nb, hkv, bs)):
                raise ValueError("scales must be float32 [num_blocks, num_kv_heads, block_size]")
        return PagedCacheDesc(_ptr(k), _ptr(v), _ptr(self.k_rope_cache), nb, bs, hkv, d, rd,
                              _dtype_code(k), _ptr(self.k_scale), _ptr(self.v_scale))


def pkv_resolve_slots(block_table: torch.Tensor, block_size: int, batch_idx: torch.Tensor,
                      pos: torch.Tensor, slots_out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """slot = block_table[b, pos // block_size] * block_size + pos % block_size (int32; pos < 0 -> -1)."""
    bt = _i32(block_table)
    n = batch_idx.numel()
    if bt.dim() != 2:
        raise ValueError("block_table must be [batch, max_blocks_per_seq]")
    _expect(pos, (n,), "pos")
    _expect(slots_out, (n,), "slots_out")
    if _check_indices:
        from . import checks
        _run_check(checks.check_resolve, bt, block_size, batch_idx, pos)
    if slots_out is None:
        slots_out = torch.empty(n, dtype=torch.int32, device=bt.device)
    _check(load().pkv_resolve_slots(_ptr(bt), bt.shape[0], bt.shape[1], block_size,
                                    _ptr(_i32(batch_idx)), _ptr(_i32(pos)), n, _ptr(slots_out),
                                    _stream(stream)))
    return slots_out


def paged_resolve_slots(block_table: torch.Tensor, block_size: int, batch_idx: torch.Tensor,
                        pos: torch.Tensor, slots_out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """pkv_resolve_slots through the entry point that takes no batch count."""
    bt = _i32(block_table)
    n = batch_idx.numel()
    if bt.dim() != 2:
        raise ValueError("block_table must be [batch, max_blocks_per_seq]")
    _expect(pos, (n,), "pos")
    _expect(slots_out, (n,), "slots_out")
    if _check_indices:
        from . import checks
        _run_check(checks.check_resolve, bt, block_size, batch_idx, pos)
    if slots_out is None:
        slots_out = torch.empty(n, dtype=torch.int32, device=bt.device)
    _check(load().paged_resolve_slots(_ptr(bt), bt.shape[1], block_size, _ptr(_i32(batch_idx)),
                                      _ptr(_i32(pos)), n, _ptr(slots_out), _stream(stream)))
    return slots_out


def kv_cache_write(slot_mapping: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor],
                   cache: PagedKVCache, k_rope: Optional[torch.Tensor] = None, stream=None) -> None:
    """Copy row t of k (v, k_rope) to cache row slot_mapping[t] (negative slots skip); an int8 cache
    quantizes the bf16 rows instead."""
    n = slot_mapping.numel()
    _, _, hkv, hd = cache.k_cache.shape
    _expect(k, (n, hkv, hd), "k")
    _expect(v, (n, hkv, hd), "v")
    if k_rope is not None:
        _expect(k_rope, (n, hkv, cache.k_rope_cache.shape[3]), "k_rope")
    _check_elems(cache, k, v, k_rope)
    d = cache.desc()
    if _check_indices:
        from . import checks
        _run_check(checks.check_slots, slot_mapping, d.num_blocks * d.block_size)
    _check(load().kv_cache_write(_ptr(_i32(slot_mapping)), slot_mapping.numel(), _ptr(k), _ptr(v),
                                 _ptr(k_rope), ctypes.byref(d), _stream(stream)))


def kv_cache_write_at(block_table: torch.Tensor, batch_idx: torch.Tensor, pos: torch.Tensor, k: torch.Tensor,
                      v: Optional[torch.Tensor], cache: PagedKVCache, k_rope: Optional[torch.Tensor] = None,
                      slots_out: Optional[torch.Tensor] = None, stream=None) -> Optional[torch.Tensor]:
    """Resolve (batch_idx[t], pos[t]) through block_table and write row t there, in one launch
    (pos < 0 skips the row).  Returns slots_out, which receives the resolved slots when given."""
    bt = _i32(block_table)
    n = batch_idx.numel()
    if bt.dim() != 2:
        raise ValueError("block_table must be [batch, max_blocks_per_seq]")
    _expect(pos, (n,), "pos")
    _expect(slots_out, (n,), "slots_out")
    _, bs, hkv, hd = cache.k_cache.shape
    _expect(k, (n, hkv, hd), "k")
    _expect(v, (n, hkv, hd), "v")
    if k_rope is not None:
        _expect(k_rope, (n, hkv, cache.k_rope_cache.shape[3]), "k_rope")
    _check_elems(cache, k, v, k_rope)
    d = cache.desc()
    if _check_indices:
        from . import checks
        _run_check(checks.check_write_at, bt, bs, batch_idx, pos, d.num_blocks)
    if slots_out is not None:
        _i32(slots_out)
    _check(load().kv_cache_write_at(_ptr(bt), bt.shape[1], _ptr(_i32(batch_idx)), _ptr(_i32(pos)), n, _ptr(k), _ptr(v),
                                    _ptr(k_rope), ctypes.byref(d), _ptr(slots_out), _stream(stream)))
    return slots_out


def kv_rmsnorm_rope_cache(latent: torch.Tensor, gamma: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                          slot_mapping: torch.Tensor, eps: float, cache: PagedKVCache,
                          rope_layout: int = PKV_ROPE_HALF, k_nope_out: Optional[torch.Tensor] = None,
                          k_rope_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """RMSNorm(latent[:, :512]) * gamma and RoPE(latent[:, 512:]; cos, sin) into the MLA cache rows
    slot_mapping[t] (negative slots skip), and into k_nope_out / k_rope_out when given."""
    n = slot_mapping.numel()
    _expect(latent, (n, 576), "latent")
    _expect(gamma, (512,), "gamma")
    _expect(cos, (n, 64), "cos")
    _expect(sin, (n, 64), "sin")
    _expect(k_nope_out, (n, 512), "k_nope_out")
    _expect(k_rope_out, (n, 64), "k_rope_out")
    d = cache.desc()
    for t in (latent, gamma, cos, sin, k_nope_out, k_rope_out):
        if t is not None and t.dtype != cache.k_cache.dtype:
            raise TypeError("every array must have the cache dtype")
    if _check_indices:
        from . import checks
        _run_check(checks.check_slots, slot_mapping, d.num_blocks * d.block_size)
    _check(load().kv_rmsnorm_rope_cache(_ptr(latent), _ptr(gamma), _ptr(cos), _ptr(sin), _ptr(_i32(slot_mapping)), n,
                                        float(eps), rope_layout, ctypes.byref(d), _ptr(k_nope_out), _ptr(k_rope_out),
                                        _stream(stream)))


def _check_attn_shapes(cache: PagedKVCache, q, q_rope, block_table, batch: int, out) -> None:
    rows, H, D = q.shape
    if D != cache.k_cache.shape[3]:
        raise ValueError(f"q head_dim {D} differs from the cache's {cache.k_cache.shape[3]}")
    if q_rope is not None and cache.k_rope_cache is not None:
        _expect(q_rope, (rows, H, cache.k_rope_cache.shape[3]), "q_rope")
    if block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError(f"block_table must be [{batch}, max_blocks_per_seq], got {tuple(block_table.shape)}")
    _expect(out, (rows, H, D), "out")


def _params(batch, num_q_heads, block_table, scale, window, out_dtype, split_tokens) -> AttnParams:
    return AttnParams(int(batch), int(num_q_heads), int(block_table.shape[1]), float(scale),
                      int(window), int(out_dtype), int(split_tokens))


def paged_attn_decode_workspace(cache: PagedKVCache, batch: int, num_q_heads: int,
                                max_blocks_per_seq: int, scale: float, window: int = 0,
                                out_dtype: int = PKV_BF16, split_tokens: int = 0) -> int:
    p = AttnParams(batch, num_q_heads, max_blocks_per_seq, scale, window, out_dtype, split_tokens)
    return int(load().paged_attn_decode_workspace(ctypes.byref(p), ctypes.byref(cache.desc())))


def paged_attn_decode(q: torch.Tensor, cache: PagedKVCache, block_table: torch.Tensor,
                      seq_lens: torch.Tensor, scale: float, window: int = 0,
                      q_rope: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                      out_dtype: Optional[torch.dtype] = None, split_tokens: int = 0,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q [B, H, D] -> out [B, H, D]; seq_lens counts keys including this step's token."""
    B, H, D = q.shape
    _check_attn_shapes(cache, q, q_rope, block_table, B, out)
    _expect(seq_lens, (B,), "seq_lens")
    _check_elems(cache, q, q_rope)
    if out is None:
        out = torch.empty((B, H, D), dtype=out_dtype or q.dtype, device=q.device)
    d = cache.desc()
    p = _params(B, H, block_table, scale, window, _dtype_code(out), split_tokens)
    if _check_indices:
        from . import checks
        _run_check(checks.check_decode, block_table, seq_lens, d.block_size, d.num_blocks, int(window))
    lib = load()
    need = int(lib.paged_attn_decode_workspace(ctypes.byref(p), ctypes.byref(d)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attn_decode(_ptr(q), _ptr(q_rope), ctypes.byref(d), _ptr(_i32(block_table)),
                                 _ptr(_i32(seq_lens)), ctypes.byref(p), _ptr(out), _ptr(workspace),
                                 ws_bytes, _stream(stream)))
    return out


def paged_attn_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: Optional[torch.Tensor],
                             cache: PagedKVCache, block_table: torch.Tensor, seq_lens: torch.Tensor,
                             scale: float, window: int = 0, q_rope: Optional[torch.Tensor] = None,
                             k_rope_new: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                             out_dtype: Optional[torch.dtype] = None, split_tokens: int = 0,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Write each sequence's newest K/V row (k_new, v_new [B, H_kv, D]; k_rope_new [B, 1, R]
    for MLA) at position seq_lens[b] - 1, then decode as paged_attn_decode: one launch on
    the bf16 stream-split path."""
    B, H, D = q.shape
    _check_attn_shapes(cache, q, q_rope, block_table, B, out)
    _expect(seq_lens, (B,), "seq_lens")
    _, _, hkv, hd = cache.k_cache.shape
    _expect(k_new, (B, hkv, hd), "k_new")
    _expect(v_new, (B, hkv, hd), "v_new")
    if k_rope_new is not None:
        _expect(k_rope_new, (B, hkv, cache.k_rope_cache.shape[3]), "k_rope_new")
    _check_elems(cache, q, q_rope, k_new, v_new, k_rope_new)
    if out is None:
        out = torch.empty((B, H, D), dtype=out_dtype or q.dtype, device=q.device)
    d = cache.desc()
    p = _params(B, H, block_table, scale, window, _dtype_code(out), split_tokens)
    if _check_indices:
        from . import checks
        _run_check(checks.check_append, block_table, seq_lens, d.block_size, d.num_blocks, int(window))
    lib = load()
    need = int(lib.paged_attn_decode_workspace(ctypes.byref(p), ctypes.byref(d)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attn_decode_append(_ptr(q), _ptr(q_rope), _ptr(k_new), _ptr(v_new), _ptr(k_rope_new),
                                        ctypes.byref(d), _ptr(_i32(block_table)), _ptr(_i32(seq_lens)),
                                        ctypes.byref(p), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def paged_attn_decode_noalloc(q: torch.Tensor, cache: PagedKVCache, block_table: torch.Tensor,
                              seq_lens: torch.Tensor, scale: float, out: torch.Tensor, window: int = 0,
                              q_rope: Optional[torch.Tensor] = None, split_tokens: int = 0,
                              stream=None) -> torch.Tensor:
    """paged_attn_decode for callers that cannot allocate: the caller passes `out`, the split's
    scratch is the library's static per-GPU array (paged_attn_decode_noalloc_capacity() bytes).
    Calls that overlap on one GPU race on that array."""
    B, H, D = q.shape
    _check_attn_shapes(cache, q, q_rope, block_table, B, out)
    _expect(seq_lens, (B,), "seq_lens")
    _check_elems(cache, q, q_rope)
    d = cache.desc()
    p = _params(B, H, block_table, scale, window, _dtype_code(out), split_tokens)
    if _check_indices:
        from . import checks
        _run_check(checks.check_decode, block_table, seq_lens, d.block_size, d.num_blocks, int(window))
    _check(load().paged_attn_decode_noalloc(_ptr(q), _ptr(q_rope), ctypes.byref(d), _ptr(_i32(block_table)),
                                            _ptr(_i32(seq_lens)), ctypes.byref(p), _ptr(out), _stream(stream)))
    return out


def paged_attn_decode_noalloc_capacity() -> int:
    return int(load().paged_attn_decode_noalloc_capacity())


def paged_attn_prefill_workspace(cache: PagedKVCache, batch: int, num_q_heads: int, max_blocks_per_seq: int,
                                 total_q: int, scale: float, window: int = 0, out_dtype: int = PKV_BF16) -> int:
    """Bytes of workspace a prefill call of these sizes needs (0 when its keys are not split)."""
    p = AttnParams(batch, num_q_heads, max_blocks_per_seq, scale, window, out_dtype, 0)
    return int(load().paged_attn_prefill_workspace(ctypes.byref(p), ctypes.byref(cache.desc()), int(total_q)))


def paged_attn_prefill(q: torch.Tensor, cache: PagedKVCache, block_table: torch.Tensor,
                       cu_seqlens_q: torch.Tensor, seq_lens_kv: torch.Tensor, max_q_len: Optional[int],
                       scale: float, window: int = 0, q_rope: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q TND [T, H, D] -> out [T, H, D], bottom-right causal over each sequence's keys.

    max_q_len must be at least every sequence's row count (it sizes the grid; rows past
    it would stay unwritten).  None derives it from cu_seqlens_q, which costs a
    synchronising device-to-host copy when cu_seqlens_q lives on the GPU."""
    T, H, D = q.shape
    B = cu_seqlens_q.numel() - 1
    _check_attn_shapes(cache, q, q_rope, block_table, B, out)
    _expect(seq_lens_kv, (B,), "seq_lens_kv")
    _check_elems(cache, q, q_rope)
    if max_q_len is None:
        max_q_len = int(torch.diff(cu_seqlens_q.detach().cpu().long()).max()) if B > 0 else 0
    if out is None:
        out = torch.empty((T, H, D), dtype=out_dtype or q.dtype, device=q.device)
    d = cache.desc()
    p = _params(B, H, block_table, scale, window, _dtype_code(out), 0)
    if _check_indices:
        from . import checks
        _run_check(checks.check_prefill, block_table, cu_seqlens_q, seq_lens_kv, T, int(max_q_len),
                   d.block_size, d.num_blocks, int(window))
    lib = load()
    need = int(lib.paged_attn_prefill_workspace(ctypes.byref(p), ctypes.byref(d), T))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attn_prefill(_ptr(q), _ptr(q_rope), ctypes.byref(d), _ptr(_i32(block_table)),
                                  _ptr(_i32(cu_seqlens_q)), _ptr(_i32(seq_lens_kv)), T, int(max_q_len),
                                  ctypes.byref(p), _ptr(out), _ptr(workspace), ws_bytes,
                                  _stream(stream)))
    return out


def version() -> str:
    return load().pkv_version().decode()
