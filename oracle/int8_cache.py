"""INT8 cache oracle: symmetric per-(token, head) int8 quantization of K and V rows and
its dequantization, written out plainly.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check and the benchmark's CPU
baseline may import this module; the HIP library never calls it and shares no code
with it.

The pages name KV-cache quantization as the lever that trades read bandwidth for
memory ("KV Cache notes", the quantized-cache section: the quantized store is
dequantized on every layer and step, which saves memory but can eat the decode-time
gain; "KVCache optimisation skill", advanced features: INT8 cache quantization).
They fix neither the grouping nor the rounding, so this oracle takes the plainest
reading that keeps a paged cache writable one token at a time:

  * one group = one head row of one token (D values); its scale is
    s = max|x| / 127 and its codes are q = round_half_even(x * (127 / max|x|)),
    clamped to [-127, 127]; an all-zero row has s = 0 and q = 0;
  * the value a code stands for is q * s;
  * attention over an int8 cache is the attention of the oracle in pkv_oracle.c over
    the dequantized cache q * s, held in float64 (exact: an 8-bit integer times a
    float32).

The integer decisions (the codes) and the scales are taken in float32 -- the pages
fix no precision, so the kernel's is used, as it must be for codes to match bit for
bit: s = fl32(max / 127), r = fl32(127 / max), q = rint(fl32(x * r)), every
operation IEEE float32 with round to nearest even.

Layout (a choice of this library, not of the pages): codes sit where the bf16 values
would, [num_blocks, block_size, num_kv_heads, D] int8; scales are float32
[num_blocks, num_kv_heads, block_size], so the scales of consecutive keys of one head
are adjacent.
"""
from __future__ import annotations

import numpy as np


def _as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32)


def quantize_rows(x: np.ndarray, dtype: str = "bf16"):
    """Rows of the last axis -> (codes int8 [..., D], scales float32 [...])."""
    xf = _as_f32(x, dtype)
    amax = np.max(np.abs(xf), axis=-1)
    nz = amax > 0
    one27 = np.float32(127.0)
    scale = np.zeros(amax.shape, dtype=np.float32)
    inv = np.zeros(amax.shape, dtype=np.float32)
    scale[nz] = amax[nz] / one27          # float32 / float32: IEEE, round to nearest even
    inv[nz] = one27 / amax[nz]
    prod = (xf * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return codes, scale


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [..., D], scales [...] -> float64 values codes * scales (exact)."""
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None]


def quantize_cache(cache: np.ndarray, dtype: str = "bf16"):
    """A paged cache [NB, bs, Hkv, D] -> (codes [NB, bs, Hkv, D] int8, scales [NB, Hkv, bs] float32)."""
    codes, s = quantize_rows(cache, dtype)
    return codes, np.ascontiguousarray(s.transpose(0, 2, 1))


def dequantize_cache(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(codes [NB, bs, Hkv, D], scales [NB, Hkv, bs]) -> float64 cache [NB, bs, Hkv, D]."""
    return np.ascontiguousarray(dequantize(codes, scales.transpose(0, 2, 1)))


def write_rows(codes: np.ndarray, scales: np.ndarray, slot_mapping, rows: np.ndarray, dtype: str = "bf16"):
    """In place: quantize rows[t] ([Hkv, D]) into slot slot_mapping[t] of (codes, scales); a negative
    slot writes nothing."""
    nb, bs, hkv, d = codes.shape
    q, s = quantize_rows(rows, dtype)
    for t, slot in enumerate(np.asarray(slot_mapping)):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), bs)
        codes[blk, off] = q[t]
        scales[blk, :, off] = s[t]
