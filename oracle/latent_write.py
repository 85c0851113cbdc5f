"""Latent-write oracle: RMSNorm + RoPE + paged cache write of the MLA latent, in fp64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check and the benchmark's
CPU baseline may import this module; the HIP library never calls it and shares
no code with it.

What it computes is the fused cache write the "Ascend NPU standalone-deployment
KVCache guide" names for the MLA absorbed form (its MLA section: one step that
normalises, rotates and writes the latent, with the normalised and rotated
rows also returned), and that the "KVCache optimisation skill" page lists as
the fused writer fed by slot_mapping (mode 2 and the appendix on fused
operators).  Per token t, with the row of the KV down-projection split as
[c (kv_lora_rank wide) | k_pe (rope_dim wide)]:

    nope[t] = c / sqrt(mean(c * c) + eps) * gamma                       (RMSNorm)
    rope[t] = k_pe rotated pairwise by the angles whose cosines and
              sines the caller gives in cos[t], sin[t]                  (RoPE)
    cache_nope[slot_mapping[t]] = nope[t];  cache_rope[slot_mapping[t]] = rope[t]

Readings where the pages leave a step open (the native kernel takes the same):
  * The latent part is the first kv_lora_rank values of the row and the rotary
    part the last rope_dim (the order of the split the MLA section gives:
    cache_nope, then cache_rope); RMSNorm touches only the latent part and RoPE
    only the rotary part.
  * cos and sin are per token and per element, [T, rope_dim], already taken at
    the token's position (the guide derives RoPE positions from kv_len and hands
    the operator cos/sin tensors).  Element i pairs with a partner j:
      half (rotate-half) layout:  j = i + rope_dim/2 for i < rope_dim/2, else i - rope_dim/2
      interleaved layout:         j = i ^ 1
    and out[i] = x[i] * cos[i] - x[j] * sin[i] for the first element of a pair,
        out[i] = x[i] * cos[i] + x[j] * sin[i] for the second,
    i.e. the pair (first, second) turned by the angle as the complex number
    first + i * second multiplied by cos + i sin.
  * A negative slot writes nothing (padding tokens); the returned rows are
    produced for every token.
  * The cache layout is the plain [num_blocks * block_size, width] row layout the
    attention kernels read (the Ascend PA_NZ fractal layout is that machine's).
"""
from __future__ import annotations

import numpy as np

HALF, INTERLEAVED = 0, 1


def rms_norm(c: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis, in fp64."""
    c = np.asarray(c, dtype=np.float64)
    ms = np.mean(c * c, axis=-1, keepdims=True)
    return c / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def partner(rope_dim: int, layout: int) -> tuple:
    """(partner index of each element, +1 where the element is the second of its pair)."""
    i = np.arange(rope_dim)
    if layout == HALF:
        h = rope_dim // 2
        return np.where(i < h, i + h, i - h), (i >= h)
    if layout == INTERLEAVED:
        return i ^ 1, (i & 1) == 1
    raise ValueError(f"unknown rope layout {layout}")


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, layout: int) -> np.ndarray:
    """Pairwise rotation of the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    j, second = partner(x.shape[-1], layout)
    sign = np.where(second, 1.0, -1.0)
    return x * cos + sign * x[..., j] * sin


def latent_write(latent, gamma, cos, sin, slot_mapping, eps, cache_nope, cache_rope, layout=HALF):
    """The fused step over T tokens.

    latent [T, kv_lora_rank + rope_dim]; gamma [kv_lora_rank]; cos, sin [T, rope_dim];
    slot_mapping [T]; cache_nope [slots, kv_lora_rank] and cache_rope [slots, rope_dim]
    are updated in place (as fp64 or whatever dtype they hold).  Returns the fp64
    (nope [T, kv_lora_rank], rope [T, rope_dim]) rows."""
    latent = np.asarray(latent, dtype=np.float64)
    rope_dim = cache_rope.shape[-1]
    rank = latent.shape[-1] - rope_dim
    nope = rms_norm(latent[:, :rank], gamma, eps)
    rot = rope(latent[:, rank:], cos, sin, layout)
    for t, s in enumerate(np.asarray(slot_mapping)):
        if s >= 0:
            cache_nope[s] = nope[t]
            cache_rope[s] = rot[t]
    return nope, rot
