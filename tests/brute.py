"""Brute-force attention in numpy float64, used to pin the oracle on tiny inputs.

This takes a different route from the oracle on purpose: it gathers each
sequence's keys and values block by block (the way the HF paged path gathers
through its read index into a logically contiguous tensor, "KV Cache notes",
paged section), expands the KV heads with repeat_kv (np.repeat over the head
axis, "KV Cache notes", MHA -> MQA -> GQA), materialises the full score matrix
with an additive 0 / -inf mask (the eager path of the same page, with the
bottom-right mask of its 40-line minimal implementation and the sliding-window
band), and applies softmax over whole rows.  Tiny sizes only: it builds S x S.
"""
from __future__ import annotations

import numpy as np


def to_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gather_blocks(cache: np.ndarray, table_row: np.ndarray, length: int) -> np.ndarray:
    """[num_blocks, bs, Hkv, D] -> the first `length` logical rows [length, Hkv, D]."""
    bs = cache.shape[1]
    nblk = -(-length // bs)
    blocks = cache[table_row[:nblk]]  # whole blocks, logical order
    return blocks.reshape((nblk * bs,) + cache.shape[2:])[:length]


def eager(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray, scale: float,
          window: int = 0) -> np.ndarray:
    """q [Sq, H, Dk], k [Skv, Hkv, Dk], v [Skv, Hkv, Dv] (float64) -> [Sq, H, Dv].

    Query row r sits at absolute position q_pos[r] and sees keys j <= q_pos[r]
    (and j > q_pos[r] - window when window > 0)."""
    Sq, H, _ = q.shape
    Skv, Hkv, _ = k.shape
    g = H // Hkv
    kr = np.repeat(k, g, axis=1)  # head h <- kv head h // g
    vr = np.repeat(v, g, axis=1)
    scores = np.einsum("qhd,khd->hqk", q, kr) * scale
    j = np.arange(Skv)[None, :]
    p = np.asarray(q_pos)[:, None]
    masked = j > p
    if window > 0:
        masked |= j <= p - window
    # additive mask; masked entries are selected away (not multiplied by 0) so that
    # whatever a padding block holds (NaN included) cannot reach the result
    scores = np.where(masked[None], -np.inf, scores)
    out = np.zeros((Sq, H, v.shape[2]))
    for h in range(H):
        for r in range(Sq):
            vis = ~masked[r]
            if not vis.any():
                continue
            row = scores[h, r, vis]
            e = np.exp(row - row.max())
            out[r, h] = (e / e.sum()) @ vr[vis, h, :]
    return out


def _kv(case, cache_k, cache_v, cache_r, b, L):
    k = to_f64(gather_blocks(cache_k, case.block_table[b], L))
    v = to_f64(gather_blocks(cache_v, case.block_table[b], L))
    if cache_r is not None:  # MLA: key = [latent | rope], value = latent
        k = np.concatenate([k, to_f64(gather_blocks(cache_r, case.block_table[b], L))], axis=-1)
    return k, v


def decode(case, k_cache, v_cache, k_rope_cache=None) -> np.ndarray:
    """Brute-force decode of a workloads.Case whose caches already hold the new tokens."""
    out = np.zeros((case.B, case.H, v_cache.shape[3]))
    for b in range(case.B):
        L = int(case.seq_lens[b])
        if L == 0:
            continue
        k, v = _kv(case, k_cache, v_cache, k_rope_cache, b, L)
        q = to_f64(case.q[b:b + 1])
        if case.q_rope is not None:
            q = np.concatenate([q, to_f64(case.q_rope[b:b + 1])], axis=-1)
        out[b] = eager(q, k, v, np.array([L - 1]), case.scale, case.window)[0]
    return out


def prefill(case, k_cache, v_cache, k_rope_cache=None) -> np.ndarray:
    """Brute-force chunked prefill of a workloads.Case (caches hold the new rows)."""
    T = case.q.shape[0]
    out = np.zeros((T, case.H, v_cache.shape[3]))
    cu = case.cu_seqlens_q
    for b in range(case.B):
        L = int(case.seq_lens[b])
        n = int(cu[b + 1] - cu[b])
        if n == 0:
            continue
        k, v = _kv(case, k_cache, v_cache, k_rope_cache, b, L)
        q = to_f64(case.q[cu[b]:cu[b + 1]])
        if case.q_rope is not None:
            q = np.concatenate([q, to_f64(case.q_rope[cu[b]:cu[b + 1]])], axis=-1)
        pos = np.arange(L - n, L)
        out[cu[b]:cu[b + 1]] = eager(q, k, v, pos, case.scale, case.window)
    return out
