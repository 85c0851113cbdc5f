"""Seeded synthetic inputs for paged-KV-cache attention.

This module is shared by the tests, the benchmark and the smoke check, and it
holds none of the method's arithmetic: it draws sequence lengths, block-table
permutations and N(0, 1) values, and lists which logical positions receive new
tokens.  Slots, scores, softmax and outputs are computed elsewhere (the oracle
and the HIP library, independently).

Draw order for every case (fixed, so a seed names one input):
    seq_lens -> block permutation -> q (-> q_rope) -> cache pool -> new k, v (-> k_rope)

Values are N(0, 1) float32 (see Draws for how each array's stream is laid
out); bf16 cases round them to bfloat16 by round-to-nearest-even and store
the raw uint16 bits.

Shapes follow the pages' workloads: the 2-batch / 128-token-block layout of the
skill page's section 3.1, llama2-7B (MHA 32 heads) and llama2-70B (GQA 64/8)
head geometry from the "KV Cache notes" accounting table, and the MLA latent
(512 wide, 64-wide rope part) of the MLA sections.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
from typing import Optional

import numpy as np

NAN_BF16 = np.uint16(0x7FC0)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 raw bits, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 raw bits -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 26) -> np.ndarray:
    """N(0,1) values of the given shape from one generator: float32 array or bf16 raw bits."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = rng.standard_normal(e - s, dtype=np.float32)
        out[s:e] = v if dtype == "f32" else bf16_bits(v)
    return out.reshape(shape)


_CHUNK = 1 << 22  # values per independent sub-stream; fixed, so results do not depend on threads
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL


class Draws:
    """The random source of one case.

    Integers (lengths, permutations) come from one generator seeded by the
    case seed.  Each value array gets its own child of the case's SeedSequence,
    spawned in draw order, and is filled in fixed chunks of 2^22 values, chunk i
    drawn from the i-th grandchild -- so large arrays fill in parallel threads
    and the values depend only on (seed, draw order, shape)."""

    def __init__(self, seed: int):
        self.ss = np.random.SeedSequence(seed)
        self.rng = np.random.default_rng(self.ss.spawn(1)[0])

    def normal(self, shape, dtype: str) -> np.ndarray:
        child = self.ss.spawn(1)[0]
        n = int(np.prod(shape)) if len(shape) else 1
        out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
        starts = list(range(0, n, _CHUNK))
        seeds = child.spawn(len(starts))

        def fill(i):
            s = starts[i]
            e = min(n, s + _CHUNK)
            v = np.random.default_rng(seeds[i]).standard_normal(e - s, dtype=np.float32)
            out[s:e] = v if dtype == "f32" else bf16_bits(v)

        list(_pool().map(fill, range(len(starts))))
        return out.reshape(shape)


def nan_fill(a: np.ndarray) -> None:
    if a.dtype == np.float32:
        a[...] = np.float32("nan")
    else:
        a[...] = NAN_BF16


@dataclasses.dataclass
class Case:
    """One synthetic call of the hot path.

    Decode (kind == "decode"): q [B, H, D]; the new token of sequence b sits at
    position seq_lens[b] - 1 (-1: an empty sequence has no new token).  Prefill (kind == "prefill"): q TND [T, H, D],
    cu_seqlens_q [B+1]; the new rows of sequence b sit at positions
    seq_lens[b] - n_b .. seq_lens[b] - 1.  In both, new_k / new_v rows (one per
    new token, in new_batch_idx / new_pos order) must be written to the cache
    before attention reads it.  MLA cases (rope_dim > 0) keep the latent in
    k_cache, use it as the value too (v_cache is None) and keep the rope part in
    k_rope_cache.
    """
    name: str
    kind: str
    dtype: str
    B: int
    H: int
    Hkv: int
    D: int
    rope_dim: int
    block_size: int
    num_blocks: int
    block_table: np.ndarray
    seq_lens: np.ndarray
    q: np.ndarray
    q_rope: Optional[np.ndarray]
    k_cache: np.ndarray
    v_cache: Optional[np.ndarray]
    k_rope_cache: Optional[np.ndarray]
    new_k: np.ndarray
    new_v: Optional[np.ndarray]
    new_k_rope: Optional[np.ndarray]
    new_batch_idx: np.ndarray
    new_pos: np.ndarray
    scale: float
    window: int = 0
    cu_seqlens_q: Optional[np.ndarray] = None
    null_block: bool = False
    int8: bool = False  # the cache is stored as int8 codes + scales, quantized from these bf16 values

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]

    @property
    def G(self) -> int:
        return self.H // self.Hkv

    @property
    def is_mla(self) -> bool:
        return self.rope_dim > 0

    @property
    def v_cache_or_k(self) -> np.ndarray:
        return self.k_cache if self.v_cache is None else self.v_cache

    def copy_caches(self) -> "Case":
        """Shallow copy with private cache arrays (for writing into)."""
        c = dataclasses.replace(self)
        c.k_cache = self.k_cache.copy()
        c.v_cache = None if self.v_cache is None else self.v_cache.copy()
        c.k_rope_cache = None if self.k_rope_cache is None else self.k_rope_cache.copy()
        return c


def _tables(rng, B, seq_lens, block_size, max_blocks, num_blocks_exact, spare_frac, null_block,
            window):
    """Block tables drawn as a seeded permutation of the pool.

    Without a null block every pool block is data and the table is a
    permutation of the whole pool (num_blocks_exact = B * max_blocks).  With a
    null block, block 0 is reserved, the pool holds 1 + ceil((1+spare) * need)
    blocks, each sequence gets blocks only for the logical blocks it needs
    (ceil(L/bs), minus the ones wholly before its window), and every other table
    entry is 0."""
    if not null_block:
        nb = num_blocks_exact
        perm = rng.permutation(nb).astype(np.int32)
        return perm.reshape(B, max_blocks), nb
    first_real = []
    need = 0
    for L in seq_lens:
        nblk = -(-int(L) // block_size)
        lo = max(0, int(L) - window) if window > 0 else 0
        fb = lo // block_size
        first_real.append(fb)
        need += nblk - fb
    nb = 1 + int(math.ceil((1.0 + spare_frac) * need))
    perm = (rng.permutation(nb - 1) + 1).astype(np.int32)
    bt = np.zeros((B, max_blocks), dtype=np.int32)
    k = 0
    for b, L in enumerate(seq_lens):
        nblk = -(-int(L) // block_size)
        for lb in range(first_real[b], nblk):
            bt[b, lb] = perm[k]
            k += 1
    return bt, nb


def decode_case(seed: int, B: int, H: int, Hkv: int, D: int, dtype: str, *, block_size: int = 128,
                max_blocks: int, seq_lens=None, len_range=None, window: int = 0,
                null_block: bool = False, spare_frac: float = 0.1, rope_dim: int = 0,
                scale: Optional[float] = None, table: Optional[np.ndarray] = None,
                int8: bool = False, name: str = "decode") -> Case:
    """Decode case: one new token per sequence at position seq_lens[b] - 1."""
    dr = Draws(seed)
    rng = dr.rng
    if seq_lens is None:
        lo, hi = len_range
        seq_lens = rng.integers(lo, hi + 1, size=B)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.max(initial=0) <= max_blocks * block_size
    if table is not None:
        bt = np.asarray(table, dtype=np.int32)
        nb = int(bt.max()) + 1
    else:
        bt, nb = _tables(rng, B, seq_lens, block_size, max_blocks, B * max_blocks, spare_frac,
                         null_block, window)
    q = dr.normal((B, H, D), dtype)
    q_rope = dr.normal((B, H, rope_dim), dtype) if rope_dim else None
    k_cache = dr.normal((nb, block_size, Hkv, D), dtype)
    v_cache = None if rope_dim else dr.normal((nb, block_size, Hkv, D), dtype)
    k_rope_cache = dr.normal((nb, block_size, Hkv, rope_dim), dtype) if rope_dim else None
    if null_block:
        for a in (k_cache, v_cache, k_rope_cache):
            if a is not None:
                nan_fill(a[0])
    new_k = dr.normal((B, Hkv, D), dtype)
    new_v = None if rope_dim else dr.normal((B, Hkv, D), dtype)
    new_k_rope = dr.normal((B, Hkv, rope_dim), dtype) if rope_dim else None
    if scale is None:
        scale = 1.0 / math.sqrt(D + rope_dim)
    return Case(name=name, kind="decode", dtype=dtype, B=B, H=H, Hkv=Hkv, D=D, rope_dim=rope_dim,
                block_size=block_size, num_blocks=nb, block_table=bt, seq_lens=seq_lens, q=q,
                q_rope=q_rope, k_cache=k_cache, v_cache=v_cache, k_rope_cache=k_rope_cache,
                new_k=new_k, new_v=new_v, new_k_rope=new_k_rope,
                new_batch_idx=np.arange(B, dtype=np.int32),
                new_pos=(seq_lens - 1).astype(np.int32), scale=float(scale),
                window=window, null_block=null_block, int8=int8)


def prefill_case(seed: int, B: int, H: int, Hkv: int, D: int, dtype: str, *, cached, new,
                 block_size: int = 128, max_blocks: Optional[int] = None, window: int = 0,
                 rope_dim: int = 0, scale: Optional[float] = None, null_block: bool = False,
                 spare_frac: float = 0.1, name: str = "prefill") -> Case:
    """Chunked prefill: sequence b holds cached[b] tokens and gets new[b] more."""
    dr = Draws(seed)
    rng = dr.rng
    cached = np.broadcast_to(np.asarray(cached, dtype=np.int32), (B,)).copy()
    new = np.broadcast_to(np.asarray(new, dtype=np.int32), (B,)).copy()
    seq_lens = (cached + new).astype(np.int32)
    if max_blocks is None:
        max_blocks = max(1, -(-int(seq_lens.max()) // block_size))
    bt, nb = _tables(rng, B, seq_lens, block_size, max_blocks, B * max_blocks, spare_frac,
                     null_block, 0)
    T = int(new.sum())
    q = dr.normal((T, H, D), dtype)
    q_rope = dr.normal((T, H, rope_dim), dtype) if rope_dim else None
    k_cache = dr.normal((nb, block_size, Hkv, D), dtype)
    v_cache = None if rope_dim else dr.normal((nb, block_size, Hkv, D), dtype)
    k_rope_cache = dr.normal((nb, block_size, Hkv, rope_dim), dtype) if rope_dim else None
    if null_block:
        for a in (k_cache, v_cache, k_rope_cache):
            if a is not None:
                nan_fill(a[0])
    new_k = dr.normal((T, Hkv, D), dtype)
    new_v = None if rope_dim else dr.normal((T, Hkv, D), dtype)
    new_k_rope = dr.normal((T, Hkv, rope_dim), dtype) if rope_dim else None
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(new)
    bidx = np.repeat(np.arange(B, dtype=np.int32), new)
    pos = np.concatenate([np.arange(c, c + n, dtype=np.int32) for c, n in zip(cached, new)]) \
        if T else np.zeros(0, dtype=np.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(D + rope_dim)
    return Case(name=name, kind="prefill", dtype=dtype, B=B, H=H, Hkv=Hkv, D=D, rope_dim=rope_dim,
                block_size=block_size, num_blocks=nb, block_table=bt, seq_lens=seq_lens, q=q,
                q_rope=q_rope, k_cache=k_cache, v_cache=v_cache, k_rope_cache=k_rope_cache,
                new_k=new_k, new_v=new_v, new_k_rope=new_k_rope, new_batch_idx=bidx,
                new_pos=pos.astype(np.int32), scale=float(scale), window=window,
                cu_seqlens_q=cu, null_block=null_block)


@dataclasses.dataclass
class LatentCase:
    """One call of the fused latent write (RMSNorm + RoPE + paged write, MLA).

    latent [T, 512 + 64] is the KV down-projection's row per new token, gamma [512]
    the norm weight, cos / sin [T, 64] the rotary inputs at each token's position
    (the operator takes them as given; here they are the cosines and sines of
    position x 10000^(-2k/64), k the pair index, laid out for `layout`: 0 = the two
    halves, 1 = interleaved pairs).  New token i of sequence new_batch_idx[i] sits at
    position new_pos[i] (-1: a padding token with no slot).  The cache arrays are
    the MLA latent and rotary caches [num_blocks, block_size, 1, width]."""
    name: str
    kind: str
    dtype: str
    B: int
    block_size: int
    num_blocks: int
    block_table: np.ndarray
    new_batch_idx: np.ndarray
    new_pos: np.ndarray
    latent: np.ndarray
    gamma: np.ndarray
    cos: np.ndarray
    sin: np.ndarray
    cache_nope: np.ndarray
    cache_rope: np.ndarray
    eps: float
    layout: int
    outputs: bool = True

    @property
    def T(self) -> int:
        return int(self.new_pos.size)


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return x if dtype == "f32" else bf16_bits(x)


def latent_case(seed: int, B: int, dtype: str, *, new, cached=0, block_size: int = 128, layout: int = 0,
                eps: float = 1e-6, pad_every: int = 0, outputs: bool = True, spare_blocks: int = 3,
                name: str = "latent_write") -> LatentCase:
    """Sequence b holds cached[b] tokens and gets new[b] more; every pad_every-th
    token (when > 0) is a padding token.  Draw order: table permutation -> latent ->
    gamma -> cache pool."""
    dr = Draws(seed)
    rng = dr.rng
    cached = np.broadcast_to(np.asarray(cached, dtype=np.int64), (B,)).copy()
    new = np.broadcast_to(np.asarray(new, dtype=np.int64), (B,)).copy()
    total = cached + new
    max_blocks = max(1, -(-int(total.max(initial=1)) // block_size))
    nb = B * max_blocks + spare_blocks
    bt = rng.permutation(nb)[:B * max_blocks].astype(np.int32).reshape(B, max_blocks)
    bidx = np.repeat(np.arange(B, dtype=np.int32), new)
    pos = np.concatenate([np.arange(c, c + n) for c, n in zip(cached, new)]).astype(np.int32) \
        if new.sum() else np.zeros(0, dtype=np.int32)
    if pad_every > 0:
        pos[::pad_every] = -1
    T = pos.size
    latent = dr.normal((T, 512 + 64), dtype)
    gamma = _to_dtype(1.0 + 0.25 * dr.normal((512,), "f32"), dtype)
    cache_nope = dr.normal((nb, block_size, 1, 512), dtype)
    cache_rope = dr.normal((nb, block_size, 1, 64), dtype)
    inv = 10000.0 ** (-2.0 * np.arange(32) / 64.0)
    theta = np.outer(np.maximum(pos, 0).astype(np.float64), inv)
    theta = np.concatenate([theta, theta], axis=1) if layout == 0 else np.repeat(theta, 2, axis=1)
    return LatentCase(name=name, kind="latent_write", dtype=dtype, B=B, block_size=block_size, num_blocks=nb,
                      block_table=bt, new_batch_idx=bidx, new_pos=pos, latent=latent, gamma=gamma,
                      cos=_to_dtype(np.cos(theta), dtype), sin=_to_dtype(np.sin(theta), dtype),
                      cache_nope=cache_nope, cache_rope=cache_rope, eps=float(eps), layout=layout,
                      outputs=outputs)


# ---------------------------------------------------------------------------
# The five workloads at full size.
# ---------------------------------------------------------------------------

def tiny_f32_decode(seed: int = 0) -> Case:
    """B=2, H=H_kv=4, d_h=128, 4 blocks of 128 per sequence (max length 512),
    block_table = arange(8).reshape(2, 4), lengths uniform in [1, 512], fp32."""
    return decode_case(seed, 2, 4, 4, 128, "f32", max_blocks=4, len_range=(1, 512),
                       table=np.arange(8, dtype=np.int32).reshape(2, 4), name="tiny_f32_decode")


def mha_decode_7b(seed: int = 0, int8: bool = False) -> Case:
    """llama2-7B single layer: B=64, H=H_kv=32, d_h=128, every length 2048,
    table = a permutation of 1024 blocks, bf16 (int8: the same values held in an
    int8 cache)."""
    return decode_case(seed, 64, 32, 32, 128, "bf16", max_blocks=16,
                       seq_lens=np.full(64, 2048, dtype=np.int32), int8=int8,
                       name="mha_decode_7b" + ("_int8" if int8 else ""))


def gqa_decode_70b(seed: int = 0, window: int = 0, int8: bool = False) -> Case:
    """llama2-70B single layer: B=32, H=64, H_kv=8, d_h=128, lengths uniform in
    [1024, 32768], shuffled table over a pool with 10% spare blocks and null
    block 0; with window=4096 the blocks wholly before the window are null.
    int8: the same values held in an int8 cache (codes + per-(token, head) scales)."""
    return decode_case(seed, 32, 64, 8, 128, "bf16", max_blocks=256, len_range=(1024, 32768),
                       window=window, null_block=True, spare_frac=0.1, int8=int8,
                       name="gqa_decode_70b" + ("_window%d" % window if window else "") + ("_int8" if int8 else ""))


def chunked_prefill(seed: int = 0) -> Case:
    """B=8, H=32, H_kv=8, d_h=128: 4096 cached tokens per sequence plus 512 new
    query rows, causal over the new rows; table = a permutation of 288 blocks."""
    return prefill_case(seed, 8, 32, 8, 128, "bf16", cached=4096, new=512, max_blocks=36,
                        name="chunked_prefill")


def gqa_mtp_decode(seed: int = 0) -> Case:
    """Multi-token decode on the llama2-70B layer shapes: B=32, H=64, H_kv=8, d_h=128,
    total lengths uniform in [1024, 32768] (drawn from their own seeded stream), of which
    the last 4 positions of every sequence are new query rows under the bottom-right
    causal mask; shuffled table over a pool with 10% spare blocks and null block 0."""
    L = np.random.default_rng([seed, 70]).integers(1024, 32769, size=32).astype(np.int32)
    return prefill_case(seed, 32, 64, 8, 128, "bf16", cached=L - 4, new=4, max_blocks=256, null_block=True,
                        name="gqa_mtp_decode")


def mla_decode(seed: int = 0) -> Case:
    """MLA absorbed decode: B=64, 128 query heads, latent 512 + rope 64, every
    length 8192, table = a permutation of 4096 blocks, scale 1/sqrt(576)."""
    return decode_case(seed, 64, 128, 1, 512, "bf16", max_blocks=64,
                       seq_lens=np.full(64, 8192, dtype=np.int32), rope_dim=64,
                       scale=1.0 / math.sqrt(576.0), name="mla_decode")


def mla_mtp_decode(seed: int = 0) -> Case:
    """MLA absorbed multi-token decode: the mla_decode shapes (B=64, 128 heads,
    latent 512 + rope 64, 8192 keys per sequence) with 4 new query rows per
    sequence under the bottom-right causal mask (8188 cached + 4 new)."""
    return prefill_case(seed, 64, 128, 1, 512, "bf16", cached=8188, new=4, max_blocks=64, rope_dim=64,
                        scale=1.0 / math.sqrt(576.0), name="mla_mtp_decode")


def mla_chunked_prefill(seed: int = 0) -> Case:
    """MLA absorbed chunked prefill: B=4, 128 heads, latent 512 + rope 64,
    4096 cached tokens plus 512 new query rows per sequence, causal."""
    return prefill_case(seed, 4, 128, 1, 512, "bf16", cached=4096, new=512, max_blocks=36, rope_dim=64,
                        scale=1.0 / math.sqrt(576.0), name="mla_chunked_prefill")


def mla_latent_write(seed: int = 0) -> LatentCase:
    """Fused latent write of an MLA prefill: B=8 sequences x 4096 new tokens
    (32768 rows of latent 512 + rope 64) into a permuted pool of 259 blocks of
    128, rotate-half RoPE, eps 1e-6, normalised and rotated rows also returned,
    bf16."""
    return latent_case(seed, 8, "bf16", new=4096, name="mla_latent_write")


WORKLOADS = {
    "tiny_f32_decode": tiny_f32_decode,
    "mha_decode_7b": mha_decode_7b,
    "gqa_decode_70b": gqa_decode_70b,
    "gqa_decode_70b_window4096": lambda seed=0: gqa_decode_70b(seed, window=4096),
    "mha_decode_7b_int8": lambda seed=0: mha_decode_7b(seed, int8=True),
    "gqa_decode_70b_int8": lambda seed=0: gqa_decode_70b(seed, int8=True),
    "chunked_prefill": chunked_prefill,
    "gqa_mtp_decode": gqa_mtp_decode,
    "mla_decode": mla_decode,
    "mla_mtp_decode": mla_mtp_decode,
    "mla_chunked_prefill": mla_chunked_prefill,
    "mla_latent_write": mla_latent_write,
}
