"""GPU-side helpers for the parity tests: upload a workloads.Case, run the hot path
through the C ABI (resolve -> write -> attend), download results."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_80_amd as pkv
from helpers import round_like_output, row_rel_err


def dev(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def int8_device_cache(case) -> "pkv.PagedKVCache":
    """An int8 cache holding the case's bf16 pools, quantized on the GPU by kv_cache_write
    (every slot; with a null block, block 0 keeps zero codes and gets NaN scales)."""
    nb, bs, hkv, d = case.k_cache.shape
    cache = pkv.PagedKVCache(torch.zeros((nb, bs, hkv, d), dtype=torch.int8, device="cuda"),
                             torch.zeros((nb, bs, hkv, d), dtype=torch.int8, device="cuda"), None,
                             torch.zeros((nb, hkv, bs), dtype=torch.float32, device="cuda"),
                             torch.zeros((nb, hkv, bs), dtype=torch.float32, device="cuda"))
    slots = torch.arange(nb * bs, dtype=torch.int32, device="cuda")
    if case.null_block:
        slots[:bs] = -1
    pk, pv = dev(case.k_cache), dev(case.v_cache)
    pkv.kv_cache_write(slots, pk.view(nb * bs, hkv, d), pv.view(nb * bs, hkv, d), cache)
    if case.null_block:
        cache.k_scale[0] = float("nan")
        cache.v_scale[0] = float("nan")
    torch.cuda.synchronize()
    return cache


class DeviceCase:
    """The device copy of a case's tensors."""

    def __init__(self, case):
        self.case = case
        if case.int8:
            self.cache = int8_device_cache(case)
        else:
            self.cache = pkv.PagedKVCache(dev(case.k_cache), dev(case.v_cache), dev(case.k_rope_cache))
        self.block_table = dev(case.block_table)
        self.seq_lens = dev(case.seq_lens)
        self.q = dev(case.q)
        self.q_rope = dev(case.q_rope)
        self.new_k = dev(case.new_k)
        self.new_v = dev(case.new_v)
        self.new_k_rope = dev(case.new_k_rope)
        self.new_batch_idx = dev(case.new_batch_idx)
        self.new_pos = dev(case.new_pos)
        self.cu_seqlens_q = dev(case.cu_seqlens_q)

    def resolve(self):
        return pkv.pkv_resolve_slots(self.block_table, self.case.block_size, self.new_batch_idx,
                                     self.new_pos)

    def write(self, slots):
        pkv.kv_cache_write(slots, self.new_k, self.new_v, self.cache, k_rope=self.new_k_rope)

    def attend(self, out_dtype=None, split_tokens=0):
        c = self.case
        if c.kind == "decode":
            return pkv.paged_attn_decode(self.q, self.cache, self.block_table, self.seq_lens, c.scale,
                                         c.window, q_rope=self.q_rope, out_dtype=out_dtype,
                                         split_tokens=split_tokens)
        max_q = int(np.diff(c.cu_seqlens_q).max(initial=0))
        return pkv.paged_attn_prefill(self.q, self.cache, self.block_table, self.cu_seqlens_q,
                                      self.seq_lens, max_q, c.scale, c.window, q_rope=self.q_rope,
                                      out_dtype=out_dtype)

    def run(self, out_dtype=None, split_tokens=0):
        slots = self.resolve()
        self.write(slots)
        out = self.attend(out_dtype, split_tokens)
        torch.cuda.synchronize()
        return out, slots


def out_dtype_name(t: torch.Tensor) -> str:
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits), for x != 0."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 7), 0.0)


def assert_rows_close(got: torch.Tensor, ref: np.ndarray, tol: float, rows=None, slack: float = 1e-4):
    """Compare an attention output with the oracle's float64 result.

    fp32 output: per row, ||got - ref||_2 / ||ref||_2 <= tol (accumulation error only).
    bf16 output: (a) every element is a faithful rounding of the exact value -- within one
    bf16 ulp of it -- up to an absolute slack of `slack` x the row's largest |ref| (fp32
    cancellation in near-zero elements); (b) over all compared rows,
    ||got - bf16(ref)||_F / ||bf16(ref)||_F <= tol.  A per-row norm of the bf16 output cannot
    carry the bound: one legitimate 1-ulp rounding flip of a row's largest element already
    costs up to ~2e-3 of a 128-element row.  Returns the worst per-row relative error."""
    g = as_f64(got)
    if rows is not None:
        g, ref = g.reshape(-1, g.shape[-1])[rows], ref.reshape(-1, ref.shape[-1])[rows]
    g = g.reshape(-1, g.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(g)), "non-finite output"
    if out_dtype_name(got) == "f32":
        err = row_rel_err(g, ref)
        worst = float(err.max(initial=0.0))
        assert worst <= tol, f"max per-row relative error {worst:.3e} > {tol:.1e}"
        return worst
    rmax = np.abs(ref).max(axis=-1, keepdims=True)
    bound = bf16_ulp(ref) + slack * rmax
    over = np.abs(g - ref) > bound
    if over.any():
        r, e = np.argwhere(over)[0]
        raise AssertionError(f"{int(over.sum())} elements are not faithful roundings; first at row {r} "
                             f"elem {e}: got {g[r, e]!r}, exact {ref[r, e]!r}, bound {bound[r, e]:.3e}")
    rr = round_like_output(ref, "bf16")
    total = float(np.linalg.norm(g - rr) / max(np.linalg.norm(rr), 1e-300))
    assert total <= tol, f"aggregate relative error {total:.3e} > {tol:.1e}"
    return float(row_rel_err(g, rr).max(initial=0.0))
