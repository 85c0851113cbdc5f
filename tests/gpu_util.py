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


class DeviceCase:
    """The device copy of a case's tensors."""

    def __init__(self, case):
        self.case = case
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


def assert_rows_close(got: torch.Tensor, ref: np.ndarray, tol: float, rows=None):
    """Per output row: ||got - round(ref)|| / ||round(ref)|| <= tol, where round() expresses the
    oracle's float64 result in the output dtype (bf16 by round-to-nearest-even)."""
    g = as_f64(got)
    if rows is not None:
        g, ref = g.reshape(-1, g.shape[-1])[rows], ref.reshape(-1, ref.shape[-1])[rows]
    assert np.all(np.isfinite(g)), "non-finite output"
    err = row_rel_err(g, round_like_output(ref, out_dtype_name(got)))
    worst = float(err.max(initial=0.0))
    assert worst <= tol, f"max per-row relative error {worst:.3e} > {tol:.1e}"
    return worst
