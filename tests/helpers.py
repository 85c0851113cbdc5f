"""Test helpers: run a workloads.Case through the oracle, compare results.

Everything here is test infrastructure; expected values come only from the
oracle (or from the pages' printed numbers), never from the HIP library.
"""
from __future__ import annotations

import numpy as np

import workloads


def oracle_slots(orc, case) -> np.ndarray:
    """slot_mapping for the case's new tokens (-1 where a sequence has no token)."""
    pos = case.new_pos
    ok = pos >= 0
    slots = np.full(pos.shape, -1, dtype=np.int32)
    if ok.any():
        slots[ok] = orc.resolve_slots(case.block_table, case.block_size, case.num_blocks,
                                      case.new_batch_idx[ok], pos[ok])
    return slots


def oracle_write(orc, case, slots) -> None:
    """Write the case's new rows into its own caches (in place)."""
    orc.cache_write(case.k_cache, slots, case.new_k)
    if case.v_cache is not None:
        orc.cache_write(case.v_cache, slots, case.new_v)
    if case.k_rope_cache is not None:
        orc.cache_write(case.k_rope_cache, slots, case.new_k_rope)


def oracle_attend(orc, case, units=None, want_probs=False, nthreads=0):
    if case.kind == "decode":
        return orc.paged_decode(case.q, case.k_cache, case.v_cache_or_k, case.block_table,
                                case.seq_lens, case.scale, case.window, q_rope=case.q_rope,
                                k_rope_cache=case.k_rope_cache, units=units,
                                want_probs=want_probs, nthreads=nthreads)
    return orc.paged_prefill(case.q, case.k_cache, case.v_cache_or_k, case.block_table,
                             case.cu_seqlens_q, case.seq_lens, case.scale, case.window,
                             q_rope=case.q_rope, k_rope_cache=case.k_rope_cache, units=units,
                             want_probs=want_probs, nthreads=nthreads)


def int8_state(case):
    """The case's bf16 pools as int8 caches: (k_codes, k_scales, v_codes, v_scales).  With a
    null block, block 0 holds zero codes and NaN scales (it is never quantized)."""
    from oracle import int8_cache as q8

    out = []
    for pool in (case.k_cache, case.v_cache):
        src = pool
        if case.null_block:
            src = pool.copy()
            src[0] = 0
        c, sc = q8.quantize_cache(src, case.dtype)
        if case.null_block:
            c[0] = 0
            sc[0] = np.float32("nan")
        out += [c, sc]
    return tuple(out)


def oracle_write_int8(orc, case, state, slots) -> None:
    """Quantize the case's new rows into the int8 state (in place)."""
    from oracle import int8_cache as q8

    kc, ks, vc, vs = state
    q8.write_rows(kc, ks, slots, case.new_k, case.dtype)
    q8.write_rows(vc, vs, slots, case.new_v, case.dtype)


def oracle_attend_int8(orc, case, state, units=None, nthreads=0):
    """Decode attention over the dequantized int8 cache (float64)."""
    from oracle import int8_cache as q8

    kc, ks, vc, vs = state
    kd, vd = q8.dequantize_cache(kc, ks), q8.dequantize_cache(vc, vs)
    return orc.paged_decode(to_f64(case.q, case.dtype), kd, vd, case.block_table, case.seq_lens, case.scale,
                            case.window, units=units, nthreads=nthreads)


def oracle_run(orc, case, units=None, want_probs=False, inplace=False, nthreads=0):
    """resolve -> write -> attend on the CPU.  Returns (out, written_case, slots); for an int8
    case the second item is the int8 state (k_codes, k_scales, v_codes, v_scales) after the write."""
    if case.int8:
        assert case.kind == "decode" and not want_probs
        slots = oracle_slots(orc, case)
        state = int8_state(case)
        oracle_write_int8(orc, case, state, slots)
        return oracle_attend_int8(orc, case, state, units=units, nthreads=nthreads), state, slots
    c = case if inplace else case.copy_caches()
    slots = oracle_slots(orc, c)
    oracle_write(orc, c, slots)
    out = oracle_attend(orc, c, units=units, want_probs=want_probs, nthreads=nthreads)
    return out, c, slots


def round_like_output(ref: np.ndarray, out_dtype: str) -> np.ndarray:
    """The oracle's float64 result expressed in the output dtype (RNE), as float64."""
    if out_dtype == "bf16":
        return workloads.bf16_to_f32(workloads.bf16_bits(ref.astype(np.float32))).astype(np.float64)
    return ref.astype(np.float32).astype(np.float64)


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per output row (last axis): ||got - ref||_2 / ||ref||_2 (0 where both rows are 0)."""
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values or bfloat16 raw bits -> float64 (exact)."""
    return (a if dtype == "f32" else workloads.bf16_to_f32(a)).astype(np.float64)


def oracle_latent(orc, case, tokens=None):
    """Expected results of a workloads.LatentCase from the oracle: (slots, cache_nope,
    cache_rope, nope, rope), caches as float64 [slots, width] after the write, rows float64.
    tokens: optional index array restricting the write to those tokens (for sampling)."""
    from oracle import latent_write as lw

    slots = oracle_slots(orc, case)
    cn = to_f64(case.cache_nope, case.dtype).reshape(-1, 512)
    cr = to_f64(case.cache_rope, case.dtype).reshape(-1, 64)
    sel = slice(None) if tokens is None else tokens
    nope, rope = lw.latent_write(to_f64(case.latent[sel], case.dtype), to_f64(case.gamma, case.dtype),
                                 to_f64(case.cos[sel], case.dtype), to_f64(case.sin[sel], case.dtype),
                                 slots[sel], case.eps, cn, cr, case.layout)
    return slots, cn, cr, nope, rope
