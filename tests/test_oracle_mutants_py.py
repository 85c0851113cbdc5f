"""Plant plausible mistakes in copies of the Python oracles (the int8 cache and the fused
latent write) and check that the pins catch each.

Every mutant is a textual edit of oracle/int8_cache.py or oracle/latent_write.py,
executed as a fresh module.  The battery below restates a cross-section of the pins in
test_int8_oracle.py and test_latent_write_oracle.py -- worked values with ties, the
library 2-norm, closed forms, complex multiplication, layout and scatter invariants --
against that module.  The sources as they stand pass the whole battery; each mutant
must fail at least one check.  An edit that no longer matches the source fails the
test, so the list stays in step with the code.  CPU only.
"""
import os
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = {"int8": os.path.join(ROOT, "oracle", "int8_cache.py"),
       "latent": os.path.join(ROOT, "oracle", "latent_write.py")}

MUTANTS = {
    # int8 quantization
    "scale_over_128": ("int8", "scale[nz] = amax[nz] / one27", "scale[nz] = amax[nz] / np.float32(128.0)"),
    "round_half_away": ("int8", "np.rint(prod)", "np.trunc(prod + np.copysign(np.float32(0.5), prod))"),
    "truncate_codes": ("int8", "np.rint(prod)", "np.trunc(prod)"),
    "signed_max": ("int8", "np.max(np.abs(xf), axis=-1)", "np.max(xf, axis=-1)"),
    "scale_inverted": ("int8", "scale[nz] = amax[nz] / one27", "scale[nz] = one27 / amax[nz]"),
    "scales_not_transposed": ("int8", "np.ascontiguousarray(s.transpose(0, 2, 1))", "np.ascontiguousarray(s)"),
    "dequant_divides": ("int8", "codes.astype(np.float64) * scales", "codes.astype(np.float64) / scales"),
    "write_block_offset_swapped": ("int8", "blk, off = divmod(int(slot), bs)", "off, blk = divmod(int(slot), bs)"),
    # fused RMSNorm + RoPE + latent write
    "rms_without_eps": ("latent", "np.sqrt(ms + eps)", "np.sqrt(ms)"),
    "rms_sum_not_mean": ("latent", "np.mean(c * c, axis=-1, keepdims=True)", "np.sum(c * c, axis=-1, keepdims=True)"),
    "gamma_dropped": ("latent", " * np.asarray(gamma, dtype=np.float64)", ""),
    "rope_sign_flipped": ("latent", "np.where(second, 1.0, -1.0)", "np.where(second, -1.0, 1.0)"),
    "half_partner_adjacent": ("latent", "np.where(i < h, i + h, i - h)", "i ^ 1"),
    "sin_cos_swapped": ("latent", "x * cos + sign * x[..., j] * sin", "x * sin + sign * x[..., j] * cos"),
    "negative_slot_written": ("latent", "if s >= 0:", "if True:"),
    "rope_from_latent_head": ("latent", "rot = rope(latent[:, rank:], cos, sin, layout)",
                              "rot = rope(latent[:, :rope_dim], cos, sin, layout)"),
}


def _module(kind, edit=None):
    src = open(SRC[kind]).read()
    if edit is not None:
        old, new = edit
        assert src.count(old) == 1, f"mutant edit no longer matches {SRC[kind]}: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType(f"mutant_{kind}")
    exec(compile(src, SRC[kind], "exec"), mod.__dict__)
    return mod


def _f32_bits_as_bf16(x):
    """float32 values that are exact in bfloat16 -> their bf16 bit patterns."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _int8_battery(m):
    failed = []

    def check(name, fn):
        try:
            ok = bool(fn())
        except Exception:  # a crash is a caught mistake too
            ok = False
        if not ok:
            failed.append(name)

    # max |x| = 127 gives scale 1, so the codes are x rounded half to even
    row = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.0]], dtype=np.float32)
    check("worked_ties", lambda: (lambda q, s: s[0] == 1.0 and q[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 3])(
        *m.quantize_rows(row, "f32")))
    neg = np.array([[-127.0, 1.0, 2.0, 0.0]], dtype=np.float32)  # the largest magnitude is negative
    check("negative_max", lambda: (lambda q, s: s[0] == 1.0 and q[0].tolist() == [-127, 1, 2, 0])(
        *m.quantize_rows(neg, "f32")))
    check("zero_row", lambda: (lambda q, s: s[0] == 0.0 and not q.any())(
        *m.quantize_rows(np.zeros((1, 16), dtype=np.float32), "f32")))
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    cache = _f32_bits_as_bf16(rng.standard_normal((2, 4, 3, 8)).astype(np.float32))
    try:  # set-up that a mutant may break: a raised error counts as caught
        q, s = m.quantize_rows(x, "f32")
        codes, scales = m.quantize_cache(cache, "bf16")
    except Exception:
        return failed + ["set_up"]
    check("half_step_round_trip", lambda: np.all(np.abs(m.dequantize(q, s) - x) <= s[:, None] * 0.5000001))
    check("scale_layout", lambda: scales.shape == (2, 3, 4) and all(
        scales[b, h, o] == m.quantize_rows(cache[b, o, h], "bf16")[1] for b in range(2) for h in range(3)
        for o in range(4)))
    rows = _f32_bits_as_bf16(rng.standard_normal((1, 3, 8)).astype(np.float32))

    def write_slot():
        c2, s2 = codes.copy(), scales.copy()
        m.write_rows(c2, s2, [6], rows, "bf16")  # slot 6 = block 1, offset 2 at block_size 4
        qr, sr = m.quantize_rows(rows[0], "bf16")
        return (np.array_equal(c2[1, 2], qr) and np.array_equal(s2[1, :, 2], sr)
                and np.array_equal(np.delete(c2.reshape(8, 3, 8), 6, axis=0),
                                   np.delete(codes.reshape(8, 3, 8), 6, axis=0)))

    check("write_slot", write_slot)
    return failed


def _latent_battery(m):
    failed = []

    def check(name, fn):
        try:
            ok = bool(fn())
        except Exception:
            ok = False
        if not ok:
            failed.append(name)

    rng = np.random.default_rng(1)
    c = rng.standard_normal((3, 512))
    g = 1.0 + 0.25 * rng.standard_normal(512)
    ref = c / (np.linalg.norm(c, axis=-1, keepdims=True) / np.sqrt(512)) * g
    check("rms_library_norm", lambda: np.allclose(m.rms_norm(c, g, 0.0), ref, rtol=1e-12, atol=0))
    check("rms_eps_closed_form", lambda: np.allclose(m.rms_norm(np.full((1, 8), 3.0), np.ones(8), 16.0), 0.6,
                                                     rtol=1e-12))
    x = rng.standard_normal((2, 64))
    th = rng.uniform(-np.pi, np.pi, (2, 32))

    def complex_half():
        z = (x[:, :32] + 1j * x[:, 32:]) * np.exp(1j * th)
        cos, sin = np.cos(np.concatenate([th, th], -1)), np.sin(np.concatenate([th, th], -1))
        return np.allclose(m.rope(x, cos, sin, m.HALF), np.concatenate([z.real, z.imag], -1), rtol=0, atol=1e-12)

    def complex_interleaved():
        z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * th)
        cos, sin = np.cos(np.repeat(th, 2, -1)), np.sin(np.repeat(th, 2, -1))
        out = np.empty_like(x)
        out[:, 0::2], out[:, 1::2] = z.real, z.imag
        return np.allclose(m.rope(x, cos, sin, m.INTERLEAVED), out, rtol=0, atol=1e-12)

    check("rope_half_complex", complex_half)
    check("rope_interleaved_complex", complex_interleaved)
    lat = rng.standard_normal((3, 576))
    cos = np.cos(np.tile(np.linspace(0, 1, 64), (3, 1)))
    sin = np.sin(np.tile(np.linspace(0, 1, 64), (3, 1)))
    cn, cr = np.full((6, 512), 7.0), np.full((6, 64), 7.0)
    try:
        nope, rot = m.latent_write(lat, g, cos, sin, [4, -1, 0], 1e-6, cn, cr, m.HALF)
    except Exception:
        return failed + ["latent_write_runs"]
    check("scatter_and_skip", lambda: np.array_equal(cn[4], nope[0]) and np.array_equal(cn[0], nope[2])
          and np.all(cn[[1, 2, 3, 5]] == 7.0) and np.all(cr[[1, 2, 3, 5]] == 7.0))
    check("rope_part_of_row", lambda: np.allclose(rot, m.rope(lat[:, 512:], cos, sin, m.HALF), rtol=0, atol=0))
    return failed


BATTERY = {"int8": _int8_battery, "latent": _latent_battery}


@pytest.mark.parametrize("kind", ["int8", "latent"])
def test_sources_pass_the_battery(kind):
    assert BATTERY[kind](_module(kind)) == []


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    kind, old, new = MUTANTS[name]
    failed = BATTERY[kind](_module(kind, (old, new)))
    assert failed, f"mutant {name} passes every pin"
