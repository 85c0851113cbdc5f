"""Pins of the INT8 cache oracle (symmetric per-(token, head) quantization) against a worked
example, brute force over every code, closed-form bounds and exact special cases; and of the
float64 element type of the attention oracle against its float32 path.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import int8_cache as q8


def test_worked_row():
    # max |x| = 1: scale 1/127, codes = 127 x rounded half to even
    x = np.array([[1.0, -0.5, 0.25, 0.0, 0.75, -1.0, 0.5 / 127]], dtype=np.float32)
    codes, s = q8.quantize_rows(x, "f32")
    assert s[0] == np.float32(1.0) / np.float32(127.0)
    # -63.5 -> -64 and 0.5 -> 0: ties go to the even code
    assert codes[0].tolist() == [127, -64, 32, 0, 95, -127, 0]


def test_zero_row_and_extremes():
    codes, s = q8.quantize_rows(np.zeros((2, 16), dtype=np.float32), "f32")
    assert not codes.any() and not s.any()
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    codes, s = q8.quantize_rows(x, "f32")
    i = np.argmax(np.abs(x), axis=-1)
    assert np.all(np.abs(codes[np.arange(50), i]) == 127)
    assert np.all(np.sign(codes[np.arange(50), i]) == np.sign(x[np.arange(50), i]))
    assert np.abs(codes.astype(int)).max() <= 127


def test_codes_are_nearest_by_brute_force():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((40, 64)) * rng.uniform(1e-3, 50, (40, 1))).astype(np.float32)
    codes, s = q8.quantize_rows(x, "f32")
    grid = np.arange(-127, 128, dtype=np.float64)
    for r in range(x.shape[0]):
        cand = grid[None, :] * float(s[r])
        err = np.abs(x[r].astype(np.float64)[:, None] - cand)
        best = err.min(axis=1)
        mine = np.abs(x[r].astype(np.float64) - codes[r].astype(np.float64) * float(s[r]))
        # the code is a nearest grid point up to the float32 rounding of 127 / max (relative 2^-23)
        np.testing.assert_array_less(mine - best, 1e-6 * float(s[r]) * 127 + 1e-30)


def test_round_trip_bound_and_power_of_two_scaling():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((30, 128)).astype(np.float32)
    codes, s = q8.quantize_rows(x, "f32")
    err = np.abs(q8.dequantize(codes, s) - x.astype(np.float64))
    assert np.all(err <= 0.5 * s[:, None].astype(np.float64) * (1 + 1e-6))
    c2, s2 = q8.quantize_rows(x * np.float32(2.0 ** -9), "f32")
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, s * np.float32(2.0 ** -9))


def test_bf16_input_equals_its_float32_value():
    rng = np.random.default_rng(3)
    bits = workloads.bf16_bits(rng.standard_normal((9, 128)).astype(np.float32))
    c_b, s_b = q8.quantize_rows(bits, "bf16")
    c_f, s_f = q8.quantize_rows(workloads.bf16_to_f32(bits), "f32")
    np.testing.assert_array_equal(c_b, c_f)
    np.testing.assert_array_equal(s_b, s_f)


def test_dequantize_is_exact():
    codes = np.array([[127, -3, 1]], dtype=np.int8)
    s = np.array([np.float32(0.1)], dtype=np.float32)
    got = q8.dequantize(codes, s)
    for c, g in zip(codes[0], got[0]):
        assert Fraction(float(g)) == int(c) * Fraction(float(s[0]))


def test_cache_layout_and_row_writes():
    rng = np.random.default_rng(4)
    nb, bs, hkv, d = 3, 4, 2, 8
    cache = rng.standard_normal((nb, bs, hkv, d)).astype(np.float32)
    codes, scales = q8.quantize_cache(cache, "f32")
    assert codes.shape == (nb, bs, hkv, d) and scales.shape == (nb, hkv, bs)
    for n in range(nb):
        for o in range(bs):
            for h in range(hkv):
                c1, s1 = q8.quantize_rows(cache[n, o, h][None], "f32")
                np.testing.assert_array_equal(codes[n, o, h], c1[0])
                assert scales[n, h, o] == s1[0]
    rows = rng.standard_normal((3, hkv, d)).astype(np.float32)
    before_c, before_s = codes.copy(), scales.copy()
    q8.write_rows(codes, scales, [5, -1, 10], rows, "f32")
    c1, s1 = q8.quantize_rows(rows, "f32")
    np.testing.assert_array_equal(codes[1, 1], c1[0])
    np.testing.assert_array_equal(scales[1, :, 1], s1[0])
    np.testing.assert_array_equal(codes[2, 2], c1[2])
    np.testing.assert_array_equal(scales[2, :, 2], s1[2])
    touched = np.zeros((nb, bs), dtype=bool)
    touched[1, 1] = touched[2, 2] = True
    np.testing.assert_array_equal(codes[~touched], before_c[~touched])


def test_float64_attention_matches_float32_on_exact_values(orc):
    """When every value is exactly k * 2^-7 with some |k| = 127 per row, quantization is
    lossless, and attention over the float64 dequantized cache must equal attention over the
    float32 cache exactly: the float64 element type adds nothing but the type."""
    rng = np.random.default_rng(5)
    nb, bs, hkv, d, B, H = 4, 16, 2, 32, 2, 4
    k = rng.integers(-127, 128, (nb, bs, hkv, d)).astype(np.float32)
    k[..., 0] = 127
    v = rng.integers(-127, 128, (nb, bs, hkv, d)).astype(np.float32)
    v[..., 0] = -127
    k *= np.float32(2.0 ** -7)
    v *= np.float32(2.0 ** -7)
    ck, sk = q8.quantize_cache(k, "f32")
    cv, sv = q8.quantize_cache(v, "f32")
    kd, vd = q8.dequantize_cache(ck, sk), q8.dequantize_cache(cv, sv)
    np.testing.assert_array_equal(kd, k.astype(np.float64))
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    bt = np.arange(nb, dtype=np.int32).reshape(B, 2)
    sl = np.array([20, 32], dtype=np.int32)
    o32 = orc.paged_decode(q, k, v, bt, sl, 0.2)
    o64 = orc.paged_decode(q.astype(np.float64), kd, vd, bt, sl, 0.2)
    np.testing.assert_array_equal(o64, o32)
