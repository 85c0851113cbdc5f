"""Pins of the latent-write oracle (RMSNorm + RoPE + paged cache write) against what the
mathematics fixes on its own: library norms, complex multiplication, closed forms and the
rotation group's invariants.  CPU only."""
import numpy as np
import pytest

from oracle import latent_write as lw


def _angles(positions, rope_dim, base=10000.0):
    """Standard RoPE angles: position * base^(-2k/rope_dim) for pair k."""
    k = np.arange(rope_dim // 2)
    return np.outer(np.asarray(positions, dtype=np.float64), base ** (-2.0 * k / rope_dim))


def _cos_sin(theta, layout):
    """Per-element cos/sin rows for the two pair layouts."""
    if layout == lw.HALF:
        th = np.concatenate([theta, theta], axis=-1)
    else:
        th = np.repeat(theta, 2, axis=-1)
    return np.cos(th), np.sin(th)


def test_rmsnorm_is_the_vector_scaled_to_rms_one():
    rng = np.random.default_rng(0)
    c = rng.standard_normal((7, 512))
    out = lw.rms_norm(c, np.ones(512), 0.0)
    want = c * np.sqrt(512) / np.linalg.norm(c, axis=-1, keepdims=True)
    np.testing.assert_allclose(out, want, rtol=1e-13)
    np.testing.assert_allclose(np.mean(out * out, axis=-1), 1.0, rtol=1e-13)


def test_rmsnorm_scale_invariant_and_gamma_elementwise():
    rng = np.random.default_rng(1)
    c = rng.standard_normal((3, 64))
    g = rng.standard_normal(64)
    base = lw.rms_norm(c, np.ones(64), 0.0)
    np.testing.assert_allclose(lw.rms_norm(37.5 * c, np.ones(64), 0.0), base, rtol=1e-13)
    np.testing.assert_allclose(lw.rms_norm(c, g, 0.0), base * g, rtol=1e-13)


def test_rmsnorm_eps_closed_form():
    # a constant row a with eps: a / sqrt(a^2 + eps); 3 / sqrt(9 + 16) = 0.6
    out = lw.rms_norm(np.full((1, 8), 3.0), np.ones(8), 16.0)
    np.testing.assert_allclose(out, 0.6, rtol=1e-15)
    # the zero row stays zero for any eps > 0
    assert not np.any(lw.rms_norm(np.zeros((1, 8)), np.ones(8), 1e-6))


@pytest.mark.parametrize("layout", [lw.HALF, lw.INTERLEAVED])
def test_rope_is_complex_multiplication(layout):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    theta = rng.uniform(-7, 7, (5, 32))
    cos, sin = _cos_sin(theta, layout)
    out = lw.rope(x, cos, sin, layout)
    if layout == lw.HALF:
        z, zo = x[:, :32] + 1j * x[:, 32:], out[:, :32] + 1j * out[:, 32:]
    else:
        z, zo = x[:, 0::2] + 1j * x[:, 1::2], out[:, 0::2] + 1j * out[:, 1::2]
    np.testing.assert_allclose(zo, z * np.exp(1j * theta), rtol=1e-13, atol=1e-13)


def test_rope_quarter_turn_worked_pair():
    # the pair (1, 0) turned by a quarter turn is (0, 1); (0, 1) becomes (-1, 0)
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    cos, sin = np.zeros((2, 2)), np.ones((2, 2))
    np.testing.assert_allclose(lw.rope(x, cos, sin, lw.INTERLEAVED), [[0.0, 1.0], [-1.0, 0.0]], atol=1e-15)
    np.testing.assert_allclose(lw.rope(x, cos, sin, lw.HALF), [[0.0, 1.0], [-1.0, 0.0]], atol=1e-15)


@pytest.mark.parametrize("layout", [lw.HALF, lw.INTERLEAVED])
def test_rope_identity_at_position_zero_and_norm_preserved(layout):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 64))
    cos, sin = _cos_sin(_angles([0, 0, 0, 0], 64), layout)
    np.testing.assert_array_equal(lw.rope(x, cos, sin, layout), x)
    cos, sin = _cos_sin(_angles([5, 99, 1234, 65535], 64), layout)
    np.testing.assert_allclose(np.linalg.norm(lw.rope(x, cos, sin, layout), axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-13)


@pytest.mark.parametrize("layout", [lw.HALF, lw.INTERLEAVED])
def test_rope_scores_depend_on_relative_position_only(layout):
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)

    def rot(v, p):
        c, s = _cos_sin(_angles([p], 64), layout)
        return lw.rope(v[None], c, s, layout)[0]

    ref = rot(q, 100) @ rot(k, 93)
    for m, n in [(7, 0), (1007, 1000), (50000, 49993)]:
        np.testing.assert_allclose(rot(q, m) @ rot(k, n), ref, rtol=1e-9)
    # composition: turning by m then by n is turning by m + n
    np.testing.assert_allclose(rot(rot(q, 300), 45), rot(q, 345), rtol=1e-11, atol=1e-12)


def test_write_lands_rows_at_slots_and_skips_negative_slots():
    rng = np.random.default_rng(5)
    T, rank, rd, nslots = 6, 512, 64, 40
    latent = rng.standard_normal((T, rank + rd))
    gamma = rng.standard_normal(rank)
    cos, sin = _cos_sin(_angles(rng.integers(0, 4096, T), rd), lw.HALF)
    slots = np.array([17, -1, 3, 39, -5, 0])
    cn, cr = np.full((nslots, rank), 7.0), np.full((nslots, rd), 7.0)
    nope, rot = lw.latent_write(latent, gamma, cos, sin, slots, 1e-6, cn, cr)
    assert nope.shape == (T, rank) and rot.shape == (T, rd)
    for t, s in enumerate(slots):
        if s >= 0:
            np.testing.assert_array_equal(cn[s], nope[t])
            np.testing.assert_array_equal(cr[s], rot[t])
    untouched = np.setdiff1d(np.arange(nslots), slots[slots >= 0])
    assert np.all(cn[untouched] == 7.0) and np.all(cr[untouched] == 7.0)
    # the split: the latent part only feeds RMSNorm, the rotary part only RoPE
    np.testing.assert_allclose(nope, lw.rms_norm(latent[:, :rank], gamma, 1e-6), rtol=0)
    lat2 = latent.copy()
    lat2[:, rank:] += 1.0
    n2, r2 = lw.latent_write(lat2, gamma, cos, sin, slots, 1e-6, cn.copy(), cr.copy())
    np.testing.assert_array_equal(n2, nope)
    assert not np.allclose(r2, rot)
