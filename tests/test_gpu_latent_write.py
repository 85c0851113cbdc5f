"""GPU parity of the fused latent write (kv_rmsnorm_rope_cache: RMSNorm + RoPE + paged
write of the MLA latent) through the C ABI against the fp64 oracle.

Bars, per element, derived from the arithmetic (fp32 inside the kernel, u = 2^-24; the
final rounding to the output type adds at most half an ulp of the result, hulp below:
2^(e-8) for a bf16 result in [2^e, 2^(e+1)), at most 2^-24 |exact| for f32):
  latent part  nope = c * (1 / sqrt(mean(c^2) + eps)) * gamma: a 512-term fp32 sum of
               squares, a square root, a division and two products stay within ~16 u of
               the exact value relative to it, so
                 bf16: |got - exact| <= hulp(exact) + 2^-19 |exact|
                 f32:  |got - exact| <= 2^-18 |exact|
  rotary part  rope = x cos -/+ p sin: two products and a sum, 2 u of |x cos| + |p sin|,
                 bf16: |got - exact| <= hulp(exact) + 2^-21 (|x cos| + |p sin|)
                 f32:  |got - exact| <= 2^-23 |exact| + 2^-21 (|x cos| + |p sin|)
Cache rows no token writes stay bit-identical; the returned rows equal the cache rows
bit for bit."""
import numpy as np
import pytest

import workloads
from helpers import oracle_latent, to_f64

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_80_amd as pkv
    pkv.load()


from gpu_util import bf16_ulp, dev, host  # noqa: E402


def _run(case, outputs=True):
    import paged_kv_cache_80_amd as pkv

    cache = pkv.PagedKVCache(dev(case.cache_nope), None, dev(case.cache_rope))
    slots = pkv.pkv_resolve_slots(dev(case.block_table), case.block_size, dev(case.new_batch_idx),
                                  dev(case.new_pos))
    tdt = cache.k_cache.dtype
    kn = torch.empty((case.T, 512), dtype=tdt, device="cuda") if outputs else None
    kr = torch.empty((case.T, 64), dtype=tdt, device="cuda") if outputs else None
    pkv.kv_rmsnorm_rope_cache(dev(case.latent), dev(case.gamma), dev(case.cos), dev(case.sin), slots, case.eps,
                              cache, rope_layout=case.layout, k_nope_out=kn, k_rope_out=kr)
    torch.cuda.synchronize()
    return cache, slots, kn, kr


def _rope_scale(case, tokens):
    """|x cos| + |p sin| per rotary element (the fp32 error scale of the rotation)."""
    from oracle import latent_write as lw

    x = to_f64(case.latent[tokens, 512:], case.dtype)
    c, s = to_f64(case.cos[tokens], case.dtype), to_f64(case.sin[tokens], case.dtype)
    j, _ = lw.partner(64, case.layout)
    return np.abs(x * c) + np.abs(x[:, j] * s)


def _check_rows(got_bits, exact, dtype, kind, scale=None, what=""):
    g = to_f64(got_bits, dtype)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    if dtype == "bf16":
        hulp = 0.5 * bf16_ulp(exact)
        bound = hulp + (2.0 ** -19 * np.abs(exact) if kind == "nope" else 2.0 ** -21 * scale)
    elif kind == "nope":
        bound = 2.0 ** -18 * np.abs(exact)
    else:
        bound = 2.0 ** -23 * np.abs(exact) + 2.0 ** -21 * scale
    over = np.abs(g - exact) > bound
    if over.any():
        r, e = np.argwhere(over)[0]
        raise AssertionError(f"{what}: {int(over.sum())} elements out of bound; first row {r} elem {e}: "
                             f"got {g[r, e]!r}, exact {exact[r, e]!r}, bound {bound[r, e]:.3e}")


def _verify(orc, case, outputs=True):
    cache, slots, kn, kr = _run(case, outputs)
    want_slots, cn, cr, nope, rope = oracle_latent(orc, case)
    np.testing.assert_array_equal(host(slots), want_slots)
    toks = np.arange(case.T)
    rs = _rope_scale(case, toks)
    got_cn = host(cache.k_cache).reshape(-1, 512)
    got_cr = host(cache.k_rope_cache).reshape(-1, 64)
    written = np.zeros(got_cn.shape[0], dtype=bool)
    live = want_slots >= 0
    written[want_slots[live]] = True
    # rows no token writes: bit-identical
    np.testing.assert_array_equal(got_cn[~written], case.cache_nope.reshape(-1, 512)[~written])
    np.testing.assert_array_equal(got_cr[~written], case.cache_rope.reshape(-1, 64)[~written])
    _check_rows(got_cn[want_slots[live]], nope[live], case.dtype, "nope", what="cache latent rows")
    _check_rows(got_cr[want_slots[live]], rope[live], case.dtype, "rope", rs[live], what="cache rotary rows")
    if outputs:
        hn, hr = host(kn), host(kr)
        _check_rows(hn, nope, case.dtype, "nope", what="returned latent rows")
        _check_rows(hr, rope, case.dtype, "rope", rs, what="returned rotary rows")
        np.testing.assert_array_equal(hn[live], got_cn[want_slots[live]])
        np.testing.assert_array_equal(hr[live], got_cr[want_slots[live]])


MATRIX = [
    # (name, B, new, cached, block_size, pad_every)
    ("one token", 1, 1, 0, 16, 0),
    ("decode batch", 64, 1, [37 * i for i in range(64)], 128, 0),
    ("odd count spanning waves", 3, [5, 0, 8], [3, 10, 200], 16, 0),
    ("ragged prefill with padding tokens", 5, [257, 1, 64, 300, 13], [0, 5, 128, 33, 1000], 64, 7),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", [0, 1], ids=["half", "interleaved"])
@pytest.mark.parametrize("name,B,new,cached,bs,pad", MATRIX, ids=[m[0] for m in MATRIX])
def test_latent_write_matches_oracle(orc, dtype, layout, name, B, new, cached, bs, pad):
    case = workloads.latent_case(11, B, dtype, new=new, cached=cached, block_size=bs, layout=layout,
                                 pad_every=pad)
    print(f"latent write {name} {dtype} layout={layout} T={case.T}", flush=True)
    _verify(orc, case)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_latent_write_without_returned_rows(orc, dtype):
    case = workloads.latent_case(12, 4, dtype, new=[100, 3, 0, 77], cached=[0, 9, 4, 500], block_size=32)
    _verify(orc, case, outputs=False)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5, 1e4])
def test_latent_write_eps_and_zero_rows(orc, eps):
    case = workloads.latent_case(13, 2, "bf16", new=[40, 25], cached=[0, 60], block_size=16, eps=eps)
    if eps > 0:  # a zero latent row normalises to zero once eps > 0
        case.latent[::6, :512] = 0
    _verify(orc, case)


def test_latent_write_full_size(orc):
    """The full workload: 8 sequences x 4096 new tokens, every row checked."""
    case = workloads.mla_latent_write(0)
    print(f"latent write full size T={case.T}", flush=True)
    _verify(orc, case)


def test_latent_write_rejects_bad_arguments():
    import paged_kv_cache_80_amd as pkv

    case = workloads.latent_case(14, 1, "bf16", new=8, block_size=16)
    cn, cr = dev(case.cache_nope), dev(case.cache_rope)
    cache = pkv.PagedKVCache(cn, None, cr)
    lat, g, c, s = dev(case.latent), dev(case.gamma), dev(case.cos), dev(case.sin)
    slots = torch.zeros(case.T, dtype=torch.int32, device="cuda")
    before = host(cn).copy()
    out = torch.empty((case.T, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pkv.PkvError, match="eps"):
        pkv.kv_rmsnorm_rope_cache(lat, g, c, s, slots, float("nan"), cache)
    with pytest.raises(pkv.PkvError, match="eps"):
        pkv.kv_rmsnorm_rope_cache(lat, g, c, s, slots, -1.0, cache)
    with pytest.raises(pkv.PkvError, match="rope_layout"):
        pkv.kv_rmsnorm_rope_cache(lat, g, c, s, slots, 1e-6, cache, rope_layout=2)
    with pytest.raises(pkv.PkvError, match="together"):
        pkv.kv_rmsnorm_rope_cache(lat, g, c, s, slots, 1e-6, cache, k_nope_out=out)
    plain = pkv.PagedKVCache(torch.zeros((4, 16, 1, 512), dtype=torch.bfloat16, device="cuda"),
                             torch.zeros((4, 16, 1, 512), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(pkv.PkvError, match="MLA cache"):
        pkv.kv_rmsnorm_rope_cache(lat, g, c, s, slots, 1e-6, plain)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(cn), before)
    # zero tokens: nothing launched, nothing changed
    z = torch.zeros((0, 576), dtype=torch.bfloat16, device="cuda")
    z64 = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    pkv.kv_rmsnorm_rope_cache(z, g, z64, z64, slots[:0], 1e-6, cache)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(cn), before)
