"""GPU parity of the INT8 paged cache through the C ABI: the quantizing write against the
oracle's float32 decisions (codes and scales bit for bit), and decode over int8 codes
against the float64 oracle attention over the dequantized cache.

Bars: codes and scales bit-exact (the oracle takes every decision in float32, as the
kernel does); outputs as for the bf16 decode (gpu_util.assert_rows_close): bf16 outputs
faithful per element and 2e-3 aggregate, fp32 outputs 1e-4 per row.  The kernel computes
the same dot products on exact bf16 images of the codes and applies the per-key scales
in fp32, so quantization adds no error beyond the oracle's."""
import numpy as np
import pytest

import workloads
from helpers import int8_state, oracle_run, oracle_slots, oracle_write_int8

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3
ACC_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_80_amd as pkv
    pkv.load()


from gpu_util import DeviceCase, assert_rows_close, dev, host, int8_device_cache  # noqa: E402


def _codes_scales(cache):
    return host(cache.k_cache), host(cache.k_scale), host(cache.v_cache), host(cache.v_scale)


def _assert_state_equal(got, want, what):
    for g, w, name in zip(got, want, ("k codes", "k scales", "v codes", "v scales")):
        if g.dtype == np.float32:
            same = (g.view(np.uint32) == w.view(np.uint32)) | (np.isnan(g) & np.isnan(w))
            assert same.all(), f"{what}: {name} differ at {np.argwhere(~same)[:3].tolist()}"
        else:
            assert np.array_equal(g, w), f"{what}: {name} differ at {np.argwhere(g != w)[:3].tolist()}"


@pytest.mark.parametrize("bs,hkv", [(16, 1), (32, 8), (128, 32)])
def test_quantized_write_bit_exact(orc, bs, hkv):
    case = workloads.decode_case(70 + bs, 6, hkv, hkv, 128, "bf16", block_size=bs, max_blocks=5,
                                 len_range=(0, 5 * bs), int8=True)
    # rows that probe the decisions: all zero, one nonzero, exact ties (x * 127 / max = k + 1/2),
    # huge and tiny magnitudes
    nk = case.new_k.reshape(-1, 128)
    f = workloads.bf16_to_f32(nk)
    f[0] = 0
    f[1] = 0
    f[1, 7] = -3.5
    f[2] = np.float32(0.5) / np.float32(127.0) * np.arange(-64, 64, dtype=np.float32)
    f[2, 0] = 1.0
    f[3] *= np.float32(1e30)
    f[4] *= np.float32(1e-30)
    case.new_k = workloads.bf16_bits(f).reshape(case.new_k.shape)
    d = DeviceCase(case)
    want = int8_state(case)
    _assert_state_equal(_codes_scales(d.cache), want, "quantized pool")
    slots = d.resolve()
    d.write(slots)
    torch.cuda.synchronize()
    ref_slots = oracle_slots(orc, case)
    np.testing.assert_array_equal(host(slots), ref_slots)
    oracle_write_int8(orc, case, want, ref_slots)
    _assert_state_equal(_codes_scales(d.cache), want, "after the write")


INT8_LAYOUTS = [
    # name, B, H, Hkv, bs, max_blocks, seq_lens or len_range, window
    ("one long sequence", 1, 8, 1, 128, 64, [8192], 0),
    ("fewer tiles than groups", 3, 8, 2, 16, 4, [5, 40, 33], 0),
    ("GQA 8 with ragged lengths", 9, 64, 8, 128, 20, (1, 2560), 0),
    ("MHA 32 heads", 6, 32, 32, 64, 10, (1, 640), 0),
    ("group of 16", 5, 32, 2, 32, 12, (1, 384), 0),
    ("window with 16-token blocks", 7, 16, 4, 16, 200, (1, 3200), 100),
    ("window over 128-token blocks", 5, 8, 1, 128, 40, (1, 5000), 1000),
    ("batch past the in-LDS column prefix", 2100, 4, 2, 16, 4, (0, 64), 0),
    ("lengths on tile and block edges", 8, 16, 8, 64, 8, [32, 33, 63, 64, 65, 127, 128, 512], 0),
]


@pytest.mark.parametrize("layout", INT8_LAYOUTS, ids=[x[0] for x in INT8_LAYOUTS])
@pytest.mark.parametrize("split", [0, 2])
def test_int8_decode_layouts(orc, layout, split):
    name, B, H, Hkv, bs, mb, lens, w = layout
    kw = {"seq_lens": np.array(lens, dtype=np.int32)} if isinstance(lens, list) else {"len_range": lens}
    case = workloads.decode_case(B * 5 + Hkv + split, B, H, Hkv, 128, "bf16", block_size=bs, max_blocks=mb,
                                 window=w, null_block=True, int8=True, **kw)
    print(f"int8 decode {name} split={split}", flush=True)
    ref, state, slots_ref = oracle_run(orc, case)
    d = DeviceCase(case)
    out, slots = d.run(out_dtype=torch.float32, split_tokens=split * bs)
    np.testing.assert_array_equal(host(slots), slots_ref)
    _assert_state_equal(_codes_scales(d.cache), state, "cache after the write")
    assert_rows_close(out, ref, ACC_TOL)
    out = d.attend(split_tokens=split * bs)
    torch.cuda.synchronize()
    assert_rows_close(out, ref, BF16_TOL)


def _sampled_units(case, n, seed=0):
    rng = np.random.default_rng(seed)
    rows = case.B * case.H
    return np.sort(rng.choice(rows, size=min(n, rows), replace=False)).astype(np.int32)


@pytest.mark.parametrize("name", ["mha_decode_7b_int8", "gqa_decode_70b_int8"])
def test_int8_full_size(orc, name):
    case = workloads.WORKLOADS[name](0)
    print(f"int8 full size {name}", flush=True)
    d = DeviceCase(case)
    out, slots = d.run()
    units = _sampled_units(case, 192)
    ref, state, slots_ref = oracle_run(orc, case, units=units)
    np.testing.assert_array_equal(host(slots), slots_ref)
    # the rows written this step, bit for bit
    live = slots_ref[slots_ref >= 0]
    kc, ks, vc, vs = state
    bs = case.block_size
    gk, gv = host(d.cache.k_cache).reshape(-1, case.Hkv, 128), host(d.cache.v_cache).reshape(-1, case.Hkv, 128)
    assert np.array_equal(gk[live], kc.reshape(-1, case.Hkv, 128)[live])
    assert np.array_equal(gv[live], vc.reshape(-1, case.Hkv, 128)[live])
    gks = host(d.cache.k_scale)
    for sl in live[:64]:
        assert np.array_equal(gks[sl // bs, :, sl % bs].view(np.uint32), ks[sl // bs, :, sl % bs].view(np.uint32))
    assert_rows_close(out, ref, BF16_TOL, rows=units)
    out32 = d.attend(out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_rows_close(out32, ref, ACC_TOL, rows=units)


def test_int8_rejections():
    import paged_kv_cache_80_amd as pkv

    case = workloads.decode_case(90, 2, 64, 2, 128, "bf16", block_size=32, max_blocks=4, len_range=(1, 128),
                                 int8=True)
    d = DeviceCase(case)
    with pytest.raises(pkv.PkvError, match="groups of at most 16"):  # G = 32
        pkv.paged_attn_decode(d.q, d.cache, d.block_table, d.seq_lens, case.scale)
    cu = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError, match="prefill does not read int8"):
        pkv.paged_attn_prefill(d.q, d.cache, d.block_table, cu, d.seq_lens, 1, case.scale)
    no_scale = pkv.PagedKVCache(d.cache.k_cache, d.cache.v_cache, None, None, d.cache.v_scale)
    with pytest.raises(pkv.PkvError, match="k_scale"):
        pkv.paged_attn_decode(d.q[:, :2].contiguous(), no_scale, d.block_table, d.seq_lens, case.scale)
    with pytest.raises(TypeError):
        pkv.paged_attn_decode(d.q.float(), d.cache, d.block_table, d.seq_lens, case.scale)
    nb, bs = case.k_cache.shape[:2]
    wide = pkv.PagedKVCache(torch.zeros((nb, bs, 2, 64), dtype=torch.int8, device="cuda"),
                            torch.zeros((nb, bs, 2, 64), dtype=torch.int8, device="cuda"), None,
                            d.cache.k_scale, d.cache.v_scale)
    with pytest.raises(pkv.PkvError, match="head_dim must be 128"):
        pkv.paged_attn_decode(d.q[..., :64].contiguous(), wide, d.block_table, d.seq_lens, case.scale)
