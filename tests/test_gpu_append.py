"""GPU parity of paged_attn_decode_append: writing each sequence's newest K/V row at
position seq_lens[b] - 1 and decoding in one call gives, bit for bit, the cache and the
output of the two separate calls (kv_cache_write_at, then paged_attn_decode), which the
other GPU tests pin to the oracle; one case is also checked against the oracle directly.

On the bf16 stream-split path the two are one kernel (the newest key is read from the
caller's rows and stored by the wave that reads it); every other cache (fp32, int8, MLA)
writes first and then decodes.  The operands of every MFMA are the same bytes either way,
so equality is exact, not approximate."""
import numpy as np
import pytest

import workloads
from helpers import oracle_run

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_80_amd as pkv
    pkv.load()


from gpu_util import DeviceCase, assert_rows_close, dev, host  # noqa: E402

# name, B, H, Hkv, D, dtype, bs, max_blocks, seq_lens or len_range, window, extra
CASES = [
    ("bf16 GQA, 128-token blocks", 8, 32, 8, 128, "bf16", 128, 40, (1, 5000), 0, {}),
    ("bf16 MHA, lengths on tile and block edges", 9, 16, 16, 128, "bf16", 64, 8,
     [1, 31, 32, 33, 63, 64, 65, 511, 512], 0, {}),
    ("bf16, 16-token blocks (tiles over two blocks)", 6, 16, 4, 128, "bf16", 16, 100, (1, 1500), 0, {}),
    ("bf16, window over null-padded tables", 5, 64, 8, 128, "bf16", 64, 60, (1, 3800), 700, {}),
    ("bf16, empty sequences", 5, 8, 2, 128, "bf16", 32, 10, [0, 17, 0, 320, 1], 0, {}),
    ("bf16, batch past the in-LDS prefix", 2100, 4, 2, 128, "bf16", 16, 4, (0, 64), 0, {}),
    ("fp32 (write, then the vector-ALU decode)", 4, 8, 2, 128, "f32", 32, 40, (1, 1200), 0, {}),
    ("int8 cache (quantizing write, then decode)", 3, 32, 8, 128, "bf16", 64, 20, (1, 1200), 0, {"int8": True}),
    ("MLA (latent + rope write, then decode)", 3, 32, 1, 512, "bf16", 64, 20, (1, 1200), 0,
     {"rope_dim": 64, "scale": 576 ** -0.5}),
]


def _case(i, spec):
    name, B, H, Hkv, D, dt, bs, mb, lens, w, extra = spec
    kw = {"seq_lens": np.array(lens, dtype=np.int32)} if isinstance(lens, list) else {"len_range": lens}
    return workloads.decode_case(900 + i, B, H, Hkv, D, dt, block_size=bs, max_blocks=mb, window=w,
                                 null_block=True, **kw, **extra)


def _caches(d):
    c = d.cache
    parts = [c.k_cache, c.v_cache, c.k_rope_cache, c.k_scale, c.v_scale]
    return [host(t).tobytes() for t in parts if t is not None]


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("split", [0, 2])
def test_append_equals_write_then_decode(i, out_dtype, split):
    import paged_kv_cache_80_amd as pkv
    case = _case(i, CASES[i])
    od = torch.float32 if out_dtype == "f32" else None
    split_tokens = split * case.block_size
    two = DeviceCase(case)
    ref, _ = two.run(out_dtype=od, split_tokens=split_tokens)
    one = DeviceCase(case)
    out = pkv.paged_attn_decode_append(one.q, one.new_k, one.new_v, one.cache, one.block_table, one.seq_lens,
                                       case.scale, case.window, q_rope=one.q_rope, k_rope_new=one.new_k_rope,
                                       out_dtype=od, split_tokens=split_tokens)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), f"{CASES[i][0]}: outputs differ"
    assert _caches(one) == _caches(two), f"{CASES[i][0]}: caches differ"


def test_append_matches_oracle(orc):
    """The fused path against the oracle directly: the decode sees the appended key."""
    import paged_kv_cache_80_amd as pkv
    case = _case(0, CASES[0])
    ref, _, _ = oracle_run(orc, case)
    d = DeviceCase(case)
    out = pkv.paged_attn_decode_append(d.q, d.new_k, d.new_v, d.cache, d.block_table, d.seq_lens, case.scale,
                                       case.window, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_rows_close(out, ref, 1e-4)


def test_append_call_after_call_keeps_the_cache_consistent():
    """Three decode steps, each appending one token per sequence: the fused call and the
    separate calls leave the same cache and give the same outputs at every step."""
    import paged_kv_cache_80_amd as pkv
    # no null block: every table entry is a real block, so the appended positions are too
    case = workloads.decode_case(950, 6, 16, 4, 128, "bf16", block_size=32, max_blocks=40,
                                 len_range=(1, 1200))
    one, two = DeviceCase(case), DeviceCase(case)
    rng = np.random.default_rng(3)
    for step in range(3):
        if step:
            for d in (one, two):
                d.seq_lens += 1
                d.new_pos += 1
            k = dev(workloads.bf16_bits(rng.standard_normal(case.new_k.shape).astype(np.float32)))
            v = dev(workloads.bf16_bits(rng.standard_normal(case.new_v.shape).astype(np.float32)))
            for d in (one, two):
                d.new_k.copy_(k)
                d.new_v.copy_(v)
        ref, _ = two.run()
        out = pkv.paged_attn_decode_append(one.q, one.new_k, one.new_v, one.cache, one.block_table, one.seq_lens,
                                           case.scale, case.window)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"step {step}: outputs differ"
        assert _caches(one) == _caches(two), f"step {step}: caches differ"
