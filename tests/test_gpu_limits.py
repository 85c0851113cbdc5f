"""GPU parity at the limits of the C ABI: the largest batch decode takes (65535 sequences:
the column prefix then comes from its own scan kernel, and every combine and grid
dimension is at its widest), the rejection just past it, and an MLA prefill whose query
rows (70000) exceed one launch (rows go in launches of at most 65528).  Outputs are
compared on sampled rows -- including the last ones and those on the launch boundary --
against the oracle, at the decode and prefill bars."""
import numpy as np
import pytest

import workloads
from helpers import oracle_run

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3
F32_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_80_amd as pkv
    pkv.load()


from gpu_util import DeviceCase, as_f64, assert_rows_close, dev, host  # noqa: E402


def _units(n_rows, extra, seed=0, k=512):
    rng = np.random.default_rng(seed)
    pick = rng.choice(n_rows, size=min(k, n_rows), replace=False)
    return np.unique(np.concatenate([pick, np.asarray(extra, dtype=np.int64)])).astype(np.int32)


@pytest.mark.parametrize("dtype,int8", [("bf16", False), ("f32", False), ("bf16", True)],
                         ids=["bf16 stream", "f32 partitions", "int8 stream"])
def test_decode_at_the_batch_limit(orc, dtype, int8):
    B, H = 65535, 2
    case = workloads.decode_case(65535, B, H, 1, 128, dtype, block_size=16, max_blocks=3, len_range=(0, 40),
                                 null_block=True, int8=int8)
    print(f"decode B={B} {dtype} int8={int8}", flush=True)
    d = DeviceCase(case)
    out, slots = d.run()
    rows = B * H
    units = _units(rows, list(range(8)) + list(range(rows - 64, rows)))
    ref, _, slots_ref = oracle_run(orc, case, units=units, inplace=not int8)
    np.testing.assert_array_equal(host(slots), slots_ref)
    assert np.all(np.isfinite(as_f64(out)))
    assert_rows_close(out, ref, F32_TOL if dtype == "f32" else BF16_TOL, rows=units)


def test_decode_past_the_batch_limit_is_rejected():
    import paged_kv_cache_80_amd as pkv

    B = 65536
    cache = pkv.PagedKVCache(torch.zeros((2, 16, 1, 128), dtype=torch.bfloat16, device="cuda"),
                             torch.zeros((2, 16, 1, 128), dtype=torch.bfloat16, device="cuda"))
    q = torch.zeros((B, 2, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    sl = torch.ones(B, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError, match="exceeds 65535"):
        pkv.paged_attn_decode(q, cache, bt, sl, 0.1)


def test_mla_prefill_across_launches(orc):
    """70000 query rows: the MLA kernel runs them as two launches (65528 + 4472)."""
    case = workloads.prefill_case(7, 2, 16, 1, 512, "bf16", cached=[0, 10], new=[35000, 35000], block_size=128,
                                  rope_dim=64, scale=1.0 / np.sqrt(576.0))
    print(f"MLA prefill rows={case.q.shape[0]}", flush=True)
    d = DeviceCase(case)
    out, slots = d.run()
    H = case.H
    edge_rows = [0, 1, 34999, 35000, 35001, 65526, 65527, 65528, 65529, 69999]
    extra = [r * H + h for r in edge_rows for h in range(H)]
    units = _units(case.q.shape[0] * H, extra, k=32)
    ref, _, slots_ref = oracle_run(orc, case, units=units, inplace=True)
    np.testing.assert_array_equal(host(slots), slots_ref)
    assert np.all(np.isfinite(as_f64(out)))
    assert_rows_close(out, ref, BF16_TOL, rows=units)
