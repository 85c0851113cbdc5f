"""paged_attn_decode_noalloc, the decode entry point for callers that cannot allocate,
against paged_attn_decode on the same inputs through the C ABI: bit-identical outputs on
two calls in a row, the second with a smaller input (so stale scratch from the first call
would show), on the stream-split (bf16), partition (fp32) and MLA paths; both also within
the oracle's bars.  Calls needing more scratch than the static array holds are refused on
the host."""
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


from gpu_util import DeviceCase, assert_rows_close, host  # noqa: E402

PAIRS = [
    # name, (B, H, Hkv, D, dtype, block_size, max_blocks, len_range, window, rope) big then small
    ("bf16 stream split", (24, 32, 8, 128, "bf16", 128, 24, (1, 3000), 0, 0),
     (5, 32, 8, 128, "bf16", 128, 8, (1, 900), 0, 0)),
    ("bf16 stream split, window", (12, 16, 2, 128, "bf16", 16, 200, (1, 3000), 500, 0),
     (3, 16, 2, 128, "bf16", 16, 40, (1, 600), 100, 0)),
    ("fp32 partitions", (6, 8, 2, 128, "f32", 32, 64, (1, 2000), 0, 0),
     (2, 8, 2, 128, "f32", 32, 16, (1, 500), 0, 0)),
    ("MLA partitions", (4, 64, 1, 512, "bf16", 64, 48, (1, 3000), 0, 64),
     (2, 32, 1, 512, "bf16", 64, 12, (1, 700), 0, 64)),
]


def _case(seed, spec):
    B, H, Hkv, D, dt, bs, mb, lr, w, rope = spec
    return workloads.decode_case(seed, B, H, Hkv, D, dt, block_size=bs, max_blocks=mb, len_range=lr, window=w,
                                 null_block=True, rope_dim=rope)


@pytest.mark.parametrize("pair", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_equals_decode_on_two_calls(orc, pair):
    import paged_kv_cache_80_amd as pkv
    name, big, small = pair
    for i, spec in enumerate((big, small)):
        case = _case(80 + 10 * i + len(name), spec)
        print(f"{name}: call {i + 1}, B={case.B}, max len {int(case.seq_lens.max())}", flush=True)
        d = DeviceCase(case)
        d.write(d.resolve())
        split = 2 * case.block_size if case.dtype == "f32" or case.rope_dim else 0
        want = pkv.paged_attn_decode(d.q, d.cache, d.block_table, d.seq_lens, case.scale, case.window,
                                     q_rope=d.q_rope, split_tokens=split)
        got = torch.full_like(want, float("nan"))
        pkv.paged_attn_decode_noalloc(d.q, d.cache, d.block_table, d.seq_lens, case.scale, got, case.window,
                                      q_rope=d.q_rope, split_tokens=split)
        torch.cuda.synchronize()
        assert host(got).tobytes() == host(want).tobytes()
        ref, _, _ = oracle_run(orc, case)
        assert_rows_close(got, ref, 1e-5 if case.dtype == "f32" else 2e-3)


def test_noalloc_refuses_calls_past_its_scratch():
    """Sizes alone decide: an MLA step of 64 sequences x 128 heads over 8192-key tables needs
    ~67 MB of partials, a stream-split step of 4096 sequences x 8 KV heads x 16 heads ~280 MB;
    both exceed the 32 MiB array and are refused before anything is launched."""
    import paged_kv_cache_80_amd as pkv
    cap = pkv.paged_attn_decode_noalloc_capacity()
    assert cap == 32 << 20
    dev = "cuda"
    mla = pkv.PagedKVCache(torch.zeros((1, 128, 1, 512), dtype=torch.bfloat16, device=dev), None,
                           torch.zeros((1, 128, 1, 64), dtype=torch.bfloat16, device=dev))
    q = torch.zeros((64, 128, 512), dtype=torch.bfloat16, device=dev)
    need = pkv.paged_attn_decode_workspace(mla, 64, 128, 64, 576 ** -0.5)
    assert need > cap
    with pytest.raises(pkv.PkvError, match="static array"):
        pkv.paged_attn_decode_noalloc(q, mla, torch.zeros((64, 64), dtype=torch.int32, device=dev),
                                      torch.ones(64, dtype=torch.int32, device=dev), 576 ** -0.5,
                                      torch.empty_like(q), q_rope=torch.zeros((64, 128, 64), dtype=torch.bfloat16,
                                                                              device=dev))
    std = pkv.PagedKVCache(torch.zeros((1, 128, 8, 128), dtype=torch.bfloat16, device=dev),
                           torch.zeros((1, 128, 8, 128), dtype=torch.bfloat16, device=dev))
    q = torch.zeros((4096, 128, 128), dtype=torch.bfloat16, device=dev)
    assert pkv.paged_attn_decode_workspace(std, 4096, 128, 1, 0.088) > cap
    with pytest.raises(pkv.PkvError, match="static array"):
        pkv.paged_attn_decode_noalloc(q, std, torch.zeros((4096, 1), dtype=torch.int32, device=dev),
                                      torch.ones(4096, dtype=torch.int32, device=dev), 0.088, torch.empty_like(q))
