"""The seeded input generators: a seed names one input (so every parity case and every
bench line can be reproduced), the draws follow the documented recipe, and the shapes,
tables and null-block padding are what the workloads state.  CPU only."""
import numpy as np
import pytest

import workloads


def _arrays(case):
    return {k: v for k, v in vars(case).items() if isinstance(v, np.ndarray)}


@pytest.mark.parametrize("make", [
    lambda s: workloads.decode_case(s, 5, 8, 2, 128, "bf16", block_size=16, max_blocks=40, len_range=(0, 600),
                                    window=100, null_block=True),
    lambda s: workloads.prefill_case(s, 3, 16, 4, 64, "f32", cached=[10, 0, 300], new=[5, 40, 1], block_size=32),
    lambda s: workloads.latent_case(s, 3, "bf16", new=[5, 9, 1], cached=[0, 100, 7], block_size=16, pad_every=3),
], ids=["decode", "prefill", "latent write"])
def test_a_seed_names_one_input(make):
    a, b, c = make(3), make(3), make(4)
    for k, v in _arrays(a).items():
        np.testing.assert_array_equal(v, _arrays(b)[k], err_msg=k)
    assert any(not np.array_equal(v, _arrays(c)[k]) for k, v in _arrays(a).items() if v.size > 8)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 3.0e38], dtype=np.float32)
    back = workloads.bf16_to_f32(workloads.bf16_bits(x))
    # ties go to the even significand: 1 + 2^-8 -> 1, 1 + 3 * 2^-8 -> 1 + 2^-6
    np.testing.assert_array_equal(back[:3], np.array([1.0, 1.0, 1.0 + 2.0 ** -6], dtype=np.float32))
    assert back[3] == -2.5 and np.isfinite(back[4])


def test_null_block_tables_and_padding():
    case = workloads.decode_case(0, 6, 8, 2, 128, "bf16", block_size=16, max_blocks=64, len_range=(1, 1000),
                                 window=200, null_block=True)
    bt, L = case.block_table, case.seq_lens
    real = bt[bt != 0]
    assert len(np.unique(real)) == real.size  # every real block belongs to one table entry
    for b in range(case.B):
        first = max(0, int(L[b]) - 200) // 16
        last = (int(L[b]) - 1) // 16
        assert np.all(bt[b, first:last + 1] != 0)  # the blocks the window reads are real
        assert np.all(bt[b, :first] == 0) and np.all(bt[b, last + 1:] == 0)  # the rest is the null block
    assert np.all(case.k_cache.view(np.uint16)[0] == workloads.NAN_BF16)  # block 0 holds NaN


def test_full_size_workload_shapes():
    c = workloads.mha_decode_7b(0)
    assert (c.B, c.H, c.Hkv, c.D, c.block_size) == (64, 32, 32, 128, 128) and np.all(c.seq_lens == 2048)
    assert sorted(c.block_table.ravel().tolist()) == list(range(1024))  # a permutation of the whole pool
    p = workloads.chunked_prefill(0)
    assert p.q.shape == (4096, 32, 128) and p.cu_seqlens_q.tolist() == list(range(0, 4097, 512))
    t = workloads.gqa_mtp_decode(0)
    assert t.q.shape == (128, 64, 128) and np.all(np.diff(t.cu_seqlens_q) == 4)
    assert t.seq_lens.min() >= 1024 and t.seq_lens.max() <= 32768 and t.null_block
    m = workloads.mla_latent_write(0)
    assert m.latent.shape == (32768, 576) and m.cache_nope.shape[1:] == (128, 1, 512)
