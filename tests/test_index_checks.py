"""Host-side index checks (paged_kv_cache_80_amd.checks): the debugging mode that copies
the device index arrays to the host and refuses, before any launch, an entry a kernel
would read out of bounds.

Pinned to what the kernels dereference (include/pkv.h): only blocks holding a key some
query sees must carry valid ids -- the "KV Cache management design document" lays out
sliding-window tables with the null block before the window, and any value there must
pass -- while every planted bad entry in a visible block, an impossible length or a
repeated slot is caught."""
import numpy as np
import pytest

import workloads
from paged_kv_cache_80_amd import checks


def _window_case(seed=3, W=300, bs=16):
    return workloads.decode_case(seed, 6, 8, 2, 128, "bf16", block_size=bs, max_blocks=64,
                                 len_range=(1, 1000), window=W, null_block=True)


def test_valid_workload_tables_pass():
    for case in (workloads.decode_case(1, 4, 8, 8, 128, "bf16", block_size=128, max_blocks=8,
                                       len_range=(0, 1024)),
                 workloads.tiny_f32_decode(0), _window_case()):
        checks.check_decode(case.block_table, case.seq_lens, case.block_size, case.num_blocks, case.window)
    p = workloads.prefill_case(2, 3, 8, 2, 128, "bf16", cached=[0, 70, 300], new=[5, 0, 33], block_size=16,
                               null_block=True)
    checks.check_prefill(p.block_table, p.cu_seqlens_q, p.seq_lens, int(p.cu_seqlens_q[-1]), 33, 16,
                         p.num_blocks)
    checks.check_slots(np.arange(20, dtype=np.int32) * 3, p.num_blocks * 16)


def test_entries_outside_the_visible_blocks_may_hold_anything():
    case = _window_case()
    nb, bs = case.k_cache.shape[:2]
    bt = case.block_table.copy()
    for b, L in enumerate(case.seq_lens):
        lo = max(0, int(L) - case.window)
        first, last = lo // bs, (int(L) - 1) // bs if L > 0 else -1
        bt[b, :first] = -1                        # wholly before the window
        bt[b, last + 1:] = np.iinfo(np.int32).max  # past the last block
    checks.check_decode(bt, case.seq_lens, bs, nb, case.window)
    # without the window the same -1 entries are visible and refused
    if (bt == -1).any():
        with pytest.raises(checks.IndexCheckError, match="block id"):
            checks.check_decode(bt, case.seq_lens, bs, nb, 0)


@pytest.mark.parametrize("bad", [-1, "num_blocks"])
def test_a_bad_id_in_a_visible_block_is_caught(bad):
    case = _window_case()
    nb, bs = case.k_cache.shape[:2]
    b = int(np.argmax(case.seq_lens))
    L = int(case.seq_lens[b])
    bt = case.block_table.copy()
    bt[b, (L - 1) // bs] = -1 if bad == -1 else nb  # the block of the query's own key
    with pytest.raises(checks.IndexCheckError, match=f"sequence {b}"):
        checks.check_decode(bt, case.seq_lens, bs, nb, case.window)


def test_lengths_past_the_table_are_caught():
    case = _window_case()
    nb, bs = case.k_cache.shape[:2]
    lens = case.seq_lens.copy()
    lens[2] = case.block_table.shape[1] * bs + 1
    with pytest.raises(checks.IndexCheckError, match="seq_lens\\[2\\]"):
        checks.check_decode(case.block_table, lens, bs, nb)
    lens[2] = -1
    with pytest.raises(checks.IndexCheckError, match="seq_lens\\[2\\]"):
        checks.check_decode(case.block_table, lens, bs, nb)


def _prefill_tables():
    bt = np.array([[5, 1, 2, 3], [4, 6, 7, 0]], dtype=np.int32)
    cu = np.array([0, 3, 7], dtype=np.int32)
    L = np.array([40, 60], dtype=np.int32)
    return bt, cu, L


def test_prefill_checks():
    bt, cu, L = _prefill_tables()
    checks.check_prefill(bt, cu, L, 7, 4, 16, 8)
    with pytest.raises(checks.IndexCheckError, match="max_q_len"):
        checks.check_prefill(bt, cu, L, 7, 3, 16, 8)  # sequence 1 has 4 rows
    with pytest.raises(checks.IndexCheckError, match="total_q"):
        checks.check_prefill(bt, cu, L, 8, 4, 16, 8)
    with pytest.raises(checks.IndexCheckError, match="decreases"):
        checks.check_prefill(bt, np.array([0, 5, 3, 7][:3], dtype=np.int32), L, 3, 5, 16, 8)
    with pytest.raises(checks.IndexCheckError, match="seq_lens_kv\\[1\\]"):
        checks.check_prefill(bt, cu, np.array([40, 3], dtype=np.int32), 7, 4, 16, 8)  # fewer keys than rows
    bad = bt.copy()
    bad[1, 3] = 9  # block of keys 48..63: visible to sequence 1's rows (positions 56..59)
    with pytest.raises(checks.IndexCheckError, match="sequence 1"):
        checks.check_prefill(bad, cu, L, 7, 4, 16, 8)
    # window 8: sequence 0's first row (position 37) sees keys 30.. -> blocks 1, 2; block 0 may hold anything
    bad = bt.copy()
    bad[0, 0] = -7
    checks.check_prefill(bad, cu, L, 7, 4, 16, 8, window=8)
    with pytest.raises(checks.IndexCheckError, match="sequence 0"):
        checks.check_prefill(bad, cu, L, 7, 4, 16, 8, window=9 + 16)


def test_slot_checks():
    checks.check_slots(np.array([3, -1, 7, -1, 0], dtype=np.int32), 8)
    with pytest.raises(checks.IndexCheckError, match="past"):
        checks.check_slots(np.array([3, 8], dtype=np.int32), 8)
    with pytest.raises(checks.IndexCheckError, match="twice"):
        checks.check_slots(np.array([3, 5, 3], dtype=np.int32), 8)


def test_resolve_checks():
    bt = np.array([[2, 0], [1, -1]], dtype=np.int32)
    checks.check_resolve(bt, 16, np.array([0, 1, 1]), np.array([20, 3, -5]), num_blocks=3)
    with pytest.raises(checks.IndexCheckError, match="block id -1"):
        checks.check_resolve(bt, 16, np.array([1]), np.array([16]), num_blocks=3)
    with pytest.raises(checks.IndexCheckError, match="batch_idx"):
        checks.check_resolve(bt, 16, np.array([2]), np.array([0]))
    with pytest.raises(checks.IndexCheckError, match="pos"):
        checks.check_resolve(bt, 16, np.array([0]), np.array([32]))
    # without a pool size, ids are bounded by the int32 slot range
    huge = np.array([[2**27]], dtype=np.int32)
    with pytest.raises(checks.IndexCheckError, match="block id"):
        checks.check_resolve(huge, 16, np.array([0]), np.array([0]))


def test_write_at_checks():
    bt = np.array([[2, 0], [1, 3]], dtype=np.int32)
    checks.check_write_at(bt, 4, np.array([0, 1, 1, 0]), np.array([5, 0, -1, 1]), num_blocks=4)
    with pytest.raises(checks.IndexCheckError, match="twice"):  # positions 1 and 5 both land in slot 5
        checks.check_write_at(np.array([[1, 1]], dtype=np.int32), 4, np.array([0, 0]), np.array([1, 5]), num_blocks=2)
    with pytest.raises(checks.IndexCheckError, match="block id"):
        checks.check_write_at(bt, 4, np.array([1]), np.array([4]), num_blocks=3)


def test_append_checks():
    """paged_attn_decode_append: the decode's rules, and no two sequences append at one slot."""
    bt = np.array([[2, 0], [1, 3]], dtype=np.int32)
    checks.check_append(bt, np.array([6, 3]), 4, num_blocks=4)
    checks.check_append(bt, np.array([0, 3]), 4, num_blocks=4)  # an empty sequence appends nothing
    with pytest.raises(checks.IndexCheckError, match="twice"):  # both newest keys in slot 1 * 4 + 1
        checks.check_append(np.array([[1, 0], [1, 0]], dtype=np.int32), np.array([2, 2]), 4, num_blocks=4)
    with pytest.raises(checks.IndexCheckError, match="table width"):
        checks.check_append(bt, np.array([9, 1]), 4, num_blocks=4)
