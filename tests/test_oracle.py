"""Pins for the CPU oracle, checked against what the pages and the mathematics fix.

Each test names the page and section it rests on.  None of them compares the
oracle with itself under a retyped formula: expected values are the pages'
printed numbers, closed forms, invariants, byte-exact library routines, or the
independent block-gather brute force in brute.py.
"""
import json
import math
import os

import numpy as np
import pytest

import brute
import workloads
from helpers import oracle_attend, oracle_run, oracle_slots, oracle_write

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slot_examples.json")


@pytest.fixture(scope="module")
def gold():
    with open(GOLDEN) as f:
        return json.load(f)


def _page_table(gold):
    lay = gold["layout"]
    # skill page section 3.2: block_table = arange(total_blocks).reshape(batch_size, -1)
    return np.arange(lay["total_blocks"], dtype=np.int32).reshape(lay["batch_size"], -1), lay


# --------------------------------------------------------------------------- index resolution

def test_worked_mapping_example(orc, gold):
    """skill page 3.1: batch 1, position 300, block 128 -> block 2, offset 44, physical 18, slot 2348."""
    bt, lay = _page_table(gold)
    ex = gold["mapping_example"]
    assert ex["seq_pos"] // lay["block_size"] == ex["logical_block"]
    assert ex["seq_pos"] % lay["block_size"] == ex["offset"]
    assert bt[ex["batch_idx"], ex["logical_block"]] == ex["physical_block"]
    s = orc.resolve_slots(bt, lay["block_size"], lay["total_blocks"], [ex["batch_idx"]], [ex["seq_pos"]])
    assert s.tolist() == [ex["slot"]]


def test_prefill_slot_example(orc, gold):
    """skill page 3.3: kv_len [512, 256], max_seq_len 2048 -> [0..511] ++ [2048..2303] (768 slots)."""
    bt, lay = _page_table(gold)
    ex = gold["prefill_example"]
    bidx = np.concatenate([np.full(n, b) for b, n in enumerate(ex["kv_len"])])
    pos = np.concatenate([np.arange(n) for n in ex["kv_len"]])
    s = orc.resolve_slots(bt, lay["block_size"], lay["total_blocks"], bidx, pos)
    want = np.concatenate([np.arange(a, b) for a, b in ex["slot_ranges"]])
    assert s.size == ex["length"]
    np.testing.assert_array_equal(s, want)


def test_decode_slot_example(orc, gold):
    """skill page 3.3: kv_len [522, 266] with offsets [0, 2048] -> slot_mapping [[522], [2314]]."""
    bt, lay = _page_table(gold)
    ex = gold["decode_example"]
    s = orc.resolve_slots(bt, lay["block_size"], lay["total_blocks"], [0, 1], ex["kv_len"])
    assert s.tolist() == ex["slot_mapping"]
    assert s.tolist() == [k + o for k, o in zip(ex["kv_len"], ex["kv_len_offset"])]


def test_closed_form_under_arange_table(orc):
    """Guide, mode 2: the block-table formula equals b * max_seq_len + pos when the table is arange."""
    rng = np.random.default_rng(5)
    for bs, nblk, B in [(128, 16, 2), (16, 7, 5), (4, 3, 9)]:
        bt = np.arange(B * nblk, dtype=np.int32).reshape(B, nblk)
        bidx = rng.integers(0, B, 500)
        pos = rng.integers(0, nblk * bs, 500)
        s = orc.resolve_slots(bt, bs, B * nblk, bidx, pos)
        np.testing.assert_array_equal(s, bidx * (nblk * bs) + pos)


def test_resolve_permuted_table_by_block_gather(orc):
    """A shuffled table: the slot's row in the flat cache is the row the block gather reaches."""
    rng = np.random.default_rng(6)
    B, nblk, bs = 3, 5, 8
    bt = rng.permutation(B * nblk).astype(np.int32).reshape(B, nblk)
    ids = np.arange(B * nblk * bs).reshape(B * nblk, bs, 1, 1)  # each cache row holds its own index
    for b in range(B):
        pos = np.arange(nblk * bs)
        s = orc.resolve_slots(bt, bs, B * nblk, np.full(pos.size, b), pos)
        np.testing.assert_array_equal(s, brute.gather_blocks(ids, bt[b], nblk * bs).ravel())


def test_resolve_rejects_out_of_range(orc):
    bt = np.array([[0, 1], [2, 7]], dtype=np.int32)
    with pytest.raises(ValueError):
        orc.resolve_slots(bt, 4, 4, [1], [5])  # block 7 is not in a 4-block pool
    with pytest.raises(ValueError):
        orc.resolve_slots(bt, 4, 8, [0], [8])  # position past the table
    with pytest.raises(ValueError):
        orc.resolve_slots(bt, 4, 8, [2], [0])  # no such sequence


# --------------------------------------------------------------------------- cache write

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_write_is_fancy_index_assignment(orc, dtype):
    """Guide, mode 2: the write is a row scatter into the cache viewed as [slots, H_kv, D]."""
    rng = np.random.default_rng(7)
    nb, bs, hkv, d = 6, 16, 2, 8
    cache = workloads.normal(rng, (nb, bs, hkv, d), dtype)
    rows = workloads.normal(rng, (20, hkv, d), dtype)
    slots = rng.choice(nb * bs, 20, replace=False).astype(np.int32)
    slots[3] = -1  # skipped row
    want = cache.copy()
    flat = want.reshape(nb * bs, hkv, d)
    keep = slots >= 0
    flat[slots[keep]] = rows[keep]  # numpy fancy-index assignment
    got = cache.copy()
    orc.cache_write(got, slots, rows)
    assert got.tobytes() == want.tobytes()
    untouched = np.setdiff1d(np.arange(nb * bs), slots[keep])
    assert got.reshape(nb * bs, -1)[untouched].tobytes() == cache.reshape(nb * bs, -1)[untouched].tobytes()


def test_write_rejects_slot_past_cache(orc):
    cache = np.zeros((2, 4, 1, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        orc.cache_write(cache, [8], np.ones((1, 1, 4), dtype=np.float32))


# --------------------------------------------------------------------------- attention vs brute force

DECODE_SHAPES = [
    # B, H, Hkv, D, dtype, bs, max_blocks, len_range, window, rope
    (3, 4, 4, 16, "f32", 8, 6, (1, 48), 0, 0),      # MHA, ragged
    (4, 8, 2, 32, "bf16", 16, 5, (1, 80), 0, 0),    # GQA 4
    (2, 6, 1, 16, "bf16", 4, 9, (1, 36), 0, 0),     # MQA
    (5, 4, 2, 16, "f32", 8, 8, (1, 64), 5, 0),      # sliding window
    (3, 8, 1, 32, "bf16", 8, 6, (1, 48), 0, 8),     # MLA absorbed (latent 32 + rope 8)
    (2, 4, 1, 16, "f32", 4, 8, (1, 32), 3, 4),      # MLA + window
]


@pytest.mark.parametrize("shape", DECODE_SHAPES)
@pytest.mark.parametrize("seed", [0, 1])
def test_decode_matches_brute_force(orc, shape, seed):
    B, H, Hkv, D, dt, bs, mb, lr, w, r = shape
    case = workloads.decode_case(seed, B, H, Hkv, D, dt, block_size=bs, max_blocks=mb, len_range=lr,
                                 window=w, null_block=True, rope_dim=r)
    out, c, _ = oracle_run(orc, case)
    want = brute.decode(c, c.k_cache, c.v_cache_or_k, c.k_rope_cache)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)


PREFILL_SHAPES = [
    # B, H, Hkv, D, dtype, bs, cached, new, window, rope
    (2, 4, 4, 16, "f32", 8, [5, 0], [7, 12], 0, 0),
    (3, 8, 2, 16, "bf16", 4, [9, 1, 16], [3, 8, 5], 0, 0),
    (2, 4, 2, 16, "f32", 8, [20, 3], [6, 9], 4, 0),
    (2, 4, 1, 16, "bf16", 8, [10, 4], [5, 3], 0, 8),
]


@pytest.mark.parametrize("shape", PREFILL_SHAPES)
def test_prefill_matches_brute_force(orc, shape):
    B, H, Hkv, D, dt, bs, cached, new, w, r = shape
    case = workloads.prefill_case(3, B, H, Hkv, D, dt, cached=cached, new=new, block_size=bs,
                                  window=w, rope_dim=r, null_block=True)
    out, c, _ = oracle_run(orc, case)
    want = brute.prefill(c, c.k_cache, c.v_cache_or_k, c.k_rope_cache)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)


def test_tnd_cumulative_lengths_prefill(orc, gold):
    """Guide / skill page 3.4: a TND prefill of kv_len [512, 256] carries cumulative q lengths
    [512, 768]; with no cached prefix each sequence's rows are a plain causal prefill."""
    ex = gold["tnd_cumsum_example"]
    kv = ex["kv_len"]
    case = workloads.prefill_case(4, 2, 2, 1, 8, "f32", cached=[0, 0], new=kv, block_size=128,
                                  max_blocks=4)
    np.testing.assert_array_equal(case.cu_seqlens_q[1:], ex["actual_seq_lengths"])
    units = np.array([0, 1, 511 * 2, 512 * 2 + 1, 767 * 2])  # first/last rows of both sequences
    out, c, _ = oracle_run(orc, case, units=units)
    full = brute.prefill(c, c.k_cache, c.v_cache_or_k)
    for u in units:
        np.testing.assert_allclose(out[u // 2, u % 2], full[u // 2, u % 2], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- closed forms

def _with_lengths(seed, lens, **kw):
    kw.setdefault("block_size", 8)
    kw.setdefault("max_blocks", 8)
    return workloads.decode_case(seed, len(lens), kw.pop("H", 4), kw.pop("Hkv", 2), kw.pop("D", 16),
                                 kw.pop("dtype", "bf16"), seq_lens=lens, **kw)


def _value_row(c, b, pos, g):
    v = c.v_cache_or_k
    bs = c.block_size
    return brute.to_f64(v[c.block_table[b, pos // bs], pos % bs, g])


def test_single_key_returns_its_value_exactly(orc):
    """softmax over one key is exactly 1, so o = v_0 ("KV Cache notes", p_ij / o_i formula)."""
    case = _with_lengths(8, [1, 1, 1])
    out, c, _ = oracle_run(orc, case)
    for b in range(3):
        for h in range(case.H):
            assert np.array_equal(out[b, h], _value_row(c, b, 0, h // case.G))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_window_one_returns_newest_value_exactly(orc, dtype):
    """A window of 1 leaves only the query's own key: o = v_{L-1} for every length."""
    lens = list(range(1, 65))
    case = _with_lengths(9, lens, window=1, dtype=dtype, H=2, Hkv=1, null_block=True)
    out, c, _ = oracle_run(orc, case)
    for b, L in enumerate(lens):
        for h in range(2):
            assert np.array_equal(out[b, h], _value_row(c, b, L - 1, 0))


def test_zero_query_gives_mean_of_values(orc):
    """q = 0 makes every logit 0, so p is uniform over the visible keys and o is their mean."""
    case = _with_lengths(10, [1, 7, 33, 64], window=0, dtype="f32")
    case.q[...] = 0
    out, c, _ = oracle_run(orc, case)
    for b, L in enumerate(case.seq_lens):
        for h in range(case.H):
            vals = np.stack([_value_row(c, b, j, h // case.G) for j in range(L)])
            np.testing.assert_allclose(out[b, h], vals.mean(0), rtol=1e-12, atol=1e-14)


def test_identical_keys_give_mean_of_window(orc):
    """Equal keys give equal logits: o is the mean of the W newest values."""
    case = _with_lengths(11, [40, 64, 3], window=16, dtype="f32", null_block=True)
    out, c, _ = oracle_run(orc, case)  # first write, then overwrite every key row with one vector
    c.k_cache[...] = c.k_cache[1, 0, 0]
    out = oracle_attend(orc, c)
    for b, L in enumerate(case.seq_lens):
        lo = max(0, L - 16)
        for h in range(case.H):
            vals = np.stack([_value_row(c, b, j, h // case.G) for j in range(lo, L)])
            np.testing.assert_allclose(out[b, h], vals.mean(0), rtol=1e-12, atol=1e-14)


def test_dominant_key_survives_huge_logits(orc):
    """With logits near 1e6 exp overflows unless the row maximum is subtracted first
    ("KV Cache notes", the first engineering detail); the result is the dominant key's value."""
    case = _with_lengths(12, [50], H=1, Hkv=1, D=4, dtype="f32")
    out, c, _ = oracle_run(orc, case)
    c.k_cache[...] = 0
    c.q[...] = 1.0
    bs = c.block_size
    j = 17
    c.k_cache[c.block_table[0, j // bs], j % bs, 0, :] = 1.0
    c.scale = 1e6
    out = oracle_attend(orc, c)
    np.testing.assert_array_equal(out[0, 0], _value_row(c, 0, j, 0))


def test_empty_sequence_gives_zero_row(orc):
    case = _with_lengths(13, [0, 5], dtype="f32")
    out, c, _ = oracle_run(orc, case)
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out[1])) and np.any(out[1] != 0)


# --------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("window", [0, 6])
def test_rows_sum_to_one(orc, window):
    """Each softmax row sums to 1 and puts no weight outside the visible keys ("KV Cache notes")."""
    case = workloads.decode_case(14, 4, 4, 2, 16, "bf16", block_size=8, max_blocks=6,
                                 len_range=(1, 48), window=window, null_block=True)
    (out, probs), c, _ = oracle_run(orc, case, want_probs=True)
    for b, L in enumerate(case.seq_lens):
        lo = max(0, L - window) if window else 0
        np.testing.assert_allclose(probs[b].sum(-1), 1.0, rtol=0, atol=1e-12)
        assert np.all(probs[b][:, :lo] == 0) and np.all(probs[b][:, L:] == 0)
        assert np.all(probs[b][:, lo:L] > 0)


def test_paged_equals_contiguous(orc):
    """Skill page modes 1 and 2: the same logical rows stored under a shuffled block table
    give bit-identical results to the contiguous (arange-table, BSH) layout."""
    B, nblk, bs = 3, 5, 8
    case = workloads.decode_case(15, B, 4, 2, 16, "bf16", block_size=bs, max_blocks=nblk,
                                 len_range=(1, nblk * bs),
                                 table=np.arange(B * nblk, dtype=np.int32).reshape(B, nblk))
    out_contig, c, _ = oracle_run(orc, case)
    rng = np.random.default_rng(0)
    perm = rng.permutation(B * nblk).astype(np.int32)  # logical block i lives at physical perm[i]
    shuffled = c.copy_caches()
    shuffled.block_table = perm.reshape(B, nblk)
    shuffled.k_cache[perm] = c.k_cache
    shuffled.v_cache[perm] = c.v_cache
    out_paged = oracle_attend(orc, shuffled)
    assert np.array_equal(out_paged, out_contig)


@pytest.mark.parametrize("fill", ["nan", 1e30, -1e30])
def test_null_block_padding_is_never_read(orc, fill):
    """KV Cache management design doc: the null block only pads tables; with a window the
    expired logical blocks point at it.  Whatever it holds, the result is unchanged."""
    case = workloads.decode_case(16, 6, 4, 2, 16, "f32", block_size=4, max_blocks=12,
                                 len_range=(1, 48), window=7, null_block=True)
    assert (case.block_table == 0).any()
    out_nan, c, _ = oracle_run(orc, case)
    other = c.copy_caches()
    other.k_cache[0] = np.float32(fill)
    other.v_cache[0] = np.float32(fill)
    out = oracle_attend(orc, other)
    assert np.array_equal(out, out_nan) and np.all(np.isfinite(out))


def test_prefill_rows_equal_decode_steps(orc):
    """"KV Cache notes", 40-line minimal implementation: one-shot prefill equals token-by-token
    decode.  Row i of a chunk equals a decode whose length ends at that row (bit-identical)."""
    case = workloads.prefill_case(17, 2, 4, 2, 16, "bf16", cached=[9, 20], new=[6, 11], block_size=8,
                                  null_block=True)
    out, c, _ = oracle_run(orc, case)
    for b in range(2):
        for i in range(int(case.cu_seqlens_q[b + 1] - case.cu_seqlens_q[b])):
            t = case.cu_seqlens_q[b] + i
            L = case.seq_lens[b] - (case.cu_seqlens_q[b + 1] - t) + 1
            step = orc.paged_decode(c.q[t:t + 1], c.k_cache, c.v_cache, c.block_table[b:b + 1],
                                    [L], c.scale)
            assert np.array_equal(step[0], out[t])


def test_gqa_equals_mha_on_expanded_cache(orc):
    """"KV Cache notes", MHA -> MQA -> GQA: repeat_kv after the cache; GQA equals MHA on a cache
    whose KV heads are expanded so query head h reads copy h of KV head h // G."""
    case = workloads.decode_case(18, 3, 8, 2, 16, "bf16", block_size=8, max_blocks=5,
                                 len_range=(1, 40))
    out_gqa, c, _ = oracle_run(orc, case)
    k_exp = np.ascontiguousarray(np.repeat(c.k_cache, 4, axis=2))
    v_exp = np.ascontiguousarray(np.repeat(c.v_cache, 4, axis=2))
    out_mha = orc.paged_decode(c.q, k_exp, v_exp, c.block_table, c.seq_lens, c.scale)
    assert np.array_equal(out_mha, out_gqa)


def test_mla_equals_attention_on_concatenated_key(orc):
    """MLA absorbed form ("KVCache optimisation skill", mode 3): key = [latent | rope] of width
    k+r, value = latent.  Same numbers as standard attention on a concatenated key cache."""
    case = workloads.decode_case(19, 3, 8, 1, 32, "bf16", block_size=8, max_blocks=6,
                                 len_range=(1, 48), rope_dim=8)
    out_mla, c, _ = oracle_run(orc, case)
    kcat = np.ascontiguousarray(np.concatenate([c.k_cache, c.k_rope_cache], axis=-1))
    qcat = np.ascontiguousarray(np.concatenate([c.q, c.q_rope], axis=-1))
    out_std = orc.paged_decode(qcat, kcat, c.k_cache, c.block_table, c.seq_lens, c.scale)
    np.testing.assert_allclose(out_mla, out_std, rtol=1e-13, atol=1e-15)


def test_units_subset_matches_full_run(orc):
    case = workloads.decode_case(20, 4, 4, 2, 16, "bf16", block_size=8, max_blocks=6,
                                 len_range=(1, 48))
    full, c, _ = oracle_run(orc, case)
    units = np.array([0, 5, 15])
    part = oracle_attend(orc, c, units=units)
    for u in units:
        assert np.array_equal(part[u // 4, u % 4], full[u // 4, u % 4])


def test_thread_count_does_not_change_results(orc):
    case = workloads.decode_case(21, 4, 8, 2, 16, "bf16", block_size=8, max_blocks=6,
                                 len_range=(1, 48), window=9, null_block=True)
    a, c, _ = oracle_run(orc, case, nthreads=1)
    b = oracle_attend(orc, c, nthreads=4)
    assert np.array_equal(a, b)


def test_scale_is_explicit(orc):
    """Guide, FA v1/v2 name table: a dropped scale argument silently becomes 1.0.  The oracle
    takes the scale explicitly and it changes the result."""
    case = workloads.decode_case(22, 2, 2, 2, 16, "f32", block_size=8, max_blocks=4,
                                 len_range=(8, 32))
    a, c, _ = oracle_run(orc, case)
    c.scale = 1.0
    b = oracle_attend(orc, c)
    assert not np.allclose(a, b)
