"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check the pins catch each.

Every mutant is a textual edit of oracle/pkv_oracle.c compiled into a temporary
library.  The battery below re-runs a cross-section of the pins in
test_oracle.py (page worked examples, brute force, closed forms, invariants)
against the mutant; each mutant must fail at least one of them.  If an edit no
longer matches the source the test fails, so the list stays in step with the
code.
"""
import json
import os

import numpy as np
import pytest

import brute
import workloads
from helpers import oracle_run

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")

MUTANTS = {
    "offset_uses_divide": ("int32_t offset = pos % block_size;", "int32_t offset = pos / block_size;"),
    "block_uses_modulo": ("int32_t logical_block = pos / block_size;",
                          "int32_t logical_block = pos % block_size;"),
    "prefill_excludes_diagonal": ("int32_t hi = p + 1;", "int32_t hi = p;"),
    "prefill_upper_left_causal": ("int32_t p = seq_lens_kv[b] - n_new + i;", "int32_t p = i;"),
    "decode_window_off_by_one": ("? len - window : 0", "? len - window + 1 : 0"),
    "prefill_window_off_by_one": ("? p + 1 - window : 0", "? p - window : 0"),
    "gqa_head_modulo": ("h / group, lo, len", "h % c->num_kv_heads, lo, len"),
    "mla_rope_dropped": ("dot += rdot;", "(void)rdot;"),
    "rope_uses_latent_query": ("elem(qr_base, c->dtype, qr_off + e)", "elem(q_base, c->dtype, q_off + e)"),
    "no_max_subtraction": ("score[i] = exp(score[i] - m);", "score[i] = exp(score[i]);"),
    "no_normalisation": ("out_row[d] /= l;", "out_row[d] /= 1.0;"),
    "scale_dropped": ("score[j - lo] = scale * dot;", "score[j - lo] = dot;"),
    "key_head_major": ("int64_t krow = (s * c->num_kv_heads + g) * (int64_t)c->k_dim;",
                       "int64_t krow = ((int64_t)g * c->num_blocks * c->block_size + s) * (int64_t)c->k_dim;"),
    "value_read_from_key_cache": ("elem(c->v_cache, c->dtype, vrow + d)", "elem(c->k_cache, c->dtype, vrow + d)"),
    "bf16_widening_shift": ("[i]) << 16;", "[i]) << 15;"),
    "write_skips_last_row": ("for (int32_t t = 0; t < n; ++t) {", "for (int32_t t = 0; t + 1 < n; ++t) {"),
}


def _battery(orc, lib):
    """Returns the names of the pins the library fails."""
    failed = []

    def check(name, fn):
        try:
            ok = fn()
        except Exception:  # a crash or a raised error is a caught mistake too
            ok = False
        if not ok:
            failed.append(name)

    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "slot_examples.json")))
    bt = np.arange(32, dtype=np.int32).reshape(2, 16)

    check("worked_slot", lambda: orc.resolve_slots(bt, 128, 32, [1], [300], lib=lib).tolist() == [2348])
    check("decode_slots", lambda: orc.resolve_slots(bt, 128, 32, [0, 1], gold["decode_example"]["kv_len"],
                                                    lib=lib).tolist() == gold["decode_example"]["slot_mapping"])

    def write_ok():
        rng = np.random.default_rng(1)
        cache = workloads.normal(rng, (4, 8, 2, 4), "bf16")
        rows = workloads.normal(rng, (5, 2, 4), "bf16")
        slots = np.array([3, 9, 0, 31, 17], dtype=np.int32)
        want = cache.copy()
        want.reshape(32, 2, 4)[slots] = rows
        orc.cache_write(cache, slots, rows, lib=lib)
        return cache.tobytes() == want.tobytes()
    check("write_fancy_index", write_ok)

    def run(case):
        class _O:  # route the shared helpers through this library
            resolve_slots = staticmethod(lambda *a, **k: orc.resolve_slots(*a, lib=lib, **k))
            cache_write = staticmethod(lambda *a, **k: orc.cache_write(*a, lib=lib, **k))
            paged_decode = staticmethod(lambda *a, **k: orc.paged_decode(*a, lib=lib, **k))
            paged_prefill = staticmethod(lambda *a, **k: orc.paged_prefill(*a, lib=lib, **k))
        return oracle_run(_O, case)

    def brute_decode(shape):
        B, H, Hkv, D, dt, bs, mb, lr, w, r = shape
        case = workloads.decode_case(0, B, H, Hkv, D, dt, block_size=bs, max_blocks=mb, len_range=lr,
                                     window=w, null_block=True, rope_dim=r)
        out, c, _ = run(case)
        want = brute.decode(c, c.k_cache, c.v_cache_or_k, c.k_rope_cache)
        return np.allclose(out, want, rtol=1e-12, atol=1e-13)

    def brute_prefill(shape):
        B, H, Hkv, D, dt, bs, cached, new, w, r = shape
        case = workloads.prefill_case(3, B, H, Hkv, D, dt, cached=cached, new=new, block_size=bs,
                                      window=w, rope_dim=r, null_block=True)
        out, c, _ = run(case)
        want = brute.prefill(c, c.k_cache, c.v_cache_or_k, c.k_rope_cache)
        return np.allclose(out, want, rtol=1e-12, atol=1e-13)

    check("brute_decode_gqa", lambda: brute_decode((4, 8, 2, 32, "bf16", 16, 5, (1, 80), 0, 0)))
    check("brute_decode_window", lambda: brute_decode((5, 4, 2, 16, "f32", 8, 8, (1, 64), 5, 0)))
    check("brute_decode_mla", lambda: brute_decode((3, 8, 1, 32, "bf16", 8, 6, (1, 48), 0, 8)))
    check("brute_prefill_gqa", lambda: brute_prefill((3, 8, 2, 16, "bf16", 4, [9, 1, 16], [3, 8, 5], 0, 0)))
    check("brute_prefill_window", lambda: brute_prefill((2, 4, 2, 16, "f32", 8, [20, 3], [6, 9], 4, 0)))

    def huge_logits():
        case = workloads.decode_case(12, 1, 1, 1, 4, "f32", block_size=8, max_blocks=8, seq_lens=[50])
        out, c, _ = run(case)
        c.k_cache[...] = 0
        c.q[...] = 1.0
        c.k_cache[c.block_table[0, 2], 1, 0, :] = 1.0  # position 17
        out = orc.paged_decode(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, 1e6, lib=lib)
        return np.array_equal(out[0, 0], brute.to_f64(c.v_cache[c.block_table[0, 2], 1, 0]))
    check("dominant_key", huge_logits)
    return failed


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


def test_unmutated_oracle_passes_battery(orc):
    assert _battery(orc, orc.load()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(orc, source, tmp_path, name):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = orc.load(orc.build(str(src), str(tmp_path / "libmutant.so")))
    failed = _battery(orc, lib)
    assert failed, f"mutant {name} passed every pin"
