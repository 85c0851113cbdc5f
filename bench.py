#!/usr/bin/env python3
"""Benchmark of the paged-KV-cache hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input, all
on the GPU through the C ABI:
    kv_cache_write_at (the new tokens' slots resolved through the block table
        and their K/V rows scattered into the paged cache, one launch)
    -> paged_attn_decode (split-K decode + combine) / paged_attn_prefill.
Inputs are resident in HBM before the timed region.  Prints ONE JSON line.

Default workload: llama2-7B-shaped single-layer MHA decode (B=64, H=H_kv=32,
d=128, every length 2048, bf16, 1024-block shuffled pool).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix, published
# Cold-cache timing: the timed steps rotate over copies of the step's bulk data
# (the paged cache; for the fused write also its inputs and outputs) until the
# copies together hold at least this much, so that no step finds its bytes in
# the 256 MB last-level cache (MALL) from the step before.  The warm figure (one
# copy, the same bytes every step) is reported beside it.
COLD_SET_BYTES = 2 << 30
METRIC = "paged decode KV GB/s (% of HBM peak) + tokens/s; prefill MFMA util"


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="time this workload alone (default: the llama2-7B decode as the headline, then every "
                         "other configuration of the target list in the 'workloads' map)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--split-tokens", type=int, default=0, help="decode partition size (0 = library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-only", action="store_true",
                    help="time the cold-cache steps only (no warm pass, no copy reference), so that a profiler's "
                         "per-kernel averages cover exactly the reported steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--map-steps", type=int, default=20, help="timed steps of each workload in the map")
    ap.add_argument("--map-cpu-seconds", type=float, default=3.0,
                    help="target oracle time for each map workload's CPU baseline")
    ap.add_argument("--no-map", action="store_true", help="time the headline workload only")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the hot path, time a plain device copy of this many MiB (the reference "
                         "for scaling HBM byte counters)")
    return ap.parse_args()


def time_copy(torch, mib, steps):
    """A plain device copy of `mib` MiB: (ms per copy, read + written bytes per second in GB/s)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del src, dst
    torch.cuda.empty_cache()
    return ms, 2 * n / (ms * 1e-3) / 1e9


def copy_calibration(torch, mib, steps):
    ms, gbs = time_copy(torch, mib, steps)
    n = mib << 20
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 4),
                      "copy_GBps": round(gbs, 1)}), flush=True)


def stream_copy_reference(torch):
    """What a plain streaming copy reaches on this GPU in the same run (1 GiB, read +
    written bytes): the achievable-bandwidth reference beside the 8 TB/s datasheet peak."""
    ms, gbs = time_copy(torch, 1024, 10)
    return {"GBps": round(gbs, 1), "ms": round(ms, 4), "bytes": 2 << 30, "what": "torch device copy of 1 GiB"}


def _nbytes(*ts):
    return sum(t.numel() * t.element_size() for t in ts if t is not None)


def _copies(make, set_bytes):
    """[original, copy, ...]: enough copies of a set of `set_bytes` bytes that together they
    hold at least COLD_SET_BYTES; make(0) is the original, make(i > 0) a fresh copy."""
    n = max(1, -(-COLD_SET_BYTES // max(int(set_bytes), 1)))
    return [make(i) for i in range(n)]


def _dev(torch, a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def algorithmic_bytes(case):
    """Bytes the method must move per step, by call: (resolve, write, attention)."""
    eb = 2 if case.dtype == "bf16" else 4
    L = case.seq_lens.astype(np.int64)
    T = case.new_pos.size
    resolve = T * 16  # batch index, position, table entry, slot
    row = case.Hkv * case.D * eb
    # the write resolves its slots itself (kv_cache_write_at): rows in, rows out
    if case.int8:  # bf16 rows in; codes and one float32 scale per (token, head) out
        stored = case.Hkv * (case.D + 4)
        write = T * 2 * (row + stored)
    else:
        write = T * (2 * row * (1 if case.is_mla else 2) + (2 * case.Hkv * case.rope_dim * eb))
    if case.kind == "decode":
        lo = np.maximum(0, L - case.window) if case.window else np.zeros_like(L)
        keys = L - lo
        blocks = np.where(L > 0, (L - 1) // case.block_size - lo // case.block_size + 1, 0)
        q_rows = case.B * case.H
    else:
        keys = L
        blocks = -(-L // case.block_size)
        q_rows = case.q.shape[0] * case.H
    if case.is_mla:  # latent read once serves as key and value; rope part beside it
        kv = int(keys.sum()) * (case.D + case.rope_dim) * eb
    elif case.int8:  # int8 codes plus a float32 scale per (key, head), K and V
        kv = int(keys.sum()) * case.Hkv * 2 * (case.D + 4)
    else:
        kv = int(keys.sum()) * case.Hkv * 2 * case.D * eb
    qo = q_rows * (case.D + case.rope_dim) * eb + q_rows * case.D * eb
    attn = kv + qo + int(blocks.sum()) * 4 + case.B * 4
    return resolve, write, attn, kv


# Counter-measured HBM bytes per launch of the dominant kernel, kept in the profile
# summary together with a hash of the kernel sources they were taken on.  When the
# sources have changed since, the figure no longer describes the kernel: null.
_CSRC = "paged_kv_cache_80_amd/csrc/"
_COMMON = [_CSRC + f for f in ("api.hip", "pkv_internal.h", "device_common.h", "mfma_common.h")]
_STREAM = [_CSRC + "decode_mfma.hip"] + _COMMON
PROFILED = {
    "mha_decode_7b": ("decode_stream_mha_decode_7b.md", _STREAM),
    "gqa_decode_70b": ("decode_stream_gqa_decode_70b.md", _STREAM),
    "gqa_decode_70b_window4096": ("decode_stream_gqa_decode_70b_window4096.md", _STREAM),
    "chunked_prefill": ("prefill_mfma_chunked_prefill.md", [_CSRC + "prefill.hip"] + _COMMON),
    "gqa_mtp_decode": ("decode_stream_gqa_mtp_decode.md", _STREAM),
    "tiny_f32_decode": ("decode_valu_tiny_f32_decode.md", [_CSRC + "decode.hip"] + _COMMON),
    "mla_decode": ("mla_decode_mla_decode.md", [_CSRC + "mla.hip", _CSRC + "decode.hip"] + _COMMON),
    "mla_mtp_decode": ("mla_decode_mla_mtp_decode.md", [_CSRC + "mla.hip"] + _COMMON),
    "mla_chunked_prefill": ("mla_decode_mla_chunked_prefill.md", [_CSRC + "mla.hip"] + _COMMON),
    "mla_latent_write": ("latent_write_mla_latent_write.md", [_CSRC + "latent_write.hip"] + _COMMON),
    "mha_decode_7b_int8": ("decode_stream_mha_decode_7b_int8.md", _STREAM),
    "gqa_decode_70b_int8": ("decode_stream_gqa_decode_70b_int8.md", _STREAM),
}


def profiled_traffic(workload):
    if workload not in PROFILED:
        return None
    name, sources = PROFILED[workload]
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    import hashlib
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if fields.get("kernel_source_sha256_16") != h.hexdigest()[:16]:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_flops(case):
    """Multiply-adds x 2 of the attention call: q.k over the logit width and p.v over the value
    width, for every (query row, head, visible key)."""
    L = case.seq_lens.astype(np.int64)
    if case.kind == "decode":
        lo = np.maximum(0, L - case.window) if case.window else np.zeros_like(L)
        pairs = int((L - lo).sum()) * case.H
    else:
        cu = case.cu_seqlens_q
        pairs = 0
        for b in range(case.B):
            n = int(cu[b + 1] - cu[b])
            pos = L[b] - n + np.arange(n, dtype=np.int64)
            vis = pos + 1 if not case.window else np.minimum(pos + 1, case.window)
            pairs += int(vis.sum())
        pairs *= case.H
    return pairs * 2 * ((case.D + case.rope_dim) + case.D)


def _int8_oracle_step(oracle, case):
    """The oracle's step over an int8 cache: the pools are quantized and dequantized once
    (the cache as it stands before the step); a step resolves the slots, quantizes the new
    rows into them, refreshes their dequantized values and attends."""
    from helpers import int8_state, oracle_slots, oracle_write_int8, to_f64
    from oracle import int8_cache as q8

    state = int8_state(case)
    kc, ks, vc, vs = state
    kd, vd = q8.dequantize_cache(kc, ks), q8.dequantize_cache(vc, vs)
    q64 = to_f64(case.q, case.dtype)
    bs = case.block_size

    def step(units=None):
        slots = oracle_slots(oracle, case)
        oracle_write_int8(oracle, case, state, slots)
        for sl in slots[slots >= 0]:
            b, o = divmod(int(sl), bs)
            kd[b, o] = q8.dequantize(kc[b, o], ks[b, :, o])
            vd[b, o] = q8.dequantize(vc[b, o], vs[b, :, o])
        oracle.paged_decode(q64, kd, vd, case.block_table, case.seq_lens, case.scale, case.window, units=units)

    return step


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), for the record beside a CPU figure."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, target_s):
    """The oracle, as it stands, on the host cores.  Whole steps of the same workload
    when one fits the time target; otherwise one step whose attention covers a seeded
    random sample of the output rows, scaled to the full step by the row fraction."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from helpers import oracle_run

    oracle.build()
    threads = oracle.max_threads()
    rows = case.q.shape[0] * case.H
    rng = np.random.default_rng(0)
    pilot = np.sort(rng.choice(rows, size=min(rows, 256), replace=False))
    if case.int8:
        step = _int8_oracle_step(oracle, case)
    else:
        def step(units=None):
            oracle_run(oracle, case, units=units, inplace=True)
    t0 = time.perf_counter()
    step(pilot)
    per_row = (time.perf_counter() - t0) / pilot.size
    r, w, a, _ = algorithmic_bytes(case)
    what = "output rows" if case.kind == "decode" else "query-row x head outputs"
    if per_row * rows <= target_s:
        t0 = time.perf_counter()
        step()
        one = time.perf_counter() - t0
        reps = max(1, int(target_s / max(one, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            step()
        el = (time.perf_counter() - t0) / reps
        sample = (f"{reps} whole steps (resolve + write + attention of all {rows} {what}) of "
                  f"{case.name} seed {case.seed_label}, {el * 1e3:.1f} ms per step")
    else:
        n = max(pilot.size, min(rows, int(target_s / per_row)))
        units = np.sort(rng.choice(rows, size=n, replace=False))
        t0 = time.perf_counter()
        step(units)
        el = (time.perf_counter() - t0) * rows / n
        sample = (f"one step of {case.name} seed {case.seed_label} with the attention of {n} of its "
                  f"{rows} {what} (seeded random sample), scaled by the row fraction to "
                  f"{el * 1e3:.1f} ms per step")
    res = {"value": round((r + w + a) / el / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{sample}, fp64, {threads} threads", "ms_per_step": round(el * 1e3, 3), "cpu": cpu_model()}
    if case.name in ("tiny_f32_decode", "mha_decode_7b") and not case.int8:
        # The same oracle on one thread: a seeded sample of rows, scaled to the whole step.
        n1 = min(rows, 64)
        units1 = np.sort(np.random.default_rng(1).choice(rows, size=n1, replace=False))
        t0 = time.perf_counter()
        oracle_run(oracle, case, units=units1, inplace=True, nthreads=1)
        el1 = (time.perf_counter() - t0) * rows / n1
        res["one_thread"] = {"value": round((r + w + a) / el1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                             "sample": f"the attention of {n1} of the {rows} {what} on one thread, scaled by the "
                                       f"row fraction to {el1 * 1e3:.1f} ms per step"}
    return res


def latent_bytes(case):
    """Bytes the fused latent write must move per step, by call: (resolve, fused write)."""
    eb = 2 if case.dtype == "bf16" else 4
    T = case.T
    resolve = T * 16
    row, rope = (512 + 64) * eb, 64 * eb
    write = T * (row + 2 * rope + 4 + row * (2 if case.outputs else 1)) + 512 * eb
    return resolve, write


def cpu_baseline_latent(case, target_s):
    """The latent-write oracle on the host cores: whole steps (slots + RMSNorm + RoPE + write of
    every token), repeated to about the time target."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from helpers import oracle_latent

    oracle.build()
    t0 = time.perf_counter()
    oracle_latent(oracle, case)
    one = time.perf_counter() - t0
    reps = max(1, int(target_s / max(one, 1e-3)))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle_latent(oracle, case)
    el = (time.perf_counter() - t0) / reps
    r, w = latent_bytes(case)
    return {"value": round((r + w) / el / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} whole steps of {case.name} seed {case.seed_label} ({case.T} tokens), fp64 numpy, "
                      f"{el * 1e3:.1f} ms per step, 1 thread", "ms_per_step": round(el * 1e3, 3), "cpu": cpu_model()}


def int8_cache(torch, pkv, case):
    """The workload's bf16 pools quantized into an int8 cache on the GPU by kv_cache_write
    (set-up, before any timing; with a null block, block 0 keeps zero codes and NaN scales)."""
    nb, bs, hkv, d = case.k_cache.shape
    z8 = lambda: torch.zeros((nb, bs, hkv, d), dtype=torch.int8, device="cuda")  # noqa: E731
    zs = lambda: torch.zeros((nb, hkv, bs), dtype=torch.float32, device="cuda")  # noqa: E731
    cache = pkv.PagedKVCache(z8(), z8(), None, zs(), zs())
    slots = torch.arange(nb * bs, dtype=torch.int32, device="cuda")
    if case.null_block:
        slots[:bs] = -1
    pk, pv = _dev(torch, case.k_cache), _dev(torch, case.v_cache)
    pkv.kv_cache_write(slots, pk.view(nb * bs, hkv, d), pv.view(nb * bs, hkv, d), cache)
    if case.null_block:
        cache.k_scale[0] = float("nan")
        cache.v_scale[0] = float("nan")
    torch.cuda.synchronize()
    del pk, pv
    return cache


def run_latent(args, case, torch, pkv):
    """One step = resolve the new tokens' slots, then the fused RMSNorm + RoPE + cache write."""
    dev = lambda a: _dev(torch, a)  # noqa: E731
    cache = pkv.PagedKVCache(dev(case.cache_nope), None, dev(case.cache_rope))
    bt, bidx, pos = dev(case.block_table), dev(case.new_batch_idx), dev(case.new_pos)
    lat, gamma, cos, sin = dev(case.latent), dev(case.gamma), dev(case.cos), dev(case.sin)
    slots = torch.empty(case.T, dtype=torch.int32, device="cuda")
    tdt = lat.dtype
    kn = torch.empty((case.T, 512), dtype=tdt, device="cuda") if case.outputs else None
    kr = torch.empty((case.T, 64), dtype=tdt, device="cuda") if case.outputs else None

    # the bulk data of one step: inputs read, cache and returned rows written
    bulk = (lat, cos, sin, cache.k_cache, cache.k_rope_cache, kn, kr)
    cl = lambda t: None if t is None else t.clone()  # noqa: E731
    sets = _copies(lambda i: bulk if i == 0 else tuple(cl(t) for t in bulk), _nbytes(*bulk))

    def step(i, e0=None, e1=None):
        l_, c_, s_, cn, cr, kn_, kr_ = sets[i % len(sets)]
        pkv.pkv_resolve_slots(bt, case.block_size, bidx, pos, slots_out=slots)
        if e0 is not None:
            e0.record()
        pkv.kv_rmsnorm_rope_cache(l_, gamma, c_, s_, slots, case.eps, pkv.PagedKVCache(cn, None, cr),
                                  rope_layout=case.layout, k_nope_out=kn_, k_rope_out=kr_)
        if e1 is not None:
            e1.record()

    ms_step, ms_k, med_k = _timed(torch, step, args.steps, args.warmup)
    warm = None if args.cold_only else _timed(torch, lambda i, e0=None, e1=None: step(0, e0, e1), args.steps,
                                              args.warmup)
    r_b, w_b = latent_bytes(case)
    value = (r_b + w_b) / (ms_step * 1e-3) / 1e9
    k_gbs = w_b / (ms_k * 1e-3) / 1e9
    result = _result(args, case.name, case.dtype, value, ms_step, {"workload": case.name, "batch": case.B, "tokens": case.T,
                                                  "latent_dim": 512, "rope_dim": 64, "block_size": case.block_size,
                                                  "rope_layout": "half" if case.layout == 0 else "interleaved",
                                                  "returned_rows": case.outputs, "seed": args.seed})
    result.update({"hbm_frac": round(value / HBM_PEAK_GBS, 4), "tokens_per_s": round(case.T / (ms_step * 1e-3), 1),
                   "kernel_ms": round(ms_k, 4), "kernel_ms_median": round(med_k, 4), "kernel_GBps": round(k_gbs, 2),
                   "cold_cache": {"copies": len(sets), "bytes_per_copy": _nbytes(*bulk)}})
    if warm is not None:
        result["warm"] = {"ms_per_step": round(warm[0], 4), "kernel_ms": round(warm[1], 4),
                          "kernel_GBps": round(w_b / (warm[1] * 1e-3) / 1e9, 2)}
        result["stream_copy"] = stream_copy_reference(torch)
    result["roofline"] = {"bound": "hbm", "achieved": round(k_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(args.workload),
                          "kernel": "kv_rmsnorm_rope_cache", "bytes_per_launch": w_b}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_latent(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _timed(torch, step, steps, warmup):
    """W untimed steps, then K timed steps between synchronisations; returns (ms per step,
    mean ms between each step's two events, their median).  step(i, e0, e1) runs step
    number i."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i, (e0, e1) in enumerate(ev):
        step(warmup + i, e0, e1)
    end.record()
    torch.cuda.synchronize()
    per = [e0.elapsed_time(e1) for e0, e1 in ev]
    return start.elapsed_time(end) / steps, float(np.mean(per)), float(np.median(per))


def _result(args, name, dtype, value, ms_step, config):
    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": config,
    }


HEADLINE = "mha_decode_7b"
# Every other configuration of the target list, timed after the headline into the line's
# "workloads" map: the tiny fp32 decode (a latency figure), the llama2-70B ragged GQA decode
# and its window-4096 variant, the chunked prefill and the MLA absorbed decode.
MAP_WORKLOADS = ("tiny_f32_decode", "gqa_decode_70b", "gqa_decode_70b_window4096", "chunked_prefill", "mla_decode")


def read_ceiling(torch):
    """The read bandwidth plain streaming kernels reach on this GPU in the same run: 2 GiB
    (the size of the llama2-7B decode's cache, so that ramp-up weighs the same) read once by
    each kernel of libpkv_probe.so -- 16-byte loads into registers
    (contiguous shares, sixteen in flight per lane, 2 workgroups per CU), and
    global_load_lds DMA into LDS the way the decode kernels stream (four waves per CU,
    16 KiB per step) -- timed with HIP events on the stream they run on.  The faster is the
    attainable reference for the HBM-bound calls beside the 8 TB/s datasheet figure."""
    import ctypes

    path = os.path.join(ROOT, "paged_kv_cache_80_amd", "libpkv_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m paged_kv_cache_80_amd.build`")
    lib = ctypes.CDLL(path)
    lib.pkv_probe_sink_words.argtypes = [ctypes.c_int32]
    lib.pkv_probe_sink_words.restype = ctypes.c_size_t
    lib.pkv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.pkv_probe_stream_read.restype = ctypes.c_int
    lib.pkv_probe_stream_read_lds.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]
    lib.pkv_probe_stream_read_lds.restype = ctypes.c_int
    n = 2 << 30
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(int(lib.pkv_probe_sink_words(2 * cus)), dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()

    def regs():
        return lib.pkv_probe_stream_read(buf.data_ptr(), n, 2 * cus, sink.data_ptr(), st.cuda_stream)

    def dma():
        return lib.pkv_probe_stream_read_lds(buf.data_ptr(), n, cus, st.cuda_stream)

    out = {}
    for name, launch in (("registers", regs), ("lds_dma", dma)):
        for _ in range(3):
            if launch() != 0:
                raise RuntimeError(f"read probe ({name}) launch failed")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(st)
        for _ in range(reps):
            launch()
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"GBps": round(n / (ms * 1e-3) / 1e9, 1), "ms": round(ms, 4)}
    del buf, sink
    torch.cuda.empty_cache()
    best = max(v["GBps"] for v in out.values())
    return {"GBps": best, "bytes": n, **out,
            "what": "read-only streaming kernels over 2 GiB (libpkv_probe.so); GBps is the faster"}


def fused_append(case) -> bool:
    """Decode steps the library runs as one call (paged_attn_decode_append: the bf16
    stream split writes each sequence's newest row inside the decode kernel)."""
    return (case.kind == "decode" and case.dtype == "bf16" and not case.int8 and not case.is_mla
            and case.D == 128 and case.G <= 16)


def measure(args, case, torch, pkv, steps, warmup, cpu_seconds, warm_pass, graph=None, warm_every_copy=False):
    """Time `steps` steps of one workload after `warmup` untimed ones, on cold-cache copies;
    returns the result fields of the JSON line.  A step is the append fused into the decode
    (one call) where the library fuses it, else the write (slots resolved in the writer)
    and then the attention call."""
    dev = lambda a: _dev(torch, a)  # noqa: E731
    if case.int8:
        cache = int8_cache(torch, pkv, case)
    else:
        cache = pkv.PagedKVCache(dev(case.k_cache), dev(case.v_cache), dev(case.k_rope_cache))
    bt, sl = dev(case.block_table), dev(case.seq_lens)
    q, q_rope = dev(case.q), dev(case.q_rope)
    new_k, new_v, new_kr = dev(case.new_k), dev(case.new_v), dev(case.new_k_rope)
    bidx, pos = dev(case.new_batch_idx), dev(case.new_pos)
    slots = torch.empty(case.new_pos.size, dtype=torch.int32, device="cuda")
    out = torch.empty((case.q.shape[0], case.H, case.D), dtype=q.dtype, device="cuda")
    out_code = pkv.PKV_BF16 if case.dtype == "bf16" else pkv.PKV_F32
    if case.kind == "decode":
        ws_bytes = pkv.paged_attn_decode_workspace(cache, case.B, case.H, case.max_blocks, case.scale,
                                                   case.window, out_code, args.split_tokens)
    else:
        ws_bytes = pkv.paged_attn_prefill_workspace(cache, case.B, case.H, case.max_blocks, case.q.shape[0],
                                                    case.scale, case.window, out_code)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    max_q = int(np.diff(case.cu_seqlens_q).max(initial=0)) if case.kind == "prefill" else 1
    cu = dev(case.cu_seqlens_q)

    def attend(c):
        if case.kind == "decode":
            pkv.paged_attn_decode(q, c, bt, sl, case.scale, case.window, q_rope=q_rope, out=out,
                                  split_tokens=args.split_tokens, workspace=ws)
        else:
            pkv.paged_attn_prefill(q, c, bt, cu, sl, max_q, case.scale, case.window, q_rope=q_rope,
                                   out=out, workspace=ws)

    cache_bytes = _nbytes(cache.k_cache, cache.v_cache, cache.k_rope_cache, cache.k_scale, cache.v_scale)
    cl = lambda t: None if t is None else t.clone()  # noqa: E731
    caches = _copies(lambda i: cache if i == 0 else pkv.PagedKVCache(cl(cache.k_cache), cl(cache.v_cache),
                                                                      cl(cache.k_rope_cache), cl(cache.k_scale),
                                                                      cl(cache.v_scale)), cache_bytes)

    fused = fused_append(case)

    def append_attend(c):
        pkv.paged_attn_decode_append(q, new_k, new_v, c, bt, sl, case.scale, case.window, out=out,
                                     split_tokens=args.split_tokens, workspace=ws)

    def step(i, e0=None, e1=None):
        c = caches[i % len(caches)]
        if not fused:
            pkv.kv_cache_write_at(bt, bidx, pos, new_k, new_v, c, k_rope=new_kr, slots_out=slots)
        if e0 is not None:
            e0.record()
        if fused:
            append_attend(c)
        else:
            attend(c)
        if e1 is not None:
            e1.record()

    if warm_every_copy:  # short runs: every cache copy is touched once before the timed steps
        warmup = max(warmup, len(caches))
    ms_step, ms_attn, med_attn = _timed(torch, step, steps, warmup)
    warm = _timed(torch, lambda i, e0=None, e1=None: step(0, e0, e1), steps, warmup) if warm_pass else None
    graph_ms = graph_step_ms(torch, step, steps) if (warm_pass if graph is None else graph) else None

    r_b, w_b, a_b, kv_b = algorithmic_bytes(case)
    flops = algorithmic_flops(case)
    step_bytes = r_b + w_b + a_b
    if fused:  # the timed call is the whole step: its bytes include the append
        a_b = step_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    attn_gbs = a_b / (ms_attn * 1e-3) / 1e9
    attn_tflops = flops / (ms_attn * 1e-3) / 1e12
    kernel = ("paged_attn_decode_append" if fused else "paged_attn_decode") if case.kind == "decode" \
        else "paged_attn_prefill"
    # The bound is the one the call's arithmetic intensity meets first: flops per
    # algorithmic byte against the ridge of 2.5 PFLOP/s over 8 TB/s (312.5 flop/B).
    if flops / a_b >= MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roofline = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(attn_gbs / HBM_PEAK_GBS, 4)}
    roofline.update({"traffic": profiled_traffic(case.name), "kernel": kernel, "bytes_per_launch": a_b,
                     "flops_per_launch": flops})
    res = {"value": value, "ms_per_step": ms_step, "dtype": case.dtype,
           "config": {"workload": case.name, "batch": case.B, "num_q_heads": case.H, "num_kv_heads": case.Hkv,
                      "head_dim": case.D, "rope_dim": case.rope_dim, "block_size": case.block_size,
                      "window": case.window, "seq_len_total": int(case.seq_lens.sum()), "seed": args.seed,
                      "cache": "int8 codes + float32 scale per (token, head)" if case.int8 else case.dtype},
           "hbm_frac": round(value / HBM_PEAK_GBS, 4),
           "tokens_per_s": round(case.new_pos.size / (ms_step * 1e-3), 1),
           "attention_ms": round(ms_attn, 4),
           "attention_ms_median": round(med_attn, 4),
           "attention_GBps": round(attn_gbs, 2),
           "mfma_util": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
           "roofline": roofline,
           "cold_cache": {"copies": len(caches), "bytes_per_copy": cache_bytes}}
    if warm is not None:
        res["warm"] = {"ms_per_step": round(warm[0], 4), "attention_ms": round(warm[1], 4),
                       "attention_GBps": round(a_b / (warm[1] * 1e-3) / 1e9, 2),
                       "mfma_util": round(flops / (warm[1] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    if graph_ms is not None:
        res["graph"] = {"ms_per_step": round(graph_ms, 4), "GBps": round(step_bytes / (graph_ms * 1e-3) / 1e9, 2),
                        "steps": steps, "what": "the same cold-cache steps captured once in a HIP graph and "
                                                "replayed, with no host launch between kernels"}
    if a_b < LATENCY_BYTES:
        res["device_latency"] = backlogged_times(torch, lambda: (append_attend if fused else attend)(caches[0]),
                                                 lambda: step(0))
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(case, cpu_seconds)
    return res


def graph_step_ms(torch, step, steps):
    """ms per step of `steps` consecutive steps (the same rotation over cache copies) captured
    once in a HIP graph and replayed between two events: the step as a serving loop that
    captures its decode step runs it, without the host's launch gaps between kernels.  No
    entry point allocates, synchronises or clears memory, so a step captures."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    g.replay()  # warm-up replay
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del g
    return ms


# Calls that move fewer bytes than this are latency-bound: the eager event pair around the
# call then also holds the host's time to submit it.  Their device time is taken with the
# stream held back: a spin kernel (torch.cuda._sleep, a fixed number of cycles) runs first
# while the host queues `reps` calls behind it, so the two events around those calls see
# only the device executing them back to back.
LATENCY_BYTES = 64 << 20
SPIN_CYCLES = 10_000_000


def backlogged_times(torch, attend_once, step_once, reps=50):
    """Microseconds per call of the attention call alone and of the whole step, each queued
    `reps` times behind a spin kernel and timed between two events.  The spin starts at
    SPIN_CYCLES and is lengthened fourfold (up to three times) while the host needs longer
    to queue the calls than the spin lasts (as under a profiler's tracing); if it never
    does, the figure is null."""
    attend_once()
    step_once()
    torch.cuda.synchronize()
    out = {}
    for name, fn in (("attention_us", attend_once), ("step_us", step_once)):
        cycles, val = SPIN_CYCLES, None
        for _ in range(4):
            s0, e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            s0.record()
            torch.cuda._sleep(cycles)
            e0.record()
            t0 = time.perf_counter()
            for _ in range(reps):
                fn()
            host_ms = (time.perf_counter() - t0) * 1e3
            e1.record()
            torch.cuda.synchronize()
            spin_ms = s0.elapsed_time(e0)
            if spin_ms > 1.2 * host_ms:  # every call was queued before the spin ended
                val = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
                break
            cycles *= 4
        out[name] = val
        out[name.replace("_us", "_spin_ms")] = round(spin_ms, 3)
        out[name.replace("_us", "_host_ms")] = round(host_ms, 3)
    out["reps"] = reps
    out["what"] = "calls queued back to back behind a spin kernel, events around them"
    return out


def map_entry(res, ceiling):
    """The compact record of a workload in the line's "workloads" map."""
    e = {k: res[k] for k in ("config", "attention_ms", "attention_ms_median", "attention_GBps", "mfma_util",
                             "tokens_per_s", "roofline", "cold_cache", "graph", "device_latency", "cpu_baseline")
         if k in res}
    e["ms_per_step"] = round(res["ms_per_step"], 4)
    e["step_GBps"] = round(res["value"], 2)
    if "device_latency" in res:  # latency-bound: a time, not a roofline fraction, is the figure
        e["attention_us"] = res["device_latency"]["attention_us"]
        e["step_us"] = res["device_latency"]["step_us"]
    if ceiling and e["roofline"]["bound"] == "hbm":
        e["roofline"]["frac_of_read_ceiling"] = round(e["roofline"]["achieved"] / ceiling["GBps"], 4)
    return e


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the path runs "
              "unsharded on one device", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_80_amd as pkv
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        copy_calibration(torch, args.copy_calibration_mib, args.steps)
        return
    pkv.load()

    name = args.workload or HEADLINE
    case = workloads.WORKLOADS[name](args.seed)
    case.seed_label = args.seed
    if case.kind == "latent_write":
        run_latent(args, case, torch, pkv)
        return
    res = measure(args, case, torch, pkv, args.steps, args.warmup,
                  0.0 if args.no_cpu_baseline else args.cpu_seconds, not args.cold_only)
    del case
    result = _result(args, res["config"]["workload"], res["dtype"], res["value"], res["ms_per_step"], res["config"])
    result.update({k: v for k, v in res.items() if k not in ("value", "ms_per_step", "config", "dtype")})
    ceiling = None
    if not args.cold_only:
        result["stream_copy"] = stream_copy_reference(torch)
        ceiling = read_ceiling(torch)
        result["read_ceiling"] = ceiling
        if result["roofline"]["bound"] == "hbm":
            result["roofline"]["frac_of_read_ceiling"] = round(result["roofline"]["achieved"] / ceiling["GBps"], 4)
    if args.workload is None and not args.no_map:
        wl = {}
        for other in MAP_WORKLOADS:
            print(f"bench: {other}", file=sys.stderr, flush=True)
            c = workloads.WORKLOADS[other](args.seed)
            c.seed_label = args.seed
            r = measure(args, c, torch, pkv, args.map_steps, 3,
                        0.0 if args.no_cpu_baseline else args.map_cpu_seconds, False, graph=True,
                        warm_every_copy=True)
            del c
            torch.cuda.empty_cache()
            wl[other] = map_entry(r, ceiling)
        result["workloads"] = wl
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
