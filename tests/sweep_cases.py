"""Seeded random shapes for the parity sweeps (tests/test_random_sweeps.py): tiny ones for
the oracle against the brute force on the CPU, small ones within the kernels' supported
set for the GPU.  Each draw names its case, so a failure says which one."""
from __future__ import annotations

import numpy as np

import workloads


def _lens(rng, B, max_len, allow_empty=True):
    lens = rng.integers(0 if allow_empty else 1, max_len + 1, size=B)
    if allow_empty and B > 1 and rng.random() < 0.3:
        lens[rng.integers(0, B)] = 0  # an empty sequence now and then
    return lens.astype(np.int32)


def _window(rng, max_len):
    r = rng.random()
    if r < 0.35:
        return 0
    if r < 0.5:
        return 1
    if r < 0.65:
        return int(max_len + rng.integers(0, 5))  # a window that covers every key
    return int(rng.integers(1, max(2, max_len)))


def tiny_decode(i: int):
    """CPU sweep: bs in {4, 16, 128}, MHA/GQA/MQA/MLA, windows (>= L included), L = 0."""
    rng = np.random.default_rng(1000 + i)
    bs = int(rng.choice([4, 16, 128]))
    B = int(rng.integers(1, 6))
    mla = rng.random() < 0.25
    Hkv = 1 if mla else int(rng.choice([1, 2, 3]))
    H = Hkv * int(rng.choice([1, 2, 4]))
    D = int(rng.choice([8, 16, 32]))
    rope = int(rng.choice([4, 8])) if mla else 0
    mb = int(rng.integers(1, 4)) if bs == 128 else int(rng.integers(1, 10))
    max_len = mb * bs if bs < 128 else min(mb * bs, 160)
    lens = _lens(rng, B, max_len)
    W = _window(rng, int(lens.max(initial=1)))
    dt = str(rng.choice(["f32", "bf16"]))
    name = f"tiny decode #{i}: B={B} H={H} Hkv={Hkv} D={D} rope={rope} bs={bs} mb={mb} W={W} {dt} L={lens.tolist()}"
    case = workloads.decode_case(2000 + i, B, H, Hkv, D, dt, block_size=bs, max_blocks=mb, seq_lens=lens,
                                 window=W, null_block=True, rope_dim=rope,
                                 spare_frac=float(rng.choice([0.0, 0.1, 0.5])))
    return name, case


def tiny_prefill(i: int):
    rng = np.random.default_rng(3000 + i)
    bs = int(rng.choice([4, 16, 128]))
    B = int(rng.integers(1, 4))
    mla = rng.random() < 0.25
    Hkv = 1 if mla else int(rng.choice([1, 2]))
    H = Hkv * int(rng.choice([1, 2, 4]))
    D = int(rng.choice([8, 16]))
    rope = 4 if mla else 0
    cached = rng.integers(0, 40, size=B)
    new = rng.integers(0, 12, size=B)
    W = _window(rng, int((cached + new).max(initial=1)))
    dt = str(rng.choice(["f32", "bf16"]))
    name = (f"tiny prefill #{i}: B={B} H={H} Hkv={Hkv} D={D} rope={rope} bs={bs} W={W} {dt} "
            f"cached={cached.tolist()} new={new.tolist()}")
    case = workloads.prefill_case(4000 + i, B, H, Hkv, D, dt, cached=cached, new=new, block_size=bs,
                                  window=W, rope_dim=rope, null_block=True)
    return name, case


def gpu_case(i: int):
    """GPU sweep: a small decode (bf16 stream, fp32 / other head widths, int8), chunked
    prefill or MLA call with random lengths, windows, block sizes and tables."""
    rng = np.random.default_rng(5000 + i)
    kind = ["decode", "decode", "prefill", "mla", "mla_prefill", "int8"][i % 6]
    bs = int(rng.choice([16, 32, 64, 128]))
    if kind in ("decode", "int8"):
        if kind == "int8":
            dt, D = "bf16", 128
        else:
            dt, D = [("bf16", 128), ("bf16", 128), ("f32", 128), ("bf16", 64), ("f32", 256)][int(rng.integers(0, 5))]
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        if D == 256:
            G = min(G, 8)  # the vector-ALU kernel holds at most 2048 query values per lane group
        B = int(rng.integers(1, 40))
        mb = int(rng.integers(1, 2048 // bs + 2))
        lens = _lens(rng, B, mb * bs)
        W = _window(rng, int(lens.max(initial=1)))
        name = f"gpu {kind} #{i}: B={B} H={Hkv * G} Hkv={Hkv} D={D} {dt} bs={bs} mb={mb} W={W}"
        case = workloads.decode_case(6000 + i, B, Hkv * G, Hkv, D, dt, block_size=bs, max_blocks=mb, seq_lens=lens,
                                     window=W, null_block=True, int8=kind == "int8")
        return name, case, int(rng.choice([0, 0, 2])) * bs
    if kind == "mla":
        H = 16 * int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 12))
        mb = int(rng.integers(1, 1024 // bs + 2))
        lens = _lens(rng, B, mb * bs)
        W = _window(rng, int(lens.max(initial=1)))
        name = f"gpu mla #{i}: B={B} H={H} bs={bs} mb={mb} W={W}"
        case = workloads.decode_case(6000 + i, B, H, 1, 512, "bf16", block_size=bs, max_blocks=mb, seq_lens=lens,
                                     window=W, null_block=True, rope_dim=64)
        return name, case, int(rng.choice([0, 0, 2])) * bs
    B = int(rng.integers(1, 5))
    cached = rng.integers(0, 700, size=B)
    if kind == "mla_prefill":
        H, Hkv, D, rope = 16 * int(rng.choice([1, 2, 4])), 1, 512, 64
        new = rng.integers(0, 9, size=B)
    else:
        Hkv = int(rng.choice([1, 2, 4]))
        H, D, rope = Hkv * int(rng.choice([1, 2, 4, 8])), int(rng.choice([64, 128])), 0
        new = rng.integers(0, 200, size=B)
    W = _window(rng, int((cached + new).max(initial=1)))
    name = f"gpu {kind} #{i}: B={B} H={H} Hkv={Hkv} D={D} bs={bs} W={W} cached={cached.tolist()} new={new.tolist()}"
    case = workloads.prefill_case(6000 + i, B, H, Hkv, D, "bf16", cached=cached, new=new, block_size=bs,
                                  window=W, rope_dim=rope, null_block=True)
    return name, case, 0
