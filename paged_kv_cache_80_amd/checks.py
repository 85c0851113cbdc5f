"""Host-side bounds checks of the device index arrays an entry point is about to read.

The C ABI validates host-visible arguments only and trusts the contents of
block_table, seq_lens, cu_seqlens_q and slot_mapping: an id outside the pool is
undefined behaviour there, as in any kernel that takes raw indices.  The page on
KV-cache management motivates a checked mode -- the pool keeps a null block so
that operators always see a legal index, and its free list rejects a double
free -- so the binding offers one: with ``set_check_indices(True)`` every entry
point copies these arrays to the host first (a synchronising device-to-host
copy) and raises ``PkvError(PKV_ERR_INVALID_ARG)`` naming the first bad entry,
before anything is launched.

The rules are exactly what the kernels dereference (include/pkv.h): only the
table entries of blocks that hold a key some query can see must be valid block
ids; entries before a window or past a sequence's last block may hold anything.
Each function takes numpy arrays or torch tensors on any device.
"""
from __future__ import annotations

import numpy as np

INT32_MAX = 2**31 - 1


class IndexCheckError(ValueError):
    """A device index array holds an entry the kernels would read out of bounds."""


def _host(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.asarray(a)


def _fail(msg: str):
    raise IndexCheckError(msg)


def _visible_blocks(table_row: np.ndarray, lo: int, hi: int, bs: int, num_blocks: int, what: str) -> None:
    """Every entry of the blocks holding keys [lo, hi) must be a block id of the pool."""
    if hi <= lo:
        return
    ids = table_row[lo // bs:(hi - 1) // bs + 1]
    bad = np.flatnonzero((ids < 0) | (ids >= num_blocks))
    if bad.size:
        i = lo // bs + int(bad[0])
        _fail(f"{what}: block_table entry {i} = {int(table_row[i])} is not a block id of the "
              f"{num_blocks}-block pool, and it holds visible keys")


def check_slots(slot_mapping, num_slots: int) -> None:
    """kv_cache_write: every non-negative slot lies in the cache, and no slot repeats."""
    s = _host(slot_mapping).astype(np.int64).ravel()
    over = np.flatnonzero(s >= num_slots)
    if over.size:
        _fail(f"slot_mapping[{int(over[0])}] = {int(s[over[0]])} is past the cache's {num_slots} slots")
    live = s[s >= 0]
    if np.unique(live).size != live.size:
        vals, counts = np.unique(live, return_counts=True)
        _fail(f"slot {int(vals[counts > 1][0])} is written twice in one call")


def check_resolve(block_table, block_size: int, batch_idx, pos, num_blocks: int | None = None) -> None:
    """pkv_resolve_slots: every (batch_idx, pos >= 0) names a table entry that is a block id."""
    bt = _host(block_table)
    b = _host(batch_idx).astype(np.int64).ravel()
    p = _host(pos).astype(np.int64).ravel()
    B, mb = bt.shape
    live = p >= 0
    bad = np.flatnonzero(live & ((b < 0) | (b >= B)))
    if bad.size:
        _fail(f"batch_idx[{int(bad[0])}] = {int(b[bad[0]])} is outside the {B} table rows")
    bad = np.flatnonzero(live & (p >= mb * block_size))
    if bad.size:
        _fail(f"pos[{int(bad[0])}] = {int(p[bad[0]])} is past the {mb * block_size} positions of a table row")
    ids = bt[b[live], p[live] // block_size].astype(np.int64)
    limit = num_blocks if num_blocks is not None else (INT32_MAX - block_size) // block_size + 1
    bad = np.flatnonzero((ids < 0) | (ids >= limit))
    if bad.size:
        i = int(np.flatnonzero(live)[bad[0]])
        _fail(f"position {int(p[i])} of sequence {int(b[i])} resolves through block id {int(ids[bad[0]])}, "
              f"not one of {limit}")


def check_write_at(block_table, block_size: int, batch_idx, pos, num_blocks: int) -> None:
    """kv_cache_write_at: every (batch_idx, pos >= 0) resolves through a pool block id, and the
    resolved slots are distinct."""
    check_resolve(block_table, block_size, batch_idx, pos, num_blocks)
    bt = _host(block_table).astype(np.int64)
    b = _host(batch_idx).astype(np.int64).ravel()
    p = _host(pos).astype(np.int64).ravel()
    live = p >= 0
    slots = np.full(p.shape, -1, dtype=np.int64)
    slots[live] = bt[b[live], p[live] // block_size] * block_size + p[live] % block_size
    check_slots(slots, num_blocks * block_size)


def check_decode(block_table, seq_lens, block_size: int, num_blocks: int, window: int = 0) -> None:
    """paged_attn_decode: 0 <= seq_lens[b] <= table width, and the blocks of the visible keys
    [max(0, L - W), L) hold valid ids."""
    bt = _host(block_table)
    L = _host(seq_lens).astype(np.int64).ravel()
    B, mb = bt.shape
    for b in range(B):
        if L[b] < 0 or L[b] > mb * block_size:
            _fail(f"seq_lens[{b}] = {int(L[b])} is outside [0, {mb * block_size}] (the table width)")
        lo = max(0, int(L[b]) - window) if window > 0 else 0
        _visible_blocks(bt[b], lo, int(L[b]), block_size, num_blocks, f"sequence {b}")


def check_append(block_table, seq_lens, block_size: int, num_blocks: int, window: int = 0) -> None:
    """paged_attn_decode_append: the decode's rules, and the newest slots (position
    seq_lens[b] - 1 of every non-empty sequence) are distinct."""
    check_decode(block_table, seq_lens, block_size, num_blocks, window)
    bt = _host(block_table).astype(np.int64)
    L = _host(seq_lens).astype(np.int64).ravel()
    live = np.flatnonzero(L > 0)
    p = L[live] - 1
    slots = bt[live, p // block_size] * block_size + p % block_size
    check_slots(slots, num_blocks * block_size)


def check_prefill(block_table, cu_seqlens_q, seq_lens_kv, total_q: int, max_q_len: int, block_size: int,
                  num_blocks: int, window: int = 0) -> None:
    """paged_attn_prefill: cu_seqlens_q starts at 0, never decreases and ends at total_q;
    every n_b is at most max_q_len and at most seq_lens_kv[b]; seq_lens_kv fits the table;
    the blocks of every key some new row sees hold valid ids."""
    bt = _host(block_table)
    cu = _host(cu_seqlens_q).astype(np.int64).ravel()
    L = _host(seq_lens_kv).astype(np.int64).ravel()
    B, mb = bt.shape
    if cu.size != B + 1 or cu[0] != 0 or cu[-1] != total_q:
        _fail(f"cu_seqlens_q must run from 0 to total_q = {total_q} over {B + 1} entries")
    n = np.diff(cu)
    for b in range(B):
        if n[b] < 0:
            _fail(f"cu_seqlens_q decreases at sequence {b}")
        if n[b] > max_q_len:
            _fail(f"sequence {b} has {int(n[b])} query rows, more than max_q_len = {max_q_len}")
        if L[b] < n[b] or L[b] > mb * block_size:
            _fail(f"seq_lens_kv[{b}] = {int(L[b])} is outside [{int(n[b])}, {mb * block_size}]")
        if n[b] == 0:
            continue
        first = int(L[b] - n[b])  # position of the first new row
        lo = max(0, first - window + 1) if window > 0 else 0
        _visible_blocks(bt[b], lo, int(L[b]), block_size, num_blocks, f"sequence {b}")
