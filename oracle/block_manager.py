"""Block-manager oracle: the host-side KV-cache block allocation, written out plainly.

TEST INFRASTRUCTURE ONLY.  Only ``tests/`` may import this module; the native
allocator in the HIP library never calls it and shares no code with it.

It follows the three-layer design of the "KV Cache management design document"
(KV Cache 管理设计文档) page, section by section:

  BlockPool               section 2.4  (FIFO queue of free block ids plus a set for
                                        double-free checks; block 0 is taken first
                                        as the null block)
  SingleTypeManager       section 2.3  (per attention type: req_to_blocks, blocks
                                        to allocate, allocation, skipped-block
                                        removal, free), 2.3.1 FullAttentionManager,
                                        2.3.2 SlidingWindowManager
  KVCacheManager          sections 2.2 and 3 (allocate_slots in two phases:
                                        check every manager, then allocate)
  calculate_block_num_*   section 4.2.1
  prepare_block_table     section 4.2.2
  prepare_slot_mapping    section 4.2.2 with the address map of the
                                        "KVCache optimisation skill" page, section 3.1

Readings where the page leaves a step open (each is used identically by the
native allocator):
  * Skipped blocks, and the null padding of new table entries, follow the tokens
    already computed before a step (the quantity allocate_slots hands to
    remove_skipped_blocks): with c computed tokens a sliding window W skips
    max(0, c - W + 1) tokens, and table entries wholly inside them hold the null
    block.  A fresh prefill (c = 0) therefore gets real blocks for all its tokens,
    and they go back to the pool as the window moves.  The page has a prefill take
    real blocks for the window only; that presumes attention over the step's own
    keys outside the cache, while here every query of a step reads its keys from the
    cache, so each new token needs a real block during its step.  The sizing of
    section 4.2.1 then covers the decode steady state; a pool must also hold the
    longest prompt chunk.
  * remove_skipped_blocks walks the skipped entries from the last one backwards,
    stops at the first null entry (earlier ones were nulled before) and returns the
    blocks to the pool in that order.
  * free returns a request's real blocks in table order.
  * format_usage reports, per type, blocks held by requests / blocks in the pool
    (the null block counts in the total, not in the used figure).
"""
from __future__ import annotations

from collections import deque

FULL, SLIDING = 0, 1
TYPE_NAMES = {FULL: "full", SLIDING: "sliding"}


class AllocError(Exception):
    """A request the pool cannot serve, or a malformed free."""


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class BlockPool:
    """Section 2.4: block ids 0..num_blocks-1 in a FIFO queue; the first one popped
    becomes the null block; get_new_blocks pops from the head, free_blocks appends
    to the tail; a set of free ids catches double frees."""

    def __init__(self, num_blocks: int):
        if num_blocks < 1:
            raise AllocError("a pool needs at least the null block")
        self.num_blocks = num_blocks
        queue = deque(range(num_blocks))
        self.null_block = queue.popleft()
        self.free_queue = queue
        self.free_set = set(queue)

    def num_free(self) -> int:
        return len(self.free_queue)

    def get_new_blocks(self, n: int) -> list:
        if n < 0 or n > len(self.free_queue):
            raise AllocError(f"{n} blocks asked, {len(self.free_queue)} free")
        out = [self.free_queue.popleft() for _ in range(n)]
        for b in out:
            self.free_set.remove(b)
        return out

    def free_blocks(self, blocks) -> None:
        blocks = list(blocks)
        seen = set()
        for b in blocks:  # check all first: a bad call changes nothing
            if not 0 <= b < self.num_blocks or b == self.null_block or b in self.free_set or b in seen:
                raise AllocError(f"block {b} cannot be freed")
            seen.add(b)
        for b in blocks:
            self.free_queue.append(b)
            self.free_set.add(b)


class SingleTypeManager:
    """Section 2.3: the blocks of one attention type."""

    def __init__(self, attn_type: int, num_blocks: int, block_size: int, max_model_len: int,
                 sliding_window: int = 0):
        if attn_type == SLIDING and sliding_window < 1:
            raise AllocError("a sliding-window manager needs a window")
        self.attn_type = attn_type
        self.pool = BlockPool(num_blocks)
        self.block_size = block_size
        self.max_model_len = max_model_len
        self.sliding_window = sliding_window
        self.null_block = self.pool.null_block
        self.req_to_blocks = {}

    def num_skipped_tokens(self, num_computed_tokens: int) -> int:
        """2.3.1: full attention skips nothing; 2.3.2: a window W skips the tokens
        before the next query's window, max(0, computed - W + 1)."""
        if self.attn_type == FULL:
            return 0
        return max(0, num_computed_tokens - self.sliding_window + 1)

    def _skipped_blocks(self, num_computed_tokens: int) -> int:
        return self.num_skipped_tokens(num_computed_tokens) // self.block_size

    def num_blocks_to_allocate(self, req, num_tokens_need_slot: int, num_computed_tokens: int) -> int:
        """Section 3.3.1: ceil(need / bs) table entries minus the ones held; new entries
        wholly inside the skipped tokens take the null block and no pool block."""
        required = _ceil_div(num_tokens_need_slot, self.block_size)
        existing = len(self.req_to_blocks.get(req, []))
        first_real = max(existing, self._skipped_blocks(num_computed_tokens))
        return max(0, required - first_real)

    def allocate_new_blocks(self, req, num_tokens_need_slot: int, num_computed_tokens: int) -> None:
        blocks = self.req_to_blocks.setdefault(req, [])
        required = _ceil_div(num_tokens_need_slot, self.block_size)
        skipped = self._skipped_blocks(num_computed_tokens)
        n_null = max(0, min(required, skipped) - len(blocks))
        blocks.extend([self.null_block] * n_null)
        blocks.extend(self.pool.get_new_blocks(max(0, required - len(blocks))))

    def remove_skipped_blocks(self, req, num_computed_tokens: int) -> None:
        """2.3: entries that slid out of every future window become the null block and
        their blocks go back to the pool."""
        blocks = self.req_to_blocks.get(req)
        if not blocks:
            return
        freed = []
        for i in range(min(self._skipped_blocks(num_computed_tokens), len(blocks)) - 1, -1, -1):
            if blocks[i] == self.null_block:
                break
            freed.append(blocks[i])
            blocks[i] = self.null_block
        self.pool.free_blocks(freed)

    def free(self, req) -> None:
        blocks = self.req_to_blocks.pop(req, [])
        self.pool.free_blocks([b for b in blocks if b != self.null_block])

    def get_block_ids(self, req) -> list:
        return list(self.req_to_blocks.get(req, []))

    def num_used(self) -> int:
        return self.pool.num_blocks - 1 - self.pool.num_free()


class KVCacheManager:
    """Sections 2.2 and 3: one request-level entry over the managers of all types."""

    def __init__(self, groups, block_size: int, max_model_len: int):
        """groups: (attn_type, num_blocks, sliding_window) per attention type."""
        self.block_size = block_size
        self.max_model_len = max_model_len
        self.managers = [SingleTypeManager(t, n, block_size, max_model_len, w) for t, n, w in groups]

    def allocate_slots(self, req, computed_tokens: int, num_new_tokens: int, lookahead_tokens: int = 0) -> bool:
        """Section 3: the pre-check phase (remove skipped blocks, count the blocks
        needed, compare with the free blocks -- any shortfall returns False with no
        block allocated), then the allocation phase."""
        total_computed = min(computed_tokens, self.max_model_len)
        need = min(computed_tokens + num_new_tokens + lookahead_tokens, self.max_model_len)
        for m in self.managers:
            m.remove_skipped_blocks(req, total_computed)
            if m.num_blocks_to_allocate(req, need, total_computed) > m.pool.num_free():
                return False
        for m in self.managers:
            m.allocate_new_blocks(req, need, total_computed)
        return True

    def free(self, req) -> None:
        for m in self.managers:
            m.free(req)

    def get_block_ids(self, req, group: int) -> list:
        return self.managers[group].get_block_ids(req)

    def format_usage(self) -> str:
        return ",".join(f"{TYPE_NAMES[m.attn_type]}:{m.num_used()}/{m.pool.num_blocks}" for m in self.managers)

    def prepare_block_table(self, group: int, reqs, max_blocks_per_seq: int) -> list:
        """Section 4.2.2: one row per request, its table padded with the null block."""
        m = self.managers[group]
        rows = []
        for r in reqs:
            ids = m.get_block_ids(r)
            if len(ids) > max_blocks_per_seq:
                raise AllocError(f"request {r} holds {len(ids)} table entries")
            rows.append(ids + [m.null_block] * (max_blocks_per_seq - len(ids)))
        return rows


def prepare_slot_mapping(block_table, block_size: int, batch_idx, positions) -> list:
    """Section 4.2.2 with the address map: slot = table[b][p / bs] * bs + p % bs."""
    return [block_table[b][p // block_size] * block_size + p % block_size for b, p in zip(batch_idx, positions)]


def calculate_block_num_fixed(max_concurrency: int, sliding_window: int, next_n: int, block_size: int) -> int:
    """Section 4.2.1, fixed-size types (sliding window): every request keeps at most
    the window plus the 2 * next_n tokens of multi-token prediction, one more block
    for a window that straddles a block edge, and the pool one null block."""
    return max_concurrency * (_ceil_div(sliding_window + 2 * next_n, block_size) + 1) + 1


def calculate_block_num_full(max_len: int, max_concurrency: int, block_size: int) -> int:
    """Section 4.2.1, full attention with a fixed maximum length (offline), plus the
    null block."""
    return _ceil_div(max_len, block_size) * max_concurrency + 1


def calculate_block_num_budget(budget_bytes: int, fixed_bytes: int, per_token_bytes: int, block_size: int) -> int:
    """Section 4.2.1, full attention sized by memory (online): the budget left after
    the fixed-size types, in whole tokens, in whole blocks, plus the null block."""
    max_tokens = max(0, budget_bytes - fixed_bytes) // per_token_bytes
    return max_tokens // block_size + 1
