/*
 * pkv_blocks.h -- host-side KV-cache block allocation (part of libpkv.so, plain C ABI).
 *
 * The allocator produces the block tables and slot mappings the attention entry
 * points of pkv.h consume.  It follows the three-layer design of the "KV Cache
 * management design document" page:
 *   - a block pool per attention type (section 2.4): block ids 0..num_blocks-1 in a
 *     FIFO queue; the first id taken, 0, is the null block, never issued, which fills
 *     the table entries that hold no data; freed blocks go back to the tail; a free
 *     set rejects double frees;
 *   - one manager per attention type (section 2.3): full attention keeps
 *     ceil(tokens / block_size) blocks per request; a sliding window W also turns the
 *     table entries wholly before the next query's window (the first
 *     max(0, computed - W + 1) tokens) into the null block and frees their blocks,
 *     so a table stays ceil(tokens / block_size) long while holding only the window;
 *   - a request-level manager (sections 2.2 and 3) whose allocate_slots checks every
 *     type before allocating anything.
 *
 * Everything here runs on the host and touches no device memory; tables are host
 * int32 arrays the caller copies to the device.  Objects are not thread-safe: one
 * caller at a time per object.  Every function returns a pkv_status; messages go to
 * pkv_last_error().
 */
#ifndef PKV_BLOCKS_H
#define PKV_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_ATTN_FULL = 0, PKV_ATTN_SLIDING = 1 } pkv_attn_type;

/* ---- block pool ("KV Cache management design document", section 2.4) ---------- */

typedef struct pkv_block_pool pkv_block_pool;

/* A pool of num_blocks >= 1 ids; id 0 becomes the null block.  *out owns the pool. */
pkv_status pkv_pool_create(int32_t num_blocks, pkv_block_pool** out);
void pkv_pool_destroy(pkv_block_pool* pool);
/* Free ids (never counting the null block) into *count. */
pkv_status pkv_pool_num_free(const pkv_block_pool* pool, int32_t* count);
/* Pop n ids from the head of the free queue into ids[0..n).  Fewer than n free:
 * PKV_ERR_INVALID_ARG, nothing popped. */
pkv_status pkv_pool_get_new_blocks(pkv_block_pool* pool, int32_t n, int32_t* ids);
/* Append ids[0..n) to the tail of the free queue, in order.  An id out of range, the
 * null block, an id already free or repeated in the list: PKV_ERR_INVALID_ARG and the
 * pool is left unchanged. */
pkv_status pkv_pool_free_blocks(pkv_block_pool* pool, const int32_t* ids, int32_t n);

/* ---- request-level manager (sections 2.2, 2.3 and 3) ------------------------------ */

typedef struct pkv_kv_manager pkv_kv_manager;

typedef struct {
  int32_t attn_type;      /* pkv_attn_type                                     */
  int32_t num_blocks;     /* pool size of this type, null block included (>= 1) */
  int32_t sliding_window; /* W >= 1 for PKV_ATTN_SLIDING, ignored otherwise      */
} pkv_attn_group;

/* One manager and one pool per group, all with the same block_size (> 0) and a
 * request length limit max_model_len (> 0). */
pkv_status pkv_kvm_create(const pkv_attn_group* groups, int32_t num_groups, int32_t block_size,
                          int32_t max_model_len, pkv_kv_manager** out);
void pkv_kvm_destroy(pkv_kv_manager* m);

/* Make request request_id's tables cover computed_tokens + num_new_tokens +
 * lookahead_tokens tokens (capped at max_model_len), section 3:
 *   phase 1, for every group: drop the blocks that slid out of the window of the
 *   next query (computed_tokens already computed), count the new table entries that
 *   need a real block; if any group has fewer free blocks, *allocated = 0 and no
 *   block is taken anywhere (the dropped blocks stay dropped);
 *   phase 2: extend every table, entries wholly before the window with the null
 *   block, the others with blocks from the pool in FIFO order; *allocated = 1.
 * A new request_id starts an empty table.  Counts must be >= 0. */
pkv_status pkv_kvm_allocate_slots(pkv_kv_manager* m, int64_t request_id, int32_t computed_tokens,
                                  int32_t num_new_tokens, int32_t lookahead_tokens, int32_t* allocated);
/* Return every real block of the request to its pool (in table order) and forget it.
 * An unknown request is a no-op. */
pkv_status pkv_kvm_free(pkv_kv_manager* m, int64_t request_id);
/* Table of the request in group `group`: its length into *count and, when ids is not
 * NULL, the first min(count, capacity) entries into ids.  Unknown request: count 0. */
pkv_status pkv_kvm_get_block_ids(const pkv_kv_manager* m, int64_t request_id, int32_t group,
                                 int32_t* ids, int32_t capacity, int32_t* count);
pkv_status pkv_kvm_num_free_blocks(const pkv_kv_manager* m, int32_t group, int32_t* count);
/* "full:12/100,sliding:8/100": per group, blocks held by requests / pool size.  The
 * string (with its terminator) must fit in capacity bytes. */
pkv_status pkv_kvm_format_usage(const pkv_kv_manager* m, char* buf, size_t capacity);
/* Section 4.2.2: table[batch][max_blocks_per_seq] (host, row-major) with the table of
 * request_ids[b] in row b, padded with the null block.  A table longer than
 * max_blocks_per_seq: PKV_ERR_INVALID_ARG, nothing written. */
pkv_status pkv_kvm_prepare_block_table(const pkv_kv_manager* m, int32_t group, const int64_t* request_ids,
                                       int32_t batch, int32_t max_blocks_per_seq, int32_t* table);

/* ---- sizing (section 4.2.1); each result counts the null block --------------------- */

/* Sliding window: max_concurrency * (ceil((W + 2 next_n) / block_size) + 1) + 1.
 * This covers the decode steady state.  A fresh prompt chunk of P tokens takes a
 * real block for every one of its tokens during its step (each new query reads its
 * keys from the cache, so all of the chunk is written first), i.e.
 * ceil((P + 2 next_n) / block_size) blocks, and only the next step returns the ones
 * before the window.  A pool that admits one such chunk at a time therefore needs
 * this figure plus max(0, ceil((P + 2 next_n) / block_size) - peak) blocks, peak =
 * ceil((W + 2 next_n - 1) / block_size) + 1 being the most blocks a window touches;
 * several chunks in flight need that excess once per chunk. */
pkv_status pkv_block_num_fixed(int32_t max_concurrency, int32_t sliding_window, int32_t next_n,
                               int32_t block_size, int64_t* num_blocks);
/* Full attention, fixed maximum length: ceil(max_len / block_size) * max_concurrency + 1. */
pkv_status pkv_block_num_full(int32_t max_len, int32_t max_concurrency, int32_t block_size, int64_t* num_blocks);
/* Full attention sized by memory: floor(floor((budget - fixed) / per_token) / block_size) + 1,
 * budget_bytes being the cache memory share and fixed_bytes what the fixed-size types take. */
pkv_status pkv_block_num_budget(int64_t budget_bytes, int64_t fixed_bytes, int64_t per_token_bytes,
                                int32_t block_size, int64_t* num_blocks);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCKS_H */
