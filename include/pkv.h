/*
 * pkv.h -- C ABI of the MI355X (gfx950) paged-KV-cache attention library (libpkv.so).
 *
 * The cache of one layer is stored in fixed-size blocks:
 *     k_cache, v_cache : [num_blocks, block_size, num_kv_heads, head_dim]
 * and a logical (sequence b, position p) lives at the physical slot
 *     block_table[b][p / block_size] * block_size + p % block_size
 * (the layout and address map of the "KVCache optimisation skill" page,
 * mode 2 and section 3.1, and of the "Ascend NPU standalone-deployment
 * KVCache guide", mode 2).
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers to dense row-major arrays that the
 *     caller owns.  The library never allocates, frees or synchronises; it
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the default stream)
 *     and returns.  Scratch memory comes from the caller as `workspace`.
 *   - Index arrays (block_table, slot_mapping, seq_lens, cu_seqlens_q,
 *     batch_idx, pos) are int32 (the skill page's notes require an int32
 *     block table).
 *   - Element arrays are float32 or bfloat16, one dtype per call; there is no
 *     implicit conversion.  The one exception is an int8 cache (PKV_INT8),
 *     whose codes and float32 scales go with bf16 queries, rows and outputs.
 *     Every element base pointer must be 16-byte aligned.
 *   - Only host-visible arguments are validated (pointers, sizes, shapes,
 *     dtypes, scale, workspace size).  A failed check returns a non-zero
 *     status, launches nothing and leaves a message for pkv_last_error().
 *     The CONTENTS of device index arrays are trusted: a block id outside
 *     [0, num_blocks), a sequence length beyond max_blocks_per_seq *
 *     block_size or a slot outside the cache is undefined behaviour.  The
 *     Python binding can check them on the host before each launch (its
 *     set_check_indices switch), at the cost of a device-to-host copy.
 *   - Slots are int32: a cache with num_blocks * block_size above INT32_MAX is
 *     refused (PKV_ERR_UNSUPPORTED).
 *   - Launch failures return PKV_ERR_HIP.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1, /* a host-visible argument is malformed                 */
  PKV_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels implement  */
  PKV_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the *_workspace size  */
  PKV_ERR_HIP = 4          /* a HIP launch or runtime call failed                  */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_INT8 = 2 } pkv_dtype;

/* One layer's paged cache.  Standard attention: k_cache and v_cache of width
 * head_dim, k_rope_cache NULL, rope_dim 0.  MLA absorbed form ("KVCache
 * optimisation skill", mode 3): k_cache holds the latent (cache_nope, width
 * head_dim = kv_lora_rank = 512), v_cache must be the SAME pointer (key =
 * value = cache_nope), k_rope_cache holds the rotary part (cache_rope,
 * [num_blocks, block_size, 1, rope_dim] with rope_dim = 64) and
 * num_kv_heads = 1 -- the constraints that page lists for this mode.
 *
 * INT8 cache (dtype PKV_INT8; the cache quantization the "KV Cache notes"
 * quantized-cache section and the skill page's advanced features name, which
 * halves the bytes decode reads): k_cache / v_cache hold int8 codes in the same
 * [num_blocks, block_size, num_kv_heads, head_dim] layout and k_scale / v_scale
 * hold one float32 scale per (slot, head) in [num_blocks, num_kv_heads,
 * block_size] order (the scales of consecutive keys of a head are adjacent).  A
 * row x of one token and head is stored as s = max|x| / 127 and codes
 * q = round_half_even(x * (127 / max|x|)) (float32 arithmetic; an all-zero row has
 * s = 0, q = 0) and stands for q * s.  Queries, new rows and outputs stay bf16.
 * Standard attention only (no rope part), head_dim 128; kv_cache_write quantizes,
 * paged_attn_decode reads it (head groups up to 16); prefill does not take it.
 *
 * Every cache: a slot row (num_kv_heads * head_dim elements, and the rope row)
 * is a multiple of 16 bytes and at most 16 MiB; else PKV_ERR_UNSUPPORTED. */
typedef struct {
  void* k_cache;
  void* v_cache;
  void* k_rope_cache;
  int32_t num_blocks;
  int32_t block_size;   /* tokens per block: 16, 32, 64 or 128                       */
  int32_t num_kv_heads;
  int32_t head_dim;     /* 64, 128 or 256; 512 for MLA                                */
  int32_t rope_dim;     /* 0, or 64 for MLA                                           */
  int32_t dtype;        /* pkv_dtype of every cache tensor and of q / k / v / q_rope; */
                        /* PKV_INT8: int8 caches, bf16 q / k / v                    */
  void* k_scale;        /* PKV_INT8: float32 [num_blocks, num_kv_heads, block_size]; else NULL */
  void* v_scale;
} pkv_paged_cache;

/* Attention parameters.  There are no defaults: a zero or negative scale is an
 * error (the Ascend guide's FA v1/v2 name table warns that a misnamed scale
 * silently becomes 1.0). */
typedef struct {
  int32_t batch;              /* number of sequences B                                       */
  int32_t num_q_heads;        /* H; H % num_kv_heads == 0; query head h reads KV head h / (H / H_kv) */
  int32_t max_blocks_per_seq; /* row stride of block_table                                   */
  float scale;                /* softmax scale, finite and > 0 (1/sqrt(d) in the pages)      */
  int32_t window;             /* 0 = full attention; W > 0: a query at position p sees keys  */
                              /* p-W < j <= p ("KV Cache notes", sliding-window section)     */
  int32_t out_dtype;          /* pkv_dtype of `out` (f32 out is a diagnostic mode)           */
  int32_t split_tokens;       /* decode only, a multiple of block_size; 0 = library choice   */
                              /* (which for small f32 / head_dim != 128 calls may be one     */
                              /* workgroup per whole sequence, needing no workspace).        */
                              /* Partition kernels (f32, head_dim != 128, MLA): keys per     */
                              /* workgroup partition.  Stream-split kernel (bf16, head_dim   */
                              /* 128): the fewest keys one wave group streams, which caps    */
                              /* the number of groups sharing the work.  Results do not      */
                              /* depend on it beyond fp32 summation order.                   */
} pkv_attn_params;

/* slots_out[i] = block_table[batch_idx[i]][pos[i] / block_size] * block_size + pos[i] % block_size
 * for i < n ("KVCache optimisation skill", section 3.1; the framework's
 * prepare_slot_mapping of the KV Cache management design document).
 * block_table: [batch, max_blocks_per_seq]; batch_idx, pos, slots_out: [n].
 * A negative pos gives slot -1 (a row kv_cache_write skips).  The arithmetic is
 * int32: every block id read must keep id * block_size + block_size <= INT32_MAX,
 * which holds for any id below the num_blocks of a cache the other entry points
 * accept. */
pkv_status pkv_resolve_slots(const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                             int32_t block_size, const int32_t* batch_idx, const int32_t* pos,
                             int32_t n, int32_t* slots_out, void* stream);

/* The same resolution without the batch count (the row stride alone addresses
 * block_table): slots_out[i] for i < n exactly as pkv_resolve_slots computes it.
 * Same errors, except that there is no batch to check. */
pkv_status paged_resolve_slots(const int32_t* block_table, int32_t max_blocks_per_seq, int32_t block_size,
                               const int32_t* batch_idx, const int32_t* pos, int32_t n, int32_t* slots_out,
                               void* stream);

/* Cache write ("Ascend NPU standalone-deployment KVCache guide", mode 2: the
 * scatter into the cache viewed as [num_blocks*block_size, num_kv_heads, head_dim]).
 * Row t of k (and v, and k_rope) is copied bit for bit to cache row slot_mapping[t];
 * into a PKV_INT8 cache each (token, head) row of the bf16 k and v is quantized
 * instead (codes to the row, scale to the scale arrays).
 *   slot_mapping : [num_tokens]; a negative slot skips the row.  Slots must be distinct.
 *   k, v         : [num_tokens, num_kv_heads, head_dim]; v must be NULL when
 *                  cache->v_cache == cache->k_cache (MLA latent written once)
 *   k_rope       : [num_tokens, num_kv_heads, rope_dim] iff cache->rope_dim > 0, else NULL */
pkv_status kv_cache_write(const int32_t* slot_mapping, int32_t num_tokens, const void* k,
                          const void* v, const void* k_rope, const pkv_paged_cache* cache,
                          void* stream);

/* Index resolution and cache write in one launch: row t goes to the slot of
 * (batch_idx[t], pos[t]), resolved through block_table exactly as
 * pkv_resolve_slots does it ("KVCache optimisation skill", section 3.1), and is
 * written exactly as kv_cache_write writes it (the guide's mode-2 scatter;
 * quantized into a PKV_INT8 cache).  A negative pos skips the row.  When slots_out
 * is not NULL it receives the resolved slots ([num_tokens], -1 for skipped rows),
 * the slot_mapping kv_cache_write would have taken.
 *   block_table : [batch, max_blocks_per_seq]; batch_idx, pos: [num_tokens]
 *   k, v, k_rope: as for kv_cache_write.  The resolved slots must be distinct.
 * Same errors as kv_cache_write, plus NULL index arrays or max_blocks_per_seq <= 0;
 * the same int32 range rule for block ids as pkv_resolve_slots. */
pkv_status kv_cache_write_at(const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* batch_idx,
                             const int32_t* pos, int32_t num_tokens, const void* k, const void* v,
                             const void* k_rope, const pkv_paged_cache* cache, int32_t* slots_out, void* stream);

typedef enum {
  PKV_ROPE_HALF = 0,       /* element i pairs with i + rope_dim/2 (the first half with the second) */
  PKV_ROPE_INTERLEAVED = 1 /* elements 2k and 2k+1 form a pair                                  */
} pkv_rope_layout;

/* Fused RMSNorm + RoPE + cache write of the MLA latent ("Ascend NPU
 * standalone-deployment KVCache guide", MLA section: the single fused step that
 * normalises, rotates and writes the latent and can also return the rows; the
 * "KVCache optimisation skill" page lists it as the slot_mapping-driven fused
 * writer).  For each token t < num_tokens, with latent row t = [c | k_pe]
 * (c: head_dim = 512 values, k_pe: rope_dim = 64 values):
 *     nope = c / sqrt(mean(c * c) + eps) * gamma                    (fp32 arithmetic)
 *     rope[i] = k_pe[i] * cos[t][i] -/+ k_pe[j] * sin[t][i]          (j: i's pair partner;
 *               minus for the first element of the pair, plus for the second)
 *     cache->k_cache row slot_mapping[t] = nope, cache->k_rope_cache row = rope
 *     (a negative slot writes nothing), and k_nope_out[t] = nope, k_rope_out[t] = rope
 *     when the outputs are given.
 *   cache        : an MLA cache (latent 512, rope 64, one head, v_cache == k_cache), f32 or bf16
 *   latent       : [num_tokens, 512 + 64]; gamma: [512]; cos, sin: [num_tokens, 64], the
 *                  values at each token's position; all in cache->dtype
 *   rope_layout  : pkv_rope_layout
 *   eps          : finite, >= 0
 *   k_nope_out   : [num_tokens, 512] and k_rope_out [num_tokens, 64] in cache->dtype, both or
 *                  neither (NULL)
 *   slot_mapping : [num_tokens]; slots must be distinct.
 * The outputs and the cache must not overlap the inputs. */
pkv_status kv_rmsnorm_rope_cache(const void* latent, const void* gamma, const void* cos, const void* sin,
                                 const int32_t* slot_mapping, int32_t num_tokens, float eps,
                                 int32_t rope_layout, const pkv_paged_cache* cache, void* k_nope_out,
                                 void* k_rope_out, void* stream);

/* Bytes of workspace paged_attn_decode needs for these arguments (0 is possible). */
size_t paged_attn_decode_workspace(const pkv_attn_params* params, const pkv_paged_cache* cache);

/* Decode (q_len = 1): out[b, h] = softmax(q[b,h] . K_b^T * scale) V_b over the keys of
 * sequence b visible to its newest position ("KV Cache notes": the attention
 * formula and its decode form; sparse_mode 0 of the skill page's appendix C).
 *   q            : [batch, H, head_dim];  q_rope: [batch, H, rope_dim] iff MLA, else NULL
 *   block_table  : [batch, max_blocks_per_seq]
 *   seq_lens     : [batch], valid keys of each sequence INCLUDING the token written
 *                  this step (the query sits at position seq_lens[b]-1); 0 gives a zero row
 *   out          : [batch, H, head_dim] in params->out_dtype
 *   workspace    : >= paged_attn_decode_workspace(params, cache) bytes of device memory
 * Table entries of blocks that hold no visible key -- wholly before the window,
 * or past the block of key seq_lens[b]-1 -- are never used as block ids, so they
 * may hold anything: the null block, as the KV Cache management design
 * document's sliding-window manager lays them out, or an invalid id such as -1. */
pkv_status paged_attn_decode(const void* q, const void* q_rope, const pkv_paged_cache* cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const pkv_attn_params* params, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* A decode step with its cache append: for every sequence b with seq_lens[b] > 0,
 * the row k_new[b] (and v_new[b], and for MLA k_rope_new[b]) is written to the
 * cache at position seq_lens[b] - 1 -- the slot block_table[b][p / bs] * bs + p % bs
 * of the "KVCache optimisation skill" page's address map, as kv_cache_write_at would
 * -- and then the decode above runs over keys that include it, exactly as
 * paged_attn_decode.  The skill page's decode data flow writes the step's token
 * and then attends with seq_len + 1 keys; this is those two calls as one.
 *   k_new, v_new : [batch, num_kv_heads, head_dim] in the cache's storage type
 *                  (bf16 or fp32; bf16 rows for an int8 cache, quantized as
 *                  kv_cache_write does); v_new NULL when v_cache aliases k_cache
 *   k_rope_new   : [batch, 1, rope_dim] iff the cache has a rope part, else NULL
 *   other arguments, workspace, results and errors: as paged_attn_decode
 * On the bf16 stream-split path (bf16 cache, head_dim 128) it is one kernel: the
 * wave that reads a sequence's newest key takes it from k_new / v_new and stores
 * it at its slot.  Other caches write the rows first and then decode (two
 * launches, the same results).  The rows' slots must not be read by another call
 * running at the same time, and two sequences must not share the newest slot. */
pkv_status paged_attn_decode_append(const void* q, const void* q_rope, const void* k_new, const void* v_new,
                                    const void* k_rope_new, const pkv_paged_cache* cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const pkv_attn_params* params, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* For callers that cannot allocate -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc: paged_attn_decode with no workspace
 * argument.  Its scratch space (the partial outputs of the split) is a
 * library-owned device array of paged_attn_decode_noalloc_capacity() bytes
 * (32 MiB) per GPU, set up on the first call on each device and held until the
 * process ends; nothing is allocated or freed per call.  Same arguments, results
 * and errors as paged_attn_decode, plus PKV_ERR_UNSUPPORTED when the call needs
 * more scratch than the array holds (paged_attn_decode_workspace gives the need).
 * Every call on one GPU shares that GPU's array and no call clears it (no kernel
 * reads scratch it has not written in the same call), so calls that overlap on
 * one GPU -- on different streams, or from different threads -- race: order them
 * on one stream. */
pkv_status paged_attn_decode_noalloc(const void* q, const void* q_rope, const pkv_paged_cache* cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     const pkv_attn_params* params, void* out, void* stream);
size_t paged_attn_decode_noalloc_capacity(void);

/* Bytes of workspace paged_attn_prefill needs (0 when the call is not split).
 * Standard caches: when the (sequence, KV head, 128-column) workgroups of the call
 * are too few to fill the GPU (multi-token decode: a few rows per sequence), the
 * keys are split into partitions of at least 2048 and the fp32 partials
 * ([total_q * H, partitions, head_dim] plus (m, l) pairs) are merged after the
 * kernel.  The size depends on the arguments' sizes only (batch, heads, total_q,
 * max_blocks_per_seq, block_size) and the GPU's CU count, never on device data. */
size_t paged_attn_prefill_workspace(const pkv_attn_params* params, const pkv_paged_cache* cache,
                                    int32_t total_q);

/* Chunked causal prefill over an existing paged cache (sparse_mode 3 of the skill
 * page's appendix C, bottom-right aligned as in the "KV Cache notes" minimal
 * implementation): new row i of sequence b sits at position seq_lens_kv[b] - n_b + i
 * and sees keys j <= that position (and > position - window when window > 0).
 *   q            : TND [total_q, H, head_dim]; q_rope: [total_q, H, rope_dim] iff MLA
 *   cu_seqlens_q : [batch + 1], cu[0] = 0, cu[batch] = total_q, n_b = cu[b+1] - cu[b] >= 0
 *   seq_lens_kv  : [batch], cached + new keys (n_b <= seq_lens_kv[b]); the new rows
 *                  must already be in the cache (kv_cache_write first)
 *   max_q_len    : an upper bound of every n_b (it sizes the grid).  The host
 *                  checks what it can see -- 0 < max_q_len <= total_q and
 *                  max_q_len * batch >= total_q when total_q > 0, else
 *                  PKV_ERR_INVALID_ARG -- but the n_b themselves are device
 *                  contents: a sequence with more rows than max_q_len leaves
 *                  the rows past it unwritten, like any other malformed index.
 *   out          : [total_q, H, head_dim] in params->out_dtype
 * Standard caches need bf16 and head_dim 64 or 128, and a workspace of the size
 * paged_attn_prefill_workspace gives (PKV_ERR_WORKSPACE otherwise).  MLA caches (absorbed form,
 * the same constraints as decode) also cover multi-token decode (n_b of 2-4):
 * every query row is computed over all the keys it sees by one workgroup, so
 * no workspace is used and a row may span at most 1024 table blocks.  Table
 * entries of blocks that hold no key visible to any row of the sequence are
 * never used as block ids (see paged_attn_decode). */
pkv_status paged_attn_prefill(const void* q, const void* q_rope, const pkv_paged_cache* cache,
                              const int32_t* block_table, const int32_t* cu_seqlens_q,
                              const int32_t* seq_lens_kv, int32_t total_q, int32_t max_q_len,
                              const pkv_attn_params* params, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
