/*
 * pkv_oracle.c -- plain, slow CPU oracle for attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke entry point and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the HIP library and must never be used as a
 * fallback for it.
 *
 * Everything here is the plain definition written out, in double precision:
 *   - address map: logical (batch b, position p) -> physical slot
 *       block_table[b][p / block_size] * block_size + p % block_size
 *     ("KVCache optimisation skill" page, section 3.1 "physical memory layout
 *     and logical mapping", with its worked example b=1, pos=300 -> 2348);
 *   - cache write: row t of the new K/V goes to row slot_mapping[t] of the cache
 *     viewed as [num_blocks * block_size, num_kv_heads, dim]
 *     ("Ascend NPU standalone-deployment KVCache guide", mode 2, the
 *     scatter_nd_update write into the flattened cache);
 *   - attention: softmax(q k^T * scale + M) v with the row maximum subtracted
 *     before exponentiation ("KV Cache notes" page, baseline section: the
 *     attention formula, the five-step decomposition and the first of the three
 *     engineering details), one query row at a time, keys summed in ascending
 *     position order;
 *   - GQA: query head h reads KV head h / (H / H_kv) ("KV Cache notes",
 *     section "MHA -> MQA -> GQA", repeat_kv);
 *   - MLA absorbed form: logits are q_nope.c_nope + q_rope.c_rope, the value is
 *     c_nope itself ("KVCache optimisation skill", mode 3; "KV Cache notes",
 *     MLA section);
 *   - causal prefill is bottom-right aligned: new row i of a sequence with L
 *     keys of which n are new sits at absolute position L - n + i and sees keys
 *     0..L-n+i ("KV Cache notes", the 40-line minimal implementation's mask and
 *     the pitfall list on mask alignment);
 *   - sliding window of width W: a query at position p sees keys p-W < j <= p,
 *     i.e. W keys including itself ("KV Cache notes", sliding-window section:
 *     the cache keeps W-1 past keys and the new token is the W-th).
 * Where a row has no visible key the output row is zero (reading of the
 * skill page's note on fully masked rows).
 *
 * Element types: 0 = IEEE float32, 1 = bfloat16 stored as raw uint16 bits,
 * 2 = IEEE float64 (used for caches dequantized from int8 codes, whose values
 * k * scale a float32 cannot hold exactly).
 * All tensors are dense row-major host arrays.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2

#define OR_OK 0
#define OR_ERR_ARG (-1)
#define OR_ERR_INDEX (-2)
#define OR_ERR_NOMEM (-3)

typedef struct {
  const void* k_cache;      /* [num_blocks, block_size, num_kv_heads, k_dim]            */
  const void* v_cache;      /* [num_blocks, block_size, num_kv_heads, v_dim]; may be    */
                            /* the same pointer as k_cache (MLA: key = value = nope)   */
  const void* k_rope_cache; /* [num_blocks, block_size, num_kv_heads, rope_dim] or NULL */
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t k_dim;
  int32_t v_dim;
  int32_t rope_dim; /* 0 when there is no separate rope part */
  int32_t dtype;    /* element type of every cache and of q / q_rope */
} or_cache;

/* One element widened to double.  bf16 -> f32 is exact (the bf16 bits are
   the top half of the f32 bits); f32 -> double is exact. */
static double elem(const void* base, int32_t dtype, int64_t i) {
  if (dtype == OR_F64) return ((const double*)base)[i];
  if (dtype == OR_F32) return (double)((const float*)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int or_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Logical position -> physical slot, or -1 when the table entry or the
   position is out of range. */
static int64_t slot_of(const int32_t* bt_row, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t num_blocks, int32_t pos) {
  if (pos < 0) return -1;
  int32_t logical_block = pos / block_size;
  int32_t offset = pos % block_size;
  if (logical_block >= max_blocks_per_seq) return -1;
  int32_t physical_block = bt_row[logical_block];
  if (physical_block < 0 || physical_block >= num_blocks) return -1;
  return (int64_t)physical_block * block_size + offset;
}

int or_resolve_slots(const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                     int32_t block_size, int32_t num_blocks, const int32_t* batch_idx,
                     const int32_t* pos, int32_t n, int32_t* slots_out) {
  if (block_size <= 0 || max_blocks_per_seq <= 0 || n < 0) return OR_ERR_ARG;
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = batch_idx[i];
    if (b < 0 || b >= batch) return OR_ERR_INDEX;
    int64_t s = slot_of(block_table + (int64_t)b * max_blocks_per_seq, max_blocks_per_seq,
                        block_size, num_blocks, pos[i]);
    if (s < 0 || s > INT32_MAX) return OR_ERR_INDEX;
    slots_out[i] = (int32_t)s;
  }
  return OR_OK;
}

/* rows: [n, row_bytes] -> cache rows slot_mapping[t]; a negative slot skips the row. */
int or_cache_write(void* cache, int64_t num_slots, int64_t row_bytes, const int32_t* slot_mapping,
                   int32_t n, const void* rows) {
  if (row_bytes <= 0 || n < 0) return OR_ERR_ARG;
  for (int32_t t = 0; t < n; ++t) {
    int32_t s = slot_mapping[t];
    if (s < 0) continue;
    if ((int64_t)s >= num_slots) return OR_ERR_INDEX;
    memcpy((char*)cache + (int64_t)s * row_bytes, (const char*)rows + (int64_t)t * row_bytes,
           (size_t)row_bytes);
  }
  return OR_OK;
}

/*
 * One query row against keys [lo, hi) of one sequence.
 *   q_row     : k_dim elements of the query (already offset)
 *   qr_row    : rope_dim elements of the query rope part, or NULL
 *   g         : KV head this query head reads
 *   out_row   : v_dim doubles
 *   prob_row  : NULL or an array indexed by absolute key position; entries
 *               [lo, hi) receive the normalised probabilities
 */
static int attend_row(const or_cache* c, const int32_t* bt_row, int32_t max_blocks_per_seq,
                      const void* q_base, int64_t q_off, const void* qr_base, int64_t qr_off,
                      int32_t g, int32_t lo, int32_t hi, double scale, double* out_row,
                      double* prob_row) {
  for (int32_t d = 0; d < c->v_dim; ++d) out_row[d] = 0.0;
  if (hi <= lo) return OR_OK; /* no visible key: zero row */
  int32_t n = hi - lo;
  double* score = (double*)malloc(sizeof(double) * (size_t)n);
  int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
  if (!score || !slot) {
    free(score);
    free(slot);
    return OR_ERR_NOMEM;
  }
  /* step 1: gather through the block table and score each key */
  for (int32_t j = lo; j < hi; ++j) {
    int64_t s = slot_of(bt_row, max_blocks_per_seq, c->block_size, c->num_blocks, j);
    if (s < 0) {
      free(score);
      free(slot);
      return OR_ERR_INDEX;
    }
    slot[j - lo] = s;
    int64_t krow = (s * c->num_kv_heads + g) * (int64_t)c->k_dim;
    double dot = 0.0;
    for (int32_t d = 0; d < c->k_dim; ++d)
      dot += elem(q_base, c->dtype, q_off + d) * elem(c->k_cache, c->dtype, krow + d);
    if (c->rope_dim > 0) {
      int64_t rrow = (s * c->num_kv_heads + g) * (int64_t)c->rope_dim;
      double rdot = 0.0;
      for (int32_t e = 0; e < c->rope_dim; ++e)
        rdot += elem(qr_base, c->dtype, qr_off + e) * elem(c->k_rope_cache, c->dtype, rrow + e);
      dot += rdot;
    }
    score[j - lo] = scale * dot;
  }
  /* step 2: softmax with the row maximum subtracted */
  double m = score[0];
  for (int32_t i = 1; i < n; ++i)
    if (score[i] > m) m = score[i];
  double l = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    score[i] = exp(score[i] - m);
    l += score[i];
  }
  /* step 3: probability-weighted sum of the value rows */
  for (int32_t i = 0; i < n; ++i) {
    int64_t vrow = (slot[i] * c->num_kv_heads + g) * (int64_t)c->v_dim;
    double p = score[i] / l;
    if (prob_row) prob_row[lo + i] = p;
    for (int32_t d = 0; d < c->v_dim; ++d) out_row[d] += score[i] * elem(c->v_cache, c->dtype, vrow + d);
  }
  for (int32_t d = 0; d < c->v_dim; ++d) out_row[d] /= l;
  free(score);
  free(slot);
  return OR_OK;
}

static int check_cache(const or_cache* c, int32_t num_q_heads) {
  if (!c || !c->k_cache || !c->v_cache) return OR_ERR_ARG;
  if (c->block_size <= 0 || c->num_blocks <= 0 || c->num_kv_heads <= 0) return OR_ERR_ARG;
  if (c->k_dim <= 0 || c->v_dim <= 0 || c->rope_dim < 0) return OR_ERR_ARG;
  if (c->rope_dim > 0 && !c->k_rope_cache) return OR_ERR_ARG;
  if (c->dtype != OR_F32 && c->dtype != OR_BF16 && c->dtype != OR_F64) return OR_ERR_ARG;
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0) return OR_ERR_ARG;
  return OR_OK;
}

/*
 * Decode: one query row per sequence (q_len = 1).
 *   q        : [batch, H, k_dim];  q_rope: [batch, H, rope_dim] when rope_dim > 0
 *   seq_lens : number of valid keys of each sequence, including the token
 *              written this step; the query sits at position seq_lens[b] - 1
 *   units    : optional list of rows b*H + h to compute (NULL = all)
 *   out      : [batch, H, v_dim]; probs: NULL or [batch, H, max_blocks_per_seq*block_size]
 */
int or_paged_decode(const or_cache* c, int32_t batch, int32_t num_q_heads, int32_t max_blocks_per_seq,
                    double scale, int32_t window, const void* q, const void* q_rope,
                    const int32_t* block_table, const int32_t* seq_lens, const int32_t* units,
                    int32_t n_units, double* out, double* probs, int32_t nthreads) {
  int rc = check_cache(c, num_q_heads);
  if (rc) return rc;
  if (batch < 0 || max_blocks_per_seq <= 0 || window < 0 || !q || !out) return OR_ERR_ARG;
  if (c->rope_dim > 0 && !q_rope) return OR_ERR_ARG;
  int32_t group = num_q_heads / c->num_kv_heads;
  int64_t max_keys = (int64_t)max_blocks_per_seq * c->block_size;
  int64_t total = units ? n_units : (int64_t)batch * num_q_heads;
  int status = OR_OK;
  if (nthreads <= 0) nthreads = or_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t u = 0; u < total; ++u) {
    int64_t row = units ? units[u] : u;
    if (row < 0 || row >= (int64_t)batch * num_q_heads) {
#pragma omp atomic write
      status = OR_ERR_INDEX;
      continue;
    }
    int32_t b = (int32_t)(row / num_q_heads);
    int32_t h = (int32_t)(row % num_q_heads);
    int32_t len = seq_lens[b];
    if (len < 0 || len > max_keys) {
#pragma omp atomic write
      status = OR_ERR_INDEX;
      continue;
    }
    int32_t lo = (window > 0 && len > window) ? len - window : 0;
    int r = attend_row(c, block_table + (int64_t)b * max_blocks_per_seq, max_blocks_per_seq, q,
                       row * c->k_dim, q_rope, row * (int64_t)c->rope_dim, h / group, lo, len, scale,
                       out + row * c->v_dim, probs ? probs + row * max_keys : NULL);
    if (r) {
#pragma omp atomic write
      status = r;
    }
  }
  return status;
}

/*
 * Prefill over an existing paged cache: new query rows in TND layout.
 *   q            : [total_q, H, k_dim]; q_rope: [total_q, H, rope_dim] when rope_dim > 0
 *   cu_seqlens_q : [batch + 1], rows of sequence b are cu[b] .. cu[b+1]-1
 *   seq_lens_kv  : keys of sequence b, cached plus new (the new rows must
 *                  already be written to the cache)
 *   units        : optional list of rows t*H + h to compute (NULL = all)
 *   out          : [total_q, H, v_dim]; probs: NULL or [total_q, H, max_blocks_per_seq*block_size]
 */
int or_paged_prefill(const or_cache* c, int32_t batch, int32_t num_q_heads, int32_t max_blocks_per_seq,
                     double scale, int32_t window, const void* q, const void* q_rope, int32_t total_q,
                     const int32_t* block_table, const int32_t* cu_seqlens_q,
                     const int32_t* seq_lens_kv, const int32_t* units, int32_t n_units, double* out,
                     double* probs, int32_t nthreads) {
  int rc = check_cache(c, num_q_heads);
  if (rc) return rc;
  if (batch < 0 || total_q < 0 || max_blocks_per_seq <= 0 || window < 0 || !q || !out)
    return OR_ERR_ARG;
  if (c->rope_dim > 0 && !q_rope) return OR_ERR_ARG;
  if (cu_seqlens_q[0] != 0 || cu_seqlens_q[batch] != total_q) return OR_ERR_ARG;
  for (int32_t b = 0; b < batch; ++b) {
    int32_t n_new = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    if (n_new < 0 || n_new > seq_lens_kv[b]) return OR_ERR_ARG;
    if (seq_lens_kv[b] > (int64_t)max_blocks_per_seq * c->block_size) return OR_ERR_INDEX;
  }
  int32_t group = num_q_heads / c->num_kv_heads;
  int64_t max_keys = (int64_t)max_blocks_per_seq * c->block_size;
  int64_t total = units ? n_units : (int64_t)total_q * num_q_heads;
  int status = OR_OK;
  if (nthreads <= 0) nthreads = or_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t u = 0; u < total; ++u) {
    int64_t row = units ? units[u] : u;
    if (row < 0 || row >= (int64_t)total_q * num_q_heads) {
#pragma omp atomic write
      status = OR_ERR_INDEX;
      continue;
    }
    int32_t t = (int32_t)(row / num_q_heads);
    int32_t h = (int32_t)(row % num_q_heads);
    int32_t b = 0;
    while (!(cu_seqlens_q[b] <= t && t < cu_seqlens_q[b + 1])) ++b;
    int32_t i = t - cu_seqlens_q[b];
    int32_t n_new = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    int32_t p = seq_lens_kv[b] - n_new + i; /* absolute position of this query row */
    int32_t hi = p + 1;
    int32_t lo = (window > 0 && p + 1 > window) ? p + 1 - window : 0;
    int r = attend_row(c, block_table + (int64_t)b * max_blocks_per_seq, max_blocks_per_seq, q,
                       row * c->k_dim, q_rope, row * (int64_t)c->rope_dim, h / group, lo, hi, scale,
                       out + row * c->v_dim, probs ? probs + row * max_keys : NULL);
    if (r) {
#pragma omp atomic write
      status = r;
    }
  }
  return status;
}
