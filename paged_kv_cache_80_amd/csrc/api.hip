// api.hip -- the C ABI of libpkv (declared in include/pkv.h): argument checks,
// partition sizing and kernel launches on the caller's stream.  No allocation,
// no synchronisation, no device reads on the host side.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "device_common.h"
#include "pkv_error.h"
#include "pkv_internal.h"

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

pkv_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int32_t dtype) { return dtype == PKV_INT8 ? 1 : dtype == PKV_BF16 ? 2 : 4; }

bool valid_dtype(int32_t d) { return d == PKV_F32 || d == PKV_BF16; }

bool is_int8(const pkv_paged_cache* c) { return c->dtype == PKV_INT8; }

bool pow2_block(int32_t bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }

int32_t log2i(int32_t v) { return __builtin_ctz((unsigned)v); }

bool is_mla(const pkv_paged_cache* c) { return c->rope_dim > 0; }

// Shared structural checks of a cache description.
pkv_status check_cache(const pkv_paged_cache* c) {
  if (!c) return fail(PKV_ERR_INVALID_ARG, "cache is NULL");
  if (!c->k_cache || !c->v_cache) return fail(PKV_ERR_INVALID_ARG, "k_cache / v_cache is NULL");
  if (!valid_dtype(c->dtype) && c->dtype != PKV_INT8)
    return fail(PKV_ERR_INVALID_ARG, "cache dtype %d is not f32, bf16 or int8", c->dtype);
  if (c->num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "num_blocks %d must be > 0", c->num_blocks);
  if (!pow2_block(c->block_size))
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d is not one of 16, 32, 64, 128", c->block_size);
  if (c->num_kv_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads %d must be > 0", c->num_kv_heads);
  if (c->head_dim <= 0) return fail(PKV_ERR_INVALID_ARG, "head_dim %d must be > 0", c->head_dim);
  if (c->rope_dim < 0) return fail(PKV_ERR_INVALID_ARG, "rope_dim %d must be >= 0", c->rope_dim);
  if ((c->rope_dim > 0) != (c->k_rope_cache != nullptr))
    return fail(PKV_ERR_INVALID_ARG, "k_rope_cache must be given exactly when rope_dim > 0");
  const int64_t row = (int64_t)c->num_kv_heads * c->head_dim * elem_bytes(c->dtype);
  if (row % 16 != 0) return fail(PKV_ERR_UNSUPPORTED, "a cache row of %lld bytes is not a multiple of 16", (long long)row);
  // Row byte counts travel as 32-bit values and tile loads address up to 64 slot
  // rows from one base with 32-bit lane offsets.
  if (row > (int64_t(1) << 24))
    return fail(PKV_ERR_UNSUPPORTED, "a cache row of %lld bytes exceeds 16 MiB", (long long)row);
  if (c->rope_dim > 0 && ((int64_t)c->num_kv_heads * c->rope_dim * elem_bytes(c->dtype)) % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "a rope row is not a multiple of 16 bytes");
  if (!aligned16(c->k_cache) || !aligned16(c->v_cache) || (c->k_rope_cache && !aligned16(c->k_rope_cache)))
    return fail(PKV_ERR_INVALID_ARG, "cache pointers must be 16-byte aligned");
  // Slots cross the ABI and are resolved on the device as int32.
  if ((int64_t)c->num_blocks * c->block_size > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "num_blocks %d x block_size %d slots exceed the int32 slot range", c->num_blocks,
                c->block_size);
  if (is_int8(c)) {
    if (!c->k_scale || !c->v_scale) return fail(PKV_ERR_INVALID_ARG, "int8 cache: k_scale / v_scale is NULL");
    if (!aligned16(c->k_scale) || !aligned16(c->v_scale))
      return fail(PKV_ERR_INVALID_ARG, "int8 cache: scale pointers must be 16-byte aligned");
    if (is_mla(c)) return fail(PKV_ERR_UNSUPPORTED, "int8 cache: no rope part (standard attention only)");
    if (c->v_cache == c->k_cache) return fail(PKV_ERR_INVALID_ARG, "int8 cache: k_cache and v_cache must differ");
    if (c->head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "int8 cache: head_dim must be 128 (got %d)", c->head_dim);
  } else if (c->k_scale || c->v_scale) {
    return fail(PKV_ERR_INVALID_ARG, "k_scale / v_scale apply to int8 caches only");
  }
  if (is_mla(c)) {
    // "KVCache optimisation skill", mode 3 constraints: key = value = cache_nope,
    // rope D = 64, latent width 512, a single latent head.
    if (c->v_cache != c->k_cache) return fail(PKV_ERR_INVALID_ARG, "MLA: v_cache must alias k_cache (key = value = cache_nope)");
    if (c->rope_dim != 64) return fail(PKV_ERR_UNSUPPORTED, "MLA: rope_dim must be 64 (got %d)", c->rope_dim);
    if (c->num_kv_heads != 1) return fail(PKV_ERR_INVALID_ARG, "MLA: num_kv_heads must be 1 (got %d)", c->num_kv_heads);
    if (c->head_dim != 512) return fail(PKV_ERR_UNSUPPORTED, "MLA: latent width must be 512 (got %d)", c->head_dim);
  }
  return PKV_OK;
}

pkv_status check_params(const pkv_attn_params* p, const pkv_paged_cache* c) {
  if (!p) return fail(PKV_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch %d must be >= 0", p->batch);
  if (p->batch > 65535) return fail(PKV_ERR_UNSUPPORTED, "batch %d exceeds 65535", p->batch);
  if (p->num_q_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d must be > 0", p->num_q_heads);
  if (p->num_q_heads % c->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", p->num_q_heads,
                c->num_kv_heads);
  if (p->max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be > 0");
  if (!(std::isfinite(p->scale) && p->scale > 0.f))
    return fail(PKV_ERR_INVALID_ARG, "scale %g must be finite and > 0 (there is no default)", (double)p->scale);
  if (p->window < 0) return fail(PKV_ERR_INVALID_ARG, "window %d must be >= 0", p->window);
  if (!valid_dtype(p->out_dtype)) return fail(PKV_ERR_INVALID_ARG, "out_dtype %d is not f32 or bf16", p->out_dtype);
  if (p->split_tokens < 0 || (p->split_tokens % c->block_size) != 0)
    return fail(PKV_ERR_INVALID_ARG, "split_tokens %d must be a non-negative multiple of block_size %d",
                p->split_tokens, c->block_size);
  return PKV_OK;
}

// Decode work split.  The stream-split kernel (bf16, head_dim 128) spreads the
// tiles of all sequences over the resident waves; the partition kernels (VALU
// decode, MLA) split each sequence into partitions of bpp table blocks.
struct DecodePlan {
  bool stream;
  int32_t resident_waves;  // stream split
  int32_t split_tiles;     // stream split: tiles per wave target (0 = all waves)
  int32_t bpp;             // partition split
  int32_t max_np;
  int32_t valu_waves;      // vector-ALU decode: 4 per partition, 16 per whole sequence
  size_t ws_bytes;
  size_t ws_o_offset;
  size_t ws_ml_offset;
};

// Compute units of the current device (queried once per device; 256 when no
// device can be queried, so that a size query without a GPU stays defined).
int32_t device_cu_count() {
  constexpr int kMaxDev = 64;
  static int32_t cached[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// The stream split needs a wave per KV head in every wave group.
bool use_stream_decode(const pkv_attn_params* p, const pkv_paged_cache* c) {
  return !is_mla(c) && pkv::decode_mfma_supported(c->dtype, c->head_dim, p->num_q_heads / c->num_kv_heads) &&
         c->num_kv_heads <= pkv::decode_stream_resident_waves(device_cu_count(), c->dtype);
}

constexpr int32_t kMaxBpp = 1024;

DecodePlan plan_decode(const pkv_attn_params* p, const pkv_paged_cache* c) {
  DecodePlan plan{};
  if (use_stream_decode(p, c)) {
    plan.stream = true;
    plan.resident_waves = pkv::decode_stream_resident_waves(device_cu_count(), c->dtype);
    plan.split_tiles = p->split_tokens / 32;  // split_tokens is a multiple of the block size (>= 16)
    if (p->split_tokens > 0 && plan.split_tiles == 0) plan.split_tiles = 1;
    plan.max_np = 1;
    plan.ws_bytes = pkv::decode_stream_workspace(p->batch, p->num_q_heads / c->num_kv_heads, c->num_kv_heads,
                                                 plan.resident_waves,
                                                 &plan.ws_o_offset, &plan.ws_ml_offset);
    return plan;
  }
  const int32_t bs = c->block_size;
  int32_t span = p->max_blocks_per_seq;  // table blocks one sequence can touch
  if (p->window > 0) span = std::min<int64_t>(span, (p->window + bs - 1) / bs + 1);
  int32_t bpp;
  if (p->split_tokens > 0) {
    bpp = p->split_tokens / bs;
  } else {
    // Enough workgroups to fill 256 CUs several times, partitions of at most a
    // few hundred KiB so ragged lengths balance.
    int32_t part_tokens;
    if (is_mla(c)) {
      // One workgroup holds up to 128 heads; aim for about one workgroup per CU
      // with partitions long enough that the partial outputs stay a small
      // fraction of the latent bytes.
      const int64_t units = (int64_t)p->batch * std::max(1, p->num_q_heads / 128);
      part_tokens = units >= 256 ? 1 << 30 : units >= 128 ? 4096 : 2048;
    } else {
      // At most 512 keys a partition (2048 with 1024 or more (sequence, KV head)
      // pairs), fewer -- down to 128 -- while that would leave CUs without a
      // workgroup (a tiny decode, 2 sequences x 4 heads of up to 512 keys, took
      // 11.3 us as 8 four-wave workgroups each walking a whole sequence, 7.9 us
      // as 32 partitions plus the combine).
      const int64_t units = (int64_t)p->batch * c->num_kv_heads;
      const int64_t keys = (int64_t)span * bs;
      part_tokens = units >= 1024 ? 2048
                                  : (int32_t)std::min<int64_t>(512, std::max<int64_t>(128, keys * units / device_cu_count()));
    }
    bpp = (int32_t)std::max<int64_t>(1, part_tokens / bs);
  }
  bpp = std::max(1, std::min({bpp, span, kMaxBpp}));
  // The partition index is a grid dimension limited to 65535.
  while ((span + bpp - 1) / bpp > 65535 && bpp < kMaxBpp) bpp = std::min(2 * bpp, kMaxBpp);
  plan.bpp = bpp;
  plan.max_np = (span + bpp - 1) / bpp;
  plan.valu_waves = 4;
  // A sequence cut into at most 4 partitions is walked by one 16-wave workgroup
  // instead: the same keys per wave and iteration, merged in LDS rather than by
  // a second kernel over partials (unless the caller asked for partitions); the
  // tiny decode then takes 5.4 us with its cache resident, 7.5 us from HBM.
  if (!is_mla(c) && p->split_tokens == 0 && plan.max_np > 1 && plan.max_np <= 4 && span <= kMaxBpp &&
      pkv::decode_valu_wide_supported(c->dtype, c->head_dim, p->num_q_heads / c->num_kv_heads)) {
    plan.bpp = span;
    plan.max_np = 1;
    plan.valu_waves = 16;
  }
  if (plan.max_np > 1) {
    const size_t rows = (size_t)p->batch * p->num_q_heads * plan.max_np;
    const size_t o_bytes = (rows * c->head_dim * sizeof(float) + 255) & ~size_t(255);
    plan.ws_o_offset = 0;
    plan.ws_ml_offset = o_bytes;
    plan.ws_bytes = o_bytes + rows * 2 * sizeof(float);
  }
  return plan;
}

// Prefill key split.  A prefill workgroup takes 128 query columns of one
// (sequence, KV head) and walks every key they see; with few such workgroups
// (short chunks: a handful of rows per sequence, more (row, head) columns per KV
// head than the decode's stream split takes) the chip is not filled and the
// longest sequence sets the time.  Then the keys are cut into partitions,
// enough for about 16 workgroups per CU (ragged lengths leave many partitions
// empty), of at least 2048 keys so that the fp32 partials stay a small fraction
// of the K/V bytes (8, 32 and 64 per CU, and 1024- or 512-key partitions, measured
// slower on the 70B multi-token decode when it ran here).  The plan uses only what the
// workspace query also knows (rows per sequence from total_q, keys from the table
// width), so both see the same partitions.
struct PrefillPlan {
  int32_t np = 1;
  int32_t part_tiles = 0;
  size_t ws_bytes = 0;
  size_t ws_ml_offset = 0;
};

PrefillPlan plan_prefill(const pkv_attn_params* p, const pkv_paged_cache* c, int32_t total_q) {
  PrefillPlan plan;
  if (is_mla(c) || p->batch <= 0 || total_q <= 0) return plan;
  const int64_t G = p->num_q_heads / c->num_kv_heads;
  const int64_t rows_per_seq = ((int64_t)total_q + p->batch - 1) / p->batch;
  const int64_t wgs = (int64_t)p->batch * c->num_kv_heads *
                      ((rows_per_seq * G + pkv::kPrefillColumns - 1) / pkv::kPrefillColumns);
  const int64_t cus = device_cu_count();
  if (wgs >= 2 * cus) return plan;  // the grid fills the chip: one pass over the keys
  const int64_t max_kv = (int64_t)p->max_blocks_per_seq * c->block_size;
  const int64_t want = (16 * cus + wgs - 1) / wgs;  // partitions per workgroup
  constexpr int64_t kMinPart = 2048;                // keys; a multiple of every block size and tile
  const int64_t part = std::max<int64_t>(kMinPart, ((max_kv + want - 1) / want + kMinPart - 1) / kMinPart * kMinPart);
  const int64_t np = (max_kv + part - 1) / part;
  if (np <= 1) return plan;
  plan.np = (int32_t)np;
  plan.part_tiles = (int32_t)(part / pkv::kPrefillKeyTile);
  const size_t rows = (size_t)total_q * p->num_q_heads * (size_t)np;
  const size_t o_bytes = (rows * c->head_dim * sizeof(float) + 255) & ~size_t(255);
  plan.ws_ml_offset = o_bytes;
  plan.ws_bytes = o_bytes + rows * 2 * sizeof(float);
  return plan;
}

// Scratch for callers that cannot allocate (paged_attn_decode_noalloc): one
// library-owned array per GPU, alive until the process ends.  In host code the
// array's name is only a stand-in; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

pkv_status static_scratch_ptr(void** out) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDev] = {};
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDev) return fail(PKV_ERR_UNSUPPORTED, "device %d is past the %d the library tracks", dev, kMaxDev);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess) return from_hip(g, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return PKV_OK;
}

// The newest K / V (/ rope) row of every sequence, for paged_attn_decode_append.
struct AppendRows {
  const void* k;
  const void* v;
  const void* k_rope;
};
pkv_status decode_impl(const void* q, const void* q_rope, const pkv_paged_cache* cache, const int32_t* block_table,
                       const int32_t* seq_lens, const pkv_attn_params* params, void* out, void* workspace,
                       size_t workspace_bytes, void* stream, bool static_scratch, const AppendRows* app = nullptr);

pkv_status write_impl(const pkv::SlotSource& slots, int32_t num_tokens, const void* k, const void* v,
                      const void* k_rope, const pkv_paged_cache* cache, void* stream) {
  pkv_status s = check_cache(cache);
  if (s) return s;
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens %d must be >= 0", num_tokens);
  if (num_tokens == 0) return ok();
  if (!k) return fail(PKV_ERR_INVALID_ARG, "k must not be NULL");
  const bool shared_kv = cache->v_cache == cache->k_cache;
  if (shared_kv && v) return fail(PKV_ERR_INVALID_ARG, "v must be NULL when v_cache aliases k_cache");
  if (!shared_kv && !v) return fail(PKV_ERR_INVALID_ARG, "v must not be NULL");
  if ((cache->rope_dim > 0) != (k_rope != nullptr))
    return fail(PKV_ERR_INVALID_ARG, "k_rope must be given exactly when the cache has a rope part");
  if (!aligned16(k) || (v && !aligned16(v)) || (k_rope && !aligned16(k_rope)))
    return fail(PKV_ERR_INVALID_ARG, "k / v / k_rope must be 16-byte aligned");
  if (is_int8(cache)) {
    pkv::Int8WriteArgs w{};
    w.k = k;
    w.v = v;
    w.k_cache = cache->k_cache;
    w.v_cache = cache->v_cache;
    w.k_scale = static_cast<float*>(cache->k_scale);
    w.v_scale = static_cast<float*>(cache->v_scale);
    w.num_tokens = num_tokens;
    w.num_kv_heads = cache->num_kv_heads;
    w.block_size_log2 = log2i(cache->block_size);
    return from_hip(pkv::launch_cache_write_int8(slots, w, static_cast<hipStream_t>(stream)), "cache write launch");
  }
  pkv::WriteRows rows{};
  const int32_t eb = elem_bytes(cache->dtype);
  rows.src[0] = k;
  rows.dst[0] = cache->k_cache;
  rows.row_bytes[0] = cache->num_kv_heads * cache->head_dim * eb;
  rows.count = 1;
  if (!shared_kv) {
    rows.src[1] = v;
    rows.dst[1] = cache->v_cache;
    rows.row_bytes[1] = rows.row_bytes[0];
    rows.count = 2;
  }
  if (cache->rope_dim > 0) {
    rows.src[rows.count] = k_rope;
    rows.dst[rows.count] = cache->k_rope_cache;
    rows.row_bytes[rows.count] = cache->num_kv_heads * cache->rope_dim * eb;
    rows.count++;
  }
  return from_hip(pkv::launch_cache_write(slots, num_tokens, rows, static_cast<hipStream_t>(stream)),
                  "cache write launch");
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }

pkv_status pkv_resolve_slots(const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                             int32_t block_size, const int32_t* batch_idx, const int32_t* pos, int32_t n,
                             int32_t* slots_out, void* stream) {
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n %d must be >= 0", n);
  if (n == 0) return ok();
  if (!block_table || !batch_idx || !pos || !slots_out) return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  if (batch <= 0 || max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "batch and max_blocks_per_seq must be > 0");
  if (!pow2_block(block_size)) return fail(PKV_ERR_UNSUPPORTED, "block_size %d is not one of 16, 32, 64, 128", block_size);
  return from_hip(pkv::launch_resolve_slots(block_table, batch, max_blocks_per_seq, block_size, batch_idx, pos, n,
                                            slots_out, static_cast<hipStream_t>(stream)),
                  "pkv_resolve_slots launch");
}

pkv_status paged_resolve_slots(const int32_t* block_table, int32_t max_blocks_per_seq, int32_t block_size,
                               const int32_t* batch_idx, const int32_t* pos, int32_t n, int32_t* slots_out,
                               void* stream) {
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n %d must be >= 0", n);
  if (n == 0) return ok();
  if (!block_table || !batch_idx || !pos || !slots_out) return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be > 0");
  if (!pow2_block(block_size)) return fail(PKV_ERR_UNSUPPORTED, "block_size %d is not one of 16, 32, 64, 128", block_size);
  return from_hip(pkv::launch_resolve_slots(block_table, 0, max_blocks_per_seq, block_size, batch_idx, pos, n,
                                            slots_out, static_cast<hipStream_t>(stream)),
                  "paged_resolve_slots launch");
}

pkv_status kv_cache_write(const int32_t* slot_mapping, int32_t num_tokens, const void* k, const void* v,
                          const void* k_rope, const pkv_paged_cache* cache, void* stream) {
  if (num_tokens > 0 && !slot_mapping) return fail(PKV_ERR_INVALID_ARG, "slot_mapping must not be NULL");
  pkv::SlotSource src{};
  src.slot_mapping = slot_mapping;
  return write_impl(src, num_tokens, k, v, k_rope, cache, stream);
}

pkv_status kv_cache_write_at(const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* batch_idx,
                             const int32_t* pos, int32_t num_tokens, const void* k, const void* v, const void* k_rope,
                             const pkv_paged_cache* cache, int32_t* slots_out, void* stream) {
  pkv_status st = check_cache(cache);
  if (st) return st;
  if (num_tokens > 0 && (!block_table || !batch_idx || !pos))
    return fail(PKV_ERR_INVALID_ARG, "block_table, batch_idx and pos must not be NULL");
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be > 0");
  pkv::SlotSource src{};
  src.block_table = block_table;
  src.batch_idx = batch_idx;
  src.pos = pos;
  src.slots_out = slots_out;
  src.max_blocks_per_seq = max_blocks_per_seq;
  src.block_size_log2 = log2i(cache->block_size);
  return write_impl(src, num_tokens, k, v, k_rope, cache, stream);
}

pkv_status kv_rmsnorm_rope_cache(const void* latent, const void* gamma, const void* cos, const void* sin,
                                 const int32_t* slot_mapping, int32_t num_tokens, float eps,
                                 int32_t rope_layout, const pkv_paged_cache* cache, void* k_nope_out,
                                 void* k_rope_out, void* stream) {
  pkv_status s = check_cache(cache);
  if (s) return s;
  if (!is_mla(cache)) return fail(PKV_ERR_INVALID_ARG, "kv_rmsnorm_rope_cache needs an MLA cache (rope_dim > 0)");
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens %d must be >= 0", num_tokens);
  if (!(std::isfinite(eps) && eps >= 0.0f)) return fail(PKV_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (rope_layout != PKV_ROPE_HALF && rope_layout != PKV_ROPE_INTERLEAVED)
    return fail(PKV_ERR_INVALID_ARG, "rope_layout %d is not PKV_ROPE_HALF or PKV_ROPE_INTERLEAVED", rope_layout);
  if ((k_nope_out != nullptr) != (k_rope_out != nullptr))
    return fail(PKV_ERR_INVALID_ARG, "k_nope_out and k_rope_out must be given together or not at all");
  if (num_tokens == 0) return ok();
  if (!latent || !gamma || !cos || !sin || !slot_mapping) return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned16(latent) || !aligned16(gamma) || !aligned16(cos) || !aligned16(sin) ||
      (k_nope_out && (!aligned16(k_nope_out) || !aligned16(k_rope_out))))
    return fail(PKV_ERR_INVALID_ARG, "latent / gamma / cos / sin / outputs must be 16-byte aligned");
  pkv::LatentWriteArgs a{};
  a.latent = latent;
  a.gamma = gamma;
  a.cos = cos;
  a.sin = sin;
  a.slot_mapping = slot_mapping;
  a.cache_nope = cache->k_cache;
  a.cache_rope = cache->k_rope_cache;
  a.out_nope = k_nope_out;
  a.out_rope = k_rope_out;
  a.num_tokens = num_tokens;
  a.eps = eps;
  a.bf16 = cache->dtype == PKV_BF16;
  a.interleaved = rope_layout == PKV_ROPE_INTERLEAVED;
  return from_hip(pkv::launch_latent_write(a, static_cast<hipStream_t>(stream)), "kv_rmsnorm_rope_cache launch");
}

size_t paged_attn_decode_workspace(const pkv_attn_params* params, const pkv_paged_cache* cache) {
  if (check_cache(cache) || check_params(params, cache)) return 0;
  return plan_decode(params, cache).ws_bytes;
}

pkv_status paged_attn_decode(const void* q, const void* q_rope, const pkv_paged_cache* cache,
                             const int32_t* block_table, const int32_t* seq_lens, const pkv_attn_params* params,
                             void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, q_rope, cache, block_table, seq_lens, params, out, workspace, workspace_bytes, stream,
                     false);
}

pkv_status paged_attn_decode_noalloc(const void* q, const void* q_rope, const pkv_paged_cache* cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     const pkv_attn_params* params, void* out, void* stream) {
  return decode_impl(q, q_rope, cache, block_table, seq_lens, params, out, nullptr, 0, stream, true);
}

pkv_status paged_attn_decode_append(const void* q, const void* q_rope, const void* k_new, const void* v_new,
                                    const void* k_rope_new, const pkv_paged_cache* cache, const int32_t* block_table,
                                    const int32_t* seq_lens, const pkv_attn_params* params, void* out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  const AppendRows app{k_new, v_new, k_rope_new};
  return decode_impl(q, q_rope, cache, block_table, seq_lens, params, out, workspace, workspace_bytes, stream, false,
                     &app);
}

size_t paged_attn_decode_noalloc_capacity(void) { return kStaticScratchBytes; }

}  // extern "C"

namespace {

pkv_status decode_impl(const void* q, const void* q_rope, const pkv_paged_cache* cache, const int32_t* block_table,
                       const int32_t* seq_lens, const pkv_attn_params* params, void* out, void* workspace,
                       size_t workspace_bytes, void* stream, bool static_scratch, const AppendRows* app) {
  pkv_status s = check_cache(cache);
  if (s) return s;
  s = check_params(params, cache);
  if (s) return s;
  if (params->batch == 0) return ok();
  if (!q || !block_table || !seq_lens || !out) return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  if ((q_rope != nullptr) != is_mla(cache))
    return fail(PKV_ERR_INVALID_ARG, "q_rope and k_rope must be given together or not at all");
  if (!aligned16(q) || !aligned16(out) || (q_rope && !aligned16(q_rope)))
    return fail(PKV_ERR_INVALID_ARG, "q / q_rope / out must be 16-byte aligned");
  const int32_t group = params->num_q_heads / cache->num_kv_heads;
  const DecodePlan plan = plan_decode(params, cache);
  if (plan.max_np > 65535) return fail(PKV_ERR_UNSUPPORTED, "decode: %d partitions exceed 65535", plan.max_np);
  if ((int64_t)params->batch * cache->num_kv_heads > 0x7fffffff)
    return fail(PKV_ERR_UNSUPPORTED, "decode: batch x num_kv_heads exceeds the grid");
  if (static_scratch && plan.ws_bytes > 0) {
    if (plan.ws_bytes > kStaticScratchBytes)
      return fail(PKV_ERR_UNSUPPORTED, "decode needs %zu bytes of scratch; the library's static array holds %zu",
                  plan.ws_bytes, kStaticScratchBytes);
    s = static_scratch_ptr(&workspace);
    if (s) return s;
    workspace_bytes = kStaticScratchBytes;
  }
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (plan.ws_bytes > 0 && !aligned16(workspace)) return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // Append: the bf16 stream split reads each sequence's newest row from the
  // caller's rows and stores it at its slot inside the decode kernel; every other
  // path writes the rows first (the writer of kv_cache_write_at, positions
  // seq_lens[b] - 1) and then runs the decode unchanged.
  const bool fused_append = app && plan.stream && cache->dtype == PKV_BF16;
  if (app) {
    const bool shared_kv = cache->v_cache == cache->k_cache;
    if (!app->k || (!shared_kv && !app->v) || (shared_kv && app->v))
      return fail(PKV_ERR_INVALID_ARG, "append: k_new is required, v_new exactly when v_cache is its own tensor");
    if ((app->k_rope != nullptr) != is_mla(cache))
      return fail(PKV_ERR_INVALID_ARG, "append: k_rope_new must be given exactly when the cache has a rope part");
    if (!aligned16(app->k) || (app->v && !aligned16(app->v)) || (app->k_rope && !aligned16(app->k_rope)))
      return fail(PKV_ERR_INVALID_ARG, "append: k_new / v_new / k_rope_new must be 16-byte aligned");
    if (!fused_append) {
      pkv::SlotSource src{};
      src.block_table = block_table;
      src.append_lens = seq_lens;
      src.max_blocks_per_seq = params->max_blocks_per_seq;
      src.block_size_log2 = log2i(cache->block_size);
      s = write_impl(src, params->batch, app->k, app->v, app->k_rope, cache, stream);
      if (s) return s;
    }
  }
  char* wsb = static_cast<char*>(workspace);
  float* ws_o = plan.ws_bytes > 0 ? reinterpret_cast<float*>(wsb + plan.ws_o_offset) : nullptr;
  float* ws_ml = plan.ws_bytes > 0 ? reinterpret_cast<float*>(wsb + plan.ws_ml_offset) : nullptr;
  if (is_mla(cache)) {
    if (!pkv::mla_decode_supported(cache->dtype, cache->head_dim, cache->rope_dim, params->num_q_heads))
      return fail(PKV_ERR_UNSUPPORTED, "MLA decode: needs bf16, latent 512, rope 64 and H a multiple of 16");
    pkv::MlaArgs m{};
    m.q = q;
    m.q_rope = q_rope;
    m.c_nope = cache->k_cache;
    m.c_rope = cache->k_rope_cache;
    m.block_table = block_table;
    m.seq_lens = seq_lens;
    m.out = out;
    m.ws_o = ws_o;
    m.ws_ml = ws_ml;
    m.batch = params->batch;
    m.num_q_heads = params->num_q_heads;
    m.max_blocks_per_seq = params->max_blocks_per_seq;
    m.block_size_log2 = log2i(cache->block_size);
    m.blocks_per_part = plan.bpp;
    m.max_np = plan.max_np;
    m.window = params->window;
    m.scale_log2e = params->scale * pkv::kLog2e;
    m.out_dtype = params->out_dtype;
    m.rows = params->batch;
    hipError_t e = pkv::launch_mla_decode(m, st);
    if (e != hipSuccess) return from_hip(e, "MLA decode launch");
    if (plan.max_np > 1) {
      e = pkv::launch_decode_combine(ws_o, ws_ml, seq_lens, params->batch, params->num_q_heads, cache->head_dim,
                                     plan.max_np, m.block_size_log2, plan.bpp, params->window, out,
                                     params->out_dtype, st);
      if (e != hipSuccess) return from_hip(e, "decode combine launch");
    }
    return ok();
  }
  if (!plan.stream && is_int8(cache))
    return fail(PKV_ERR_UNSUPPORTED, "int8 decode: needs head groups of at most 16 (got %d)", group);
  if (!plan.stream && !pkv::decode_valu_supported(cache->dtype, cache->head_dim, group))
    return fail(PKV_ERR_UNSUPPORTED, "decode: dtype %d, head_dim %d, group %d not supported", cache->dtype,
                cache->head_dim, group);
  pkv::DecodeArgs a{};
  a.q = q;
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.ws_o = ws_o;
  a.ws_ml = ws_ml;
  a.batch = params->batch;
  a.num_q_heads = params->num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.max_blocks_per_seq = params->max_blocks_per_seq;
  a.block_size_log2 = log2i(cache->block_size);
  a.blocks_per_part = plan.bpp;
  a.max_np = plan.max_np;
  a.window = params->window;
  a.scale_log2e = params->scale * pkv::kLog2e;
  a.dtype = cache->dtype;
  a.out_dtype = params->out_dtype;
  a.k_scale = static_cast<const float*>(cache->k_scale);
  a.v_scale = static_cast<const float*>(cache->v_scale);
  a.valu_waves = plan.valu_waves;
  if (fused_append) {
    a.k_new = app->k;
    a.v_new = app->v;
  }
  if (plan.stream) {
    // bf16 with 128-wide heads: matrix-core decode over a stream split (any head
    // group: the group is a dense contraction and every K/V row is read once).
    a.tile_prefix = reinterpret_cast<int32_t*>(wsb);
    a.resident_waves = plan.resident_waves;
    a.split_tiles = plan.split_tiles;
    return from_hip(pkv::launch_decode_stream(a, st), "decode launch");
  }
  hipError_t e = pkv::launch_decode_valu(a, st);
  if (e != hipSuccess) return from_hip(e, "decode launch");
  if (plan.max_np > 1) {
    e = pkv::launch_decode_combine(a.ws_o, a.ws_ml, seq_lens, params->batch, params->num_q_heads, cache->head_dim,
                                   plan.max_np, a.block_size_log2, plan.bpp, params->window, out,
                                   params->out_dtype, st);
    if (e != hipSuccess) return from_hip(e, "decode combine launch");
  }
  return ok();
}

// Multi-token decode (a few query rows per sequence) through the stream split of
// decode: when every sequence's rows times the head group fit the kernel's two
// 16-column tiles, its K/V are streamed once for all of them, as in decode.  The
// call decides from max_q_len; the workspace query, which only sees total_q,
// answers for both paths whenever the average row count allows this one.
bool stream_mt_supported(const pkv_attn_params* p, const pkv_paged_cache* c) {
  if (is_mla(c) || c->dtype != PKV_BF16) return false;
  const int32_t group = p->num_q_heads / c->num_kv_heads;
  return pkv::decode_mfma_supported(c->dtype, c->head_dim, group) &&
         c->num_kv_heads <= pkv::decode_stream_resident_waves(device_cu_count(), c->dtype);
}

bool stream_mt_fits(const pkv_attn_params* p, const pkv_paged_cache* c, int64_t rows) {
  return rows > 0 && rows * (p->num_q_heads / c->num_kv_heads) <= pkv::kStreamMtColumns;
}

size_t stream_mt_workspace(const pkv_attn_params* p, const pkv_paged_cache* c, size_t* o_off, size_t* ml_off) {
  return pkv::decode_stream_workspace(p->batch, pkv::kStreamMtColumns, c->num_kv_heads,
                                      pkv::decode_stream_resident_waves(device_cu_count(), c->dtype), o_off, ml_off);
}

}  // namespace

extern "C" {

size_t paged_attn_prefill_workspace(const pkv_attn_params* params, const pkv_paged_cache* cache, int32_t total_q) {
  if (check_cache(cache) || check_params(params, cache) || total_q < 0) return 0;
  size_t ws = plan_prefill(params, cache, total_q).ws_bytes;
  if (params->batch > 0 && stream_mt_supported(params, cache) &&
      stream_mt_fits(params, cache, ((int64_t)total_q + params->batch - 1) / params->batch)) {
    size_t o_off, ml_off;
    ws = std::max(ws, stream_mt_workspace(params, cache, &o_off, &ml_off));
  }
  return ws;
}

pkv_status paged_attn_prefill(const void* q, const void* q_rope, const pkv_paged_cache* cache,
                              const int32_t* block_table, const int32_t* cu_seqlens_q, const int32_t* seq_lens_kv,
                              int32_t total_q, int32_t max_q_len, const pkv_attn_params* params, void* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  pkv_status s = check_cache(cache);
  if (s) return s;
  s = check_params(params, cache);
  if (s) return s;
  if (total_q < 0 || max_q_len < 0) return fail(PKV_ERR_INVALID_ARG, "total_q and max_q_len must be >= 0");
  // max_q_len sizes the grid: rows past it would never be computed.  The bound
  // itself lives in device memory (cu_seqlens_q); what the host can check is
  // that it is not impossible for these totals.
  if (params->batch > 0 && total_q > 0) {
    if (max_q_len == 0) return fail(PKV_ERR_INVALID_ARG, "max_q_len is 0 but total_q is %d", total_q);
    if ((int64_t)max_q_len * params->batch < total_q)
      return fail(PKV_ERR_INVALID_ARG, "max_q_len %d x batch %d is below total_q %d: some sequence has more rows",
                  max_q_len, params->batch, total_q);
    if (max_q_len > total_q)
      return fail(PKV_ERR_INVALID_ARG, "max_q_len %d exceeds total_q %d", max_q_len, total_q);
  }
  if (params->split_tokens != 0) return fail(PKV_ERR_INVALID_ARG, "split_tokens applies to decode only");
  if (is_int8(cache)) return fail(PKV_ERR_UNSUPPORTED, "prefill does not read int8 caches");
  if (params->batch == 0 || total_q == 0) return ok();
  if (!q || !block_table || !cu_seqlens_q || !seq_lens_kv || !out)
    return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  if ((q_rope != nullptr) != is_mla(cache))
    return fail(PKV_ERR_INVALID_ARG, "q_rope and k_rope must be given together or not at all");
  if (!aligned16(q) || !aligned16(out)) return fail(PKV_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
  if (is_mla(cache)) {
    // Absorbed-form prefill: every query row runs the MLA decode kernel as a
    // decode over the keys up to its position, whole (one partition per row:
    // rows x head groups give the workgroups, and no partials are kept).
    if (!pkv::mla_decode_supported(cache->dtype, cache->head_dim, cache->rope_dim, params->num_q_heads))
      return fail(PKV_ERR_UNSUPPORTED, "MLA prefill: needs bf16, latent 512, rope 64 and H a multiple of 16");
    if (!q_rope || !aligned16(q_rope)) return fail(PKV_ERR_INVALID_ARG, "MLA prefill: q_rope must be 16-byte aligned");
    int32_t span = params->max_blocks_per_seq;
    if (params->window > 0) span = std::min<int64_t>(span, (params->window + cache->block_size - 1) / cache->block_size + 1);
    if (span > kMaxBpp)
      return fail(PKV_ERR_UNSUPPORTED, "MLA prefill: a row may span %d blocks, more than %d", span, kMaxBpp);
    pkv::MlaArgs m{};
    m.q = q;
    m.q_rope = q_rope;
    m.c_nope = cache->k_cache;
    m.c_rope = cache->k_rope_cache;
    m.block_table = block_table;
    m.seq_lens = seq_lens_kv;
    m.out = out;
    m.batch = params->batch;
    m.num_q_heads = params->num_q_heads;
    m.max_blocks_per_seq = params->max_blocks_per_seq;
    m.block_size_log2 = log2i(cache->block_size);
    m.blocks_per_part = span;
    m.max_np = 1;
    m.window = params->window;
    m.scale_log2e = params->scale * pkv::kLog2e;
    m.out_dtype = params->out_dtype;
    m.cu_seqlens_q = cu_seqlens_q;
    m.rows = total_q;
    return from_hip(pkv::launch_mla_decode(m, static_cast<hipStream_t>(stream)), "MLA prefill launch");
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (stream_mt_supported(params, cache) && stream_mt_fits(params, cache, max_q_len)) {
    size_t o_off = 0, ml_off = 0;
    const size_t need = stream_mt_workspace(params, cache, &o_off, &ml_off);
    if (!workspace || workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    char* wsb = static_cast<char*>(workspace);
    pkv::DecodeArgs d{};
    d.q = q;
    d.k_cache = cache->k_cache;
    d.v_cache = cache->v_cache;
    d.block_table = block_table;
    d.seq_lens = seq_lens_kv;
    d.out = out;
    d.ws_o = reinterpret_cast<float*>(wsb + o_off);
    d.ws_ml = reinterpret_cast<float*>(wsb + ml_off);
    d.batch = params->batch;
    d.num_q_heads = params->num_q_heads;
    d.num_kv_heads = cache->num_kv_heads;
    d.head_dim = cache->head_dim;
    d.max_blocks_per_seq = params->max_blocks_per_seq;
    d.block_size_log2 = log2i(cache->block_size);
    d.blocks_per_part = 1;
    d.max_np = 1;
    d.window = params->window;
    d.scale_log2e = params->scale * pkv::kLog2e;
    d.dtype = cache->dtype;
    d.out_dtype = params->out_dtype;
    d.tile_prefix = reinterpret_cast<int32_t*>(wsb);
    d.resident_waves = pkv::decode_stream_resident_waves(device_cu_count(), cache->dtype);
    d.split_tiles = 0;
    d.cu_seqlens_q = cu_seqlens_q;
    d.total_q = total_q;
    return from_hip(pkv::launch_decode_stream(d, st), "multi-token decode launch");
  }
  if (params->max_blocks_per_seq > pkv::kPrefillMaxTableBlocks)
    return fail(PKV_ERR_UNSUPPORTED, "prefill: max_blocks_per_seq %d exceeds %d", params->max_blocks_per_seq,
                pkv::kPrefillMaxTableBlocks);
  if (!pkv::prefill_mfma_supported(cache->dtype, cache->head_dim))
    return fail(PKV_ERR_UNSUPPORTED, "prefill: needs bf16 and head_dim 64 or 128 (got dtype %d, head_dim %d)",
                cache->dtype, cache->head_dim);
  const PrefillPlan plan = plan_prefill(params, cache, total_q);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (plan.ws_bytes > 0 && !aligned16(workspace)) return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  pkv::PrefillArgs a{};
  a.max_np = plan.np;
  a.part_tiles = plan.part_tiles;
  a.ws_o = plan.ws_bytes > 0 ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = plan.ws_bytes > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ws_ml_offset) : nullptr;
  a.q = q;
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.block_table = block_table;
  a.cu_seqlens_q = cu_seqlens_q;
  a.seq_lens_kv = seq_lens_kv;
  a.out = out;
  a.batch = params->batch;
  a.num_q_heads = params->num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.max_blocks_per_seq = params->max_blocks_per_seq;
  a.block_size_log2 = log2i(cache->block_size);
  a.max_q_len = max_q_len;
  a.window = params->window;
  a.scale_log2e = params->scale * pkv::kLog2e;
  a.out_dtype = params->out_dtype;
  hipError_t e = pkv::launch_prefill_mfma(a, st);
  if (e != hipSuccess) return from_hip(e, "prefill launch");
  if (plan.np > 1) {
    // rows = total_q query rows x H heads, every partition written
    e = pkv::launch_decode_combine(a.ws_o, a.ws_ml, nullptr, total_q, params->num_q_heads, cache->head_dim,
                                   plan.np, a.block_size_log2, 0, params->window, out, params->out_dtype, st);
    if (e != hipSuccess) return from_hip(e, "prefill combine launch");
  }
  return ok();
}

}  // extern "C"

namespace pkv {
void set_last_error(const std::string& msg) { g_last_error = msg; }
void clear_last_error() { g_last_error.clear(); }
}  // namespace pkv
