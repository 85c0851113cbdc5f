// pkv_internal.h -- host-side declarations shared by the C-ABI layer and the kernel
// translation units of libpkv.  Not installed; the public interface is include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Index resolution and cache write (write.hip).
hipError_t launch_resolve_slots(const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                                int32_t block_size, const int32_t* batch_idx, const int32_t* pos,
                                int32_t n, int32_t* slots_out, hipStream_t stream);

// rows: up to three source/destination pairs copied per token (K, V, rope).
struct WriteRows {
  const void* src[3];
  void* dst[3];
  int32_t row_bytes[3];
  int32_t count;
};
// Where a write's rows go: slot_mapping[t], or -- the fused form -- the slot of
// (batch_idx[t], pos[t]) resolved through block_table, stored to slots_out too
// when that is given (a negative pos gives -1: the row is skipped).
struct SlotSource {
  const int32_t* slot_mapping;  // non-null: the slots are given
  const int32_t* block_table;
  const int32_t* batch_idx;
  const int32_t* pos;
  // non-null: row t is the newest token of sequence t, at position append_lens[t] - 1
  // (a length of 0 writes nothing); batch_idx and pos are then unused
  const int32_t* append_lens;
  int32_t* slots_out;
  int32_t max_blocks_per_seq, block_size_log2;
};
hipError_t launch_cache_write(const SlotSource& slots, int32_t num_tokens, const WriteRows& rows,
                              hipStream_t stream);

// Quantizing cache write into an int8 cache (write.hip): every (token, head) row
// of 128 bf16 values of k and v becomes 128 int8 codes and one float32 scale.
struct Int8WriteArgs {
  const void* k;      // [num_tokens, num_kv_heads, 128] bf16
  const void* v;
  void* k_cache;      // [slots, num_kv_heads, 128] int8
  void* v_cache;
  float* k_scale;     // [num_blocks, num_kv_heads, block_size]
  float* v_scale;
  int32_t num_tokens, num_kv_heads, block_size_log2;
};
hipError_t launch_cache_write_int8(const SlotSource& slots, const Int8WriteArgs& a, hipStream_t stream);

// Fused RMSNorm + RoPE + cache write of the MLA latent (latent_write.hip).
// Latent width 512, rotary width 64, one latent head; every array in one dtype.
struct LatentWriteArgs {
  const void* latent;           // [num_tokens, 512 + 64]
  const void* gamma;            // [512]
  const void* cos;              // [num_tokens, 64]
  const void* sin;              // [num_tokens, 64]
  const int32_t* slot_mapping;  // [num_tokens]; negative: no cache write
  void* cache_nope;             // [slots, 512]
  void* cache_rope;             // [slots, 64]
  void* out_nope;               // [num_tokens, 512] or NULL (then out_rope is NULL too)
  void* out_rope;               // [num_tokens, 64]
  int64_t num_tokens;
  float eps;
  int32_t bf16;
  int32_t interleaved;
};
hipError_t launch_latent_write(const LatentWriteArgs& a, hipStream_t stream);

// Split-K decode on the vector ALUs (decode.hip).
struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;
  float* ws_o;   // [B*H, max_np, D] partial outputs (unnormalised), or null when max_np == 1
  float* ws_ml;  // [B*H, max_np, 2] running max (log2 domain) and sum
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  int32_t max_blocks_per_seq, block_size_log2;
  int32_t blocks_per_part, max_np;
  int32_t window;
  float scale_log2e;
  int32_t dtype, out_dtype;
  // Stream split (decode_mfma.hip) only: per-sequence tile prefix [batch + 1]
  // in the workspace, the resident waves launched, and an optional target of
  // tiles per wave (0 = spread over every resident wave).
  int32_t* tile_prefix;
  int32_t resident_waves;
  int32_t split_tiles;
  // int8 caches (dtype PKV_INT8, stream split only): per (slot, head) scales in
  // [num_blocks, num_kv_heads, block_size] order.
  const float* k_scale;
  const float* v_scale;
  // Multi-token decode through the stream split (bf16): the rows of sequence b
  // are q rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 at its last positions;
  // null in decode.  total_q: all rows.
  const int32_t* cu_seqlens_q;
  int32_t total_q;
  // Decode with the step's append fused in (bf16 stream split): each sequence's
  // newest K and V rows [batch, num_kv_heads, 128].  The key at position
  // seq_lens[b] - 1 is read from here instead of the cache, and the wave that
  // reads it also stores it at its slot.  Null otherwise.
  const void* k_new;
  const void* v_new;
  // Vector-ALU decode only: waves per workgroup, 4 (a workgroup per partition of
  // blocks_per_part blocks) or 16 (a workgroup per whole sequence, max_np == 1).
  int32_t valu_waves;
};
hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream);
bool decode_valu_supported(int32_t dtype, int32_t head_dim, int32_t group);
// Whether the 16-wave whole-sequence variant serves this shape.
bool decode_valu_wide_supported(int32_t dtype, int32_t head_dim, int32_t group);
// The same decode on the matrix cores with a stream split (decode_mfma.hip):
// bf16 or int8 caches, head_dim 128, head groups up to 16.  Launches the tile scan, the decode
// and the piece combine.
bool decode_mfma_supported(int32_t dtype, int32_t head_dim, int32_t group);
int32_t decode_stream_resident_waves(int32_t cu_count, int32_t dtype);
// Workspace of a stream-split call whose pieces hold `columns` columns (the head
// group in decode, kStreamMtColumns in multi-token decode).
size_t decode_stream_workspace(int32_t batch, int32_t columns, int32_t num_kv_heads, int32_t resident_waves,
                               size_t* ws_o_offset, size_t* ws_ml_offset);
// Multi-token decode through the stream split: (row, head) columns per KV head.
constexpr int32_t kStreamMtColumns = 32;
hipError_t launch_decode_stream(const DecodeArgs& a, hipStream_t stream);

// Second pass of split-K decode: merges the partitions of each (sequence, head).
hipError_t launch_decode_combine(const float* ws_o, const float* ws_ml, const int32_t* seq_lens,
                                 int32_t batch, int32_t num_q_heads, int32_t v_dim, int32_t max_np,
                                 int32_t block_size_log2, int32_t blocks_per_part, int32_t window,
                                 void* out, int32_t out_dtype, hipStream_t stream);

// Chunked causal prefill on MFMA (prefill.hip).
struct PrefillArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* cu_seqlens_q;
  const int32_t* seq_lens_kv;
  void* out;
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  int32_t max_blocks_per_seq, block_size_log2, max_q_len, window;
  float scale_log2e;
  int32_t out_dtype;
  int32_t q_tiles;  // query tiles per (sequence, KV head); set by the launcher
  // Key split: with max_np > 1, workgroup partition y covers key tiles
  // [y * part_tiles, (y + 1) * part_tiles) and leaves unnormalised partials
  // ([total_q * H, max_np, head_dim] and (m, l) pairs) for the split-K combine.
  int32_t max_np, part_tiles;
  float* ws_o;
  float* ws_ml;
};
// Query columns ((row, head) pairs of one KV head) per prefill workgroup, and keys
// per tile; the host sizes the key split with them.
constexpr int32_t kPrefillColumns = 128;
constexpr int32_t kPrefillKeyTile = 64;
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream);
// Widest block table the prefill kernel stages in LDS (256K tokens at 128-token blocks).
constexpr int32_t kPrefillMaxTableBlocks = 2048;
bool prefill_mfma_supported(int32_t dtype, int32_t head_dim);

// MLA absorbed decode on MFMA (mla.hip); partials share the decode workspace layout.
struct MlaArgs {
  const void* q;       // [rows, H, 512]
  const void* q_rope;  // [rows, H, 64]
  const void* c_nope;  // [num_blocks, bs, 1, 512]
  const void* c_rope;  // [num_blocks, bs, 1, 64]
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;
  float* ws_o;
  float* ws_ml;
  int32_t batch, num_q_heads;
  int32_t max_blocks_per_seq, block_size_log2, blocks_per_part, max_np, window;
  float scale_log2e;
  int32_t out_dtype;
  const int32_t* cu_seqlens_q;  // prefill: [batch + 1] row offsets of the sequences; decode: null
  int32_t rows;                 // query rows: batch (decode) or total_q (prefill)
  int32_t row0;                 // first row of this launch (set by launch_mla_decode)
};
hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t stream);
bool mla_decode_supported(int32_t dtype, int32_t head_dim, int32_t rope_dim, int32_t num_q_heads);

}  // namespace pkv
