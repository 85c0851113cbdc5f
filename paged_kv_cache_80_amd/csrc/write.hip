// write.hip -- index resolution and the slot-scatter cache writer.
//
// Address map of the "KVCache optimisation skill" page, section 3.1: a logical
// (sequence b, position p) lives in physical block block_table[b][p / bs] at
// offset p % bs, i.e. at slot block*bs + offset of the cache viewed as
// [num_blocks*bs, num_kv_heads, head_dim].  The writer is the scatter of the
// "Ascend NPU standalone-deployment KVCache guide", mode 2: row t of the new
// K (and V, and the MLA rope part) goes to cache row slot_mapping[t].
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void resolve_slots_kernel(const int32_t* __restrict__ block_table,
                                                            int32_t max_blocks_per_seq, int32_t bs_log2,
                                                            const int32_t* __restrict__ batch_idx,
                                                            const int32_t* __restrict__ pos, int32_t n,
                                                            int32_t* __restrict__ slots) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t p = pos[i];
  if (p < 0) {
    slots[i] = -1;
    return;
  }
  const int32_t b = batch_idx[i];
  const int32_t blk = block_table[(int64_t)b * max_blocks_per_seq + (p >> bs_log2)];
  slots[i] = (blk << bs_log2) + (p & ((1 << bs_log2) - 1));
}

// Slot of row t: given, or resolved from (batch_idx[t], pos[t]) as above, or --
// appending -- from (t, append_lens[t] - 1).
__device__ __forceinline__ int32_t slot_of(const SlotSource& s, int64_t t) {
  if (s.slot_mapping) return s.slot_mapping[t];
  const int32_t p = s.append_lens ? s.append_lens[t] - 1 : s.pos[t];
  if (p < 0) return -1;
  const int64_t b = s.append_lens ? t : (int64_t)s.batch_idx[t];
  const int32_t blk = s.block_table[b * s.max_blocks_per_seq + (p >> s.block_size_log2)];
  return (blk << s.block_size_log2) + (p & ((1 << s.block_size_log2) - 1));
}

// One workgroup per token.  The token's K, V and rope rows are treated as one
// list of 16-byte chunks; consecutive threads copy consecutive chunks, so every
// wave reads and writes whole 1 KiB runs of each row.  With the slots resolved
// here (kv_cache_write_at), the index resolution and the write are one launch.
__global__ __launch_bounds__(256) void cache_write_kernel(SlotSource slots, WriteRows rows) {
  const int32_t t = blockIdx.x;
  const int32_t slot = __builtin_amdgcn_readfirstlane(slot_of(slots, t));
  if (slots.slots_out && threadIdx.x == 0) slots.slots_out[t] = slot;
  if (slot < 0) return;
  for (int r = 0; r < rows.count; ++r) {
    const int32_t chunks = rows.row_bytes[r] >> 4;
    const char* src = static_cast<const char*>(rows.src[r]) + (int64_t)t * rows.row_bytes[r];
    char* dst = static_cast<char*>(rows.dst[r]) + (int64_t)slot * rows.row_bytes[r];
    for (int32_t c = threadIdx.x; c < chunks; c += blockDim.x) st16(dst + 16 * c, ld16(src + 16 * c));
  }
}

// Quantizing write into an int8 cache.  One group of 16 lanes per (token, head)
// row of 128 values; every lane holds 8 of them.  The row's scale is
// s = max|x| / 127 and its codes are rint(x * (127 / max|x|)) (both quotients
// IEEE float32, ties of rint to even), which leaves every code in [-127, 127];
// an all-zero row gets s = 0 and zero codes.  Groups take the K rows of all
// tokens first, then the V rows.
__global__ __launch_bounds__(256) void cache_write_int8_kernel(SlotSource slots, Int8WriteArgs a) {
  constexpr int kD = 128;
  const int64_t grp = (int64_t)blockIdx.x * (blockDim.x / 16) + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  const int64_t rows = (int64_t)a.num_tokens * a.num_kv_heads;  // rows of one tensor
  if (grp >= 2 * rows) return;                                  // whole groups leave together
  const bool is_v = grp >= rows;
  const int64_t r = is_v ? grp - rows : grp;
  const int64_t t = r / a.num_kv_heads;
  const int h = (int)(r - t * a.num_kv_heads);
  const int32_t slot = slot_of(slots, t);
  if (slots.slots_out && !is_v && h == 0 && l == 0) slots.slots_out[t] = slot;
  if (slot < 0) return;
  const uint4 w = ld16(static_cast<const uint16_t*>(is_v ? a.v : a.k) + r * kD + 8 * l);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = bf16_lo(u[k]);
    x[2 * k + 1] = bf16_hi(u[k]);
  }
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  m = group_max<16>(m);
  const float scale = m / 127.f;
  const float inv = m > 0.f ? 127.f / m : 0.f;
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = (int)fminf(fmaxf(rintf(x[e] * inv), -127.f), 127.f);
    packed[e >> 2] |= ((uint32_t)c & 0xffu) << (8 * (e & 3));
  }
  char* dst = static_cast<char*>(is_v ? a.v_cache : a.k_cache) + ((int64_t)slot * a.num_kv_heads + h) * kD + 8 * l;
  *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
  if (l == 0) {
    const int32_t blk = slot >> a.block_size_log2;
    const int32_t off = slot & ((1 << a.block_size_log2) - 1);
    float* sc = is_v ? a.v_scale : a.k_scale;
    sc[(((int64_t)blk * a.num_kv_heads + h) << a.block_size_log2) + off] = scale;
  }
}

hipError_t launch_resolve_slots(const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                                int32_t block_size, const int32_t* batch_idx, const int32_t* pos,
                                int32_t n, int32_t* slots_out, hipStream_t stream) {
  (void)batch;
  if (n == 0) return hipSuccess;
  const int32_t bs_log2 = __builtin_ctz((unsigned)block_size);
  resolve_slots_kernel<<<(n + 255) / 256, 256, 0, stream>>>(block_table, max_blocks_per_seq, bs_log2,
                                                            batch_idx, pos, n, slots_out);
  return hipGetLastError();
}

hipError_t launch_cache_write(const SlotSource& slots, int32_t num_tokens, const WriteRows& rows,
                              hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  cache_write_kernel<<<num_tokens, 256, 0, stream>>>(slots, rows);
  return hipGetLastError();
}

hipError_t launch_cache_write_int8(const SlotSource& slots, const Int8WriteArgs& a, hipStream_t stream) {
  const int64_t groups = 2 * (int64_t)a.num_tokens * a.num_kv_heads;
  if (groups == 0) return hipSuccess;
  cache_write_int8_kernel<<<(unsigned)((groups + 15) / 16), 256, 0, stream>>>(slots, a);
  return hipGetLastError();
}

}  // namespace pkv
