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

// One workgroup per token.  The token's K, V and rope rows are treated as one
// list of 16-byte chunks; consecutive threads copy consecutive chunks, so every
// wave reads and writes whole 1 KiB runs of each row.
__global__ __launch_bounds__(256) void cache_write_kernel(const int32_t* __restrict__ slot_mapping,
                                                          WriteRows rows) {
  const int32_t t = blockIdx.x;
  const int32_t slot = slot_mapping[t];
  if (slot < 0) return;
  for (int r = 0; r < rows.count; ++r) {
    const int32_t chunks = rows.row_bytes[r] >> 4;
    const char* src = static_cast<const char*>(rows.src[r]) + (int64_t)t * rows.row_bytes[r];
    char* dst = static_cast<char*>(rows.dst[r]) + (int64_t)slot * rows.row_bytes[r];
    for (int32_t c = threadIdx.x; c < chunks; c += blockDim.x) st16(dst + 16 * c, ld16(src + 16 * c));
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

hipError_t launch_cache_write(const int32_t* slot_mapping, int32_t num_tokens, const WriteRows& rows,
                              hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  cache_write_kernel<<<num_tokens, 256, 0, stream>>>(slot_mapping, rows);
  return hipGetLastError();
}

}  // namespace pkv
