// device_common.h -- small device helpers shared by the gfx950 kernels of libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

// ---- bfloat16 <-> float ---------------------------------------------------
// bf16 -> f32 is exact: the bf16 bits are the top half of the f32 bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// f32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- cross-lane reductions --------------------------------------------------
// DPP moves within a row of 16 lanes.  Every lane must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;       // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;       // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within each 16

// Sum over aligned groups of N consecutive lanes (N a power of two <= 64); every
// lane of a group ends with the group's sum.  Steps run in the order 1, 2, 4, 8
// so that the mirror moves always pair lanes that already hold equal partial sums.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_mov<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_mov<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_mov<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_mov<kDppMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp_mov<kDppXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_mov<kDppXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_mov<kDppMirror>(v));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// 2^x on the hardware exponential unit; 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// Rescale factor exp2(m_old - m_new) of the online softmax.  m_new == -inf means
// nothing was seen yet on either side: the factor is irrelevant, return 1.
__device__ __forceinline__ float rescale(float m_old, float m_new) {
  return m_new == kNegInf ? 1.0f : exp2_fast(m_old - m_new);
}

// ---- 16-byte global loads/stores --------------------------------------------
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

}  // namespace pkv

namespace pkv {

// Keys of one sequence that a decode query sees, and how they split into
// partitions of `bpp` table blocks.  The query sits at position L-1; with a
// window W it sees positions L-W .. L-1 (W keys including itself), otherwise
// 0 .. L-1.  Partition p covers logical blocks first_blk + p*bpp ... so table
// entries before first_blk (expired blocks, possibly the null block) are never read.
struct KeySpan {
  int32_t lo;         // first visible position
  int32_t hi;         // one past the last visible position (= L)
  int32_t first_blk;  // logical block holding `lo`
  int32_t np;         // number of partitions (0 when L == 0)
};

__host__ __device__ __forceinline__ KeySpan decode_span(int32_t L, int32_t window, int32_t bs_log2,
                                                        int32_t bpp) {
  KeySpan s;
  s.hi = L;
  s.lo = (window > 0 && L > window) ? L - window : 0;
  if (L <= 0) {
    s.lo = 0;
    s.first_blk = 0;
    s.np = 0;
    return s;
  }
  s.first_blk = s.lo >> bs_log2;
  const int32_t last_blk = (L - 1) >> bs_log2;
  s.np = (last_blk - s.first_blk) / bpp + 1;
  return s;
}

}  // namespace pkv
