// mfma_common.h -- helpers for the bf16 matrix-core (MFMA) attention kernels.
//
// v_mfma_f32_16x16x32_bf16 computes D[16x16] += A[16x32] * B[32x16] per wave.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each as 8 bf16
// covering the contraction slots of lane group l / 16; the same slot function is
// used for A and B, so any consistent assignment of contraction indices to
// (lane group, element) pairs computes the same sum.  D comes back as 4 floats
// per lane: D[4*(l/16) + r][l % 16], r = 0..3.
//
// Both attention products are taken in transposed form so that a lane's query
// column never changes:
//     S^T[key, col] = sum_d K[key, d] * Q[col, d]        (A = K tile, B = Q^T)
//     O^T[d, col]  += sum_key V^T[d, key] * P^T[key, col] (A = V^T tile, B = P^T)
// S^T's accumulator layout (lane holds column l%16, keys 4*(l/16)+r of a 16-key
// sub-tile) is exactly the B-operand layout P^T needs for a 32-key step when the
// contraction slot e of lane group g means key 4g+e (e < 4) or 16+4g+(e-4) (e >= 4).
#pragma once

#include "device_common.h"
#include "pkv.h"

namespace pkv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t mfma_bf16(const u32x4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t f32x4_zero() {
  f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// Probabilities in [0, 1] split as p = hi + lo + r with hi, lo bf16 (both taken
// by truncation, |r| < 2^-15 p), so two bf16 products carry p to ~16 bits: the
// P.V product keeps fp32-class accuracy instead of bf16's 2^-9.
__device__ __forceinline__ void split_bf16(float p, uint32_t& hi, uint32_t& lo) {
  const uint32_t u = __float_as_uint(p);
  hi = u & 0xffff0000u;
  const float r = p - __uint_as_float(hi);  // exact
  lo = __float_as_uint(r) & 0xffff0000u;
}

// Pack 8 probabilities (slot order) into hi and lo bf16x8 operands.
__device__ __forceinline__ void pack_p(const float* p8, uint4& hi, uint4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) split_bf16(p8[e], h[e], l[e]);
  hi.x = (h[0] >> 16) | h[1];
  hi.y = (h[2] >> 16) | h[3];
  hi.z = (h[4] >> 16) | h[5];
  hi.w = (h[6] >> 16) | h[7];
  lo.x = (l[0] >> 16) | l[1];
  lo.y = (l[2] >> 16) | l[3];
  lo.z = (l[4] >> 16) | l[5];
  lo.w = (l[6] >> 16) | l[7];
}

// Two bf16 of two keys at one dimension, low half = first key.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// Interleave 8 bf16 of key k0 (a) and key k1 (b) into 8 dwords, one per dimension.
__device__ __forceinline__ void interleave_pairs(const uint4& a, const uint4& b, uint32_t* w) {
  w[0] = pair_lo(a.x, b.x);
  w[1] = pair_hi(a.x, b.x);
  w[2] = pair_lo(a.y, b.y);
  w[3] = pair_hi(a.y, b.y);
  w[4] = pair_lo(a.z, b.z);
  w[5] = pair_hi(a.z, b.z);
  w[6] = pair_lo(a.w, b.w);
  w[7] = pair_hi(a.w, b.w);
}

// p0, p1 -> one dword holding bf16 truncations of both (p0 in the low half):
// v_perm_b32 picks bytes 2,3 of p0 and bytes 2,3 of p1.
__device__ __forceinline__ uint32_t pack_hi16(float p0, float p1) {
  return __builtin_amdgcn_perm(__float_as_uint(p1), __float_as_uint(p0), 0x07060302u);
}

// Split 8 probabilities (slot order) into hi and lo bf16x8 operands with
// p = hi + lo + r, |r| < 2^-15 p (hi and lo both truncated; p - hi is exact).
__device__ __forceinline__ void pack_p_split(const float* p8, uint4& hi, uint4& lo) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = p8[e] - __uint_as_float(__float_as_uint(p8[e]) & 0xffff0000u);
  hi.x = pack_hi16(p8[0], p8[1]);
  hi.y = pack_hi16(p8[2], p8[3]);
  hi.z = pack_hi16(p8[4], p8[5]);
  hi.w = pack_hi16(p8[6], p8[7]);
  lo.x = pack_hi16(r[0], r[1]);
  lo.y = pack_hi16(r[2], r[3]);
  lo.z = pack_hi16(r[4], r[5]);
  lo.w = pack_hi16(r[6], r[7]);
}

// Column maximum / sum over the four 16-lane rows of a wave (lanes l, l^16,
// l^32, l^48): v_permlane16_swap / v_permlane32_swap exchange rows in the VALU,
// with no LDS round trip.  With both operands equal, the two results of a swap
// hold the value of the lane and of its partner row in some order, so their
// maximum (sum) is the pairwise maximum (sum) on every lane.
__device__ __forceinline__ float row4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float row4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// ---- gfx950 LDS paths -------------------------------------------------------
// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane
// l's bytes land at lds_base + 16*l, lds_base being the same for the whole wave
// (it travels in M0).  The copy is asynchronous and counted by vmcnt.
//
// It is issued from inline assembly on purpose: the compiler treats an LDS DMA
// it can see as a store that may alias every later LDS read and puts
// s_waitcnt vmcnt(0) in front of them, which serialises a double buffer (the
// prefetch of tile t+1 would have to land before tile t is read).  Untracked,
// the DMA only makes the compiler's own vmcnt waits more conservative (vector
// memory operations retire in order), and the kernels wait for their buffers
// explicitly with wait_vmem / wait_vmem_n before a barrier or a read.  M0 is
// written and consumed inside the one asm statement.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void load_lds16(const void* gsrc, const void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)(lds_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(lds)
               : "memory", "m0");
}
// The same copy with a wave-uniform 64-bit base (SGPRs) and a 32-bit lane offset.
__device__ __forceinline__ void load_lds16_s(const void* sbase, uint32_t voff, const void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)(lds_base));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// vmcnt(0) as a real instruction the compiler's waitcnt pass sees: after it no
// compiler-tracked load is outstanding, so no wait for them lands inside a loop
// body (where it would also stall on the untracked prefetch).  gfx9 encoding:
// vmcnt 0, expcnt 7, lgkmcnt 15.
__device__ __forceinline__ void retire_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N == 0 || N == 8 || N == 16 || N == 24 || N == 32 || N == 36 || N == 48, "add a case");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  if constexpr (N == 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  if constexpr (N == 32) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  if constexpr (N == 36) asm volatile("s_waitcnt vmcnt(36)" ::: "memory");
  if constexpr (N == 48) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives 16-bit element (i % 4) of the 8-byte reads of lanes
// 4k + i/4, k = 0..3.  If lane j of a group addresses row R0 + j/4 at column
// C0 + 4*(j%4) of a row-major tile, lane i gets tile[R0 + k][C0 + i], k = 0..3:
// a column of four rows, i.e. the MFMA operand of the transposed tile.
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Transposing LDS read of bytes (ds_read_b64_tr_b8): within each group of 16
// lanes, lane i receives byte (i % 8) of the 8-byte reads of lanes 2k + i/8,
// k = 0..7.  If lane j of a group reads row R0 + j/2 at column C0 + 8*(j%2) of a
// row-major byte tile, lane i gets tile[R0 + k][C0 + i], k = 0..7.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
__device__ __forceinline__ uint2 lds_tr8(const void* p) {
  const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Eight int8 values (bytes 0..7 of w) as eight bf16 (exact: |q| <= 128 needs at
// most 8 significant bits).  Each byte is sign-extended and converted to f32,
// whose top half is the bf16.
__device__ __forceinline__ uint4 i8x8_to_bf16(const uint2& w) {
  uint32_t o[4];
  const uint32_t u[2] = {w.x, w.y};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int32_t x = (int32_t)u[k];
    const float f0 = (float)((x << 24) >> 24), f1 = (float)((x << 16) >> 24);
    const float f2 = (float)((x << 8) >> 24), f3 = (float)(x >> 24);
    o[2 * k] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    o[2 * k + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint4 lds16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 lds8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

// Store 4 consecutive output elements of one row.
__device__ __forceinline__ void store4(void* out, int64_t idx, const float* v, int32_t out_dtype) {
  if (out_dtype == PKV_BF16) {
    uint2 w;
    w.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    w.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = w;
  } else {
    uint4 w;
    w.x = __float_as_uint(v[0]);
    w.y = __float_as_uint(v[1]);
    w.z = __float_as_uint(v[2]);
    w.w = __float_as_uint(v[3]);
    *reinterpret_cast<uint4*>(static_cast<float*>(out) + idx) = w;
  }
}

}  // namespace pkv
