// latent_write.hip -- fused RMSNorm + RoPE + paged cache write of the MLA latent.
//
// The fused writer of the MLA absorbed form ("Ascend NPU standalone-deployment
// KVCache guide", MLA section; "KVCache optimisation skill", the fused
// cache-write operator fed by slot_mapping): the row the KV down-projection
// produces for a token is [c (512) | k_pe (64)]; c is RMS-normalised and scaled
// by gamma, k_pe is turned pairwise by the token's cos/sin, and both land in the
// paged cache at the token's slot (and, when asked, in dense output rows).
//
// The work is a stream: every byte is read or written once and the arithmetic
// is a few operations per element, so HBM bandwidth bounds it.  One wavefront
// owns TPW tokens and issues all their loads (16-byte chunks, the 512-wide
// latent spread over the 64 lanes, the 64-wide rotary part, cos and sin over the
// first few lanes) before any arithmetic.  One token per wave measured fastest
// (more resident waves beat more bytes per wave).  The sum of squares is a wave
// reduction on DPP and one permute; the rotate-half partner sits rope_dim/2
// elements away, a fixed lane distance for 16-byte chunks, so it comes over
// with one permute per word.  Stores carry the nontemporal hint: this kernel
// never reads the rows back, and the hint measured faster than plain stores.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kRank = 512;  // latent width (kv_lora_rank)
constexpr int kRope = 64;   // rotary width

template <int EPC>
__device__ __forceinline__ void unpack(const uint4& w, float (&v)[EPC]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  if constexpr (EPC == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_lo(u[k]);
      v[2 * k + 1] = bf16_hi(u[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __uint_as_float(u[k]);
  }
}

template <int EPC>
__device__ __forceinline__ uint4 pack(const float (&v)[EPC]) {
  uint32_t u[4];
  if constexpr (EPC == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) u[k] = (uint32_t)f32_to_bf16(v[2 * k]) | ((uint32_t)f32_to_bf16(v[2 * k + 1]) << 16);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) u[k] = __float_as_uint(v[k]);
  }
  return make_uint4(u[0], u[1], u[2], u[3]);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte store with the nontemporal hint (streamed past the caches).
__device__ __forceinline__ void store16(void* p, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ uint4 shfl_xor16(const uint4& w, int m) {
  return make_uint4(__shfl_xor((int)w.x, m), __shfl_xor((int)w.y, m), __shfl_xor((int)w.z, m),
                    __shfl_xor((int)w.w, m));
}

}  // namespace

// EPC: elements per 16-byte chunk (8 for bf16, 4 for f32).  INTERLEAVED: the
// rotary pairs are (2k, 2k+1); otherwise element i pairs with i +- 32.
template <int EPC, bool INTERLEAVED, int TPW>
__global__ __launch_bounds__(256) void latent_write_kernel(LatentWriteArgs a) {
  constexpr int EB = 16 / EPC;              // bytes per element
  constexpr int NC = kRank / EPC / kWave;   // latent chunks per lane: 1 (bf16) or 2 (f32)
  constexpr int RC = kRope / EPC;           // rotary chunks per row: 8 or 16
  constexpr int64_t kRowIn = (kRank + kRope) * EB;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t0 = ((int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave)) * TPW;
  if (t0 >= a.num_tokens) return;
  const int ntok = (int)min<int64_t>(TPW, a.num_tokens - t0);  // wave-uniform
  const char* lat = static_cast<const char*>(a.latent);
  const char* cosp = static_cast<const char*>(a.cos);
  const char* sinp = static_cast<const char*>(a.sin);
  const bool rope_lane = lane < RC;

  uint4 xn[TPW][NC], xr[TPW], cs[TPW], sn[TPW];
  int32_t slot[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (u < ntok) {
      const int64_t t = t0 + u;
      slot[u] = a.slot_mapping[t];
#pragma unroll
      for (int k = 0; k < NC; ++k) xn[u][k] = ld16(lat + t * kRowIn + (lane + kWave * k) * 16);
      if (rope_lane) {
        xr[u] = ld16(lat + t * kRowIn + kRank * EB + lane * 16);
        cs[u] = ld16(cosp + t * (kRope * EB) + lane * 16);
        sn[u] = ld16(sinp + t * (kRope * EB) + lane * 16);
      }
    }
  }
  float g[NC][EPC];
#pragma unroll
  for (int k = 0; k < NC; ++k) unpack<EPC>(ld16(static_cast<const char*>(a.gamma) + (lane + kWave * k) * 16), g[k]);

#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (u >= ntok) break;
    const int64_t t = t0 + u;
    // RMSNorm of the latent part.
    float v[NC][EPC];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      unpack<EPC>(xn[u][k], v[k]);
#pragma unroll
      for (int e = 0; e < EPC; ++e) ss = fmaf(v[k][e], v[k][e], ss);
    }
    ss = group_sum<kWave>(ss);
    const float r = 1.0f / sqrtf(ss * (1.0f / kRank) + a.eps);
    uint4 on[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      float o[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) o[e] = (v[k][e] * r) * g[k][e];
      on[k] = pack<EPC>(o);
    }
    // RoPE of the rotary part.  The partner permute runs on every lane.
    uint4 pr = xr[u];
    if constexpr (!INTERLEAVED) pr = shfl_xor16(xr[u], RC / 2);
    uint4 orr = make_uint4(0, 0, 0, 0);
    if (rope_lane) {
      float x[EPC], p[EPC], c[EPC], s[EPC], o[EPC];
      unpack<EPC>(xr[u], x);
      unpack<EPC>(pr, p);
      unpack<EPC>(cs[u], c);
      unpack<EPC>(sn[u], s);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float other = INTERLEAVED ? p[e ^ 1] : p[e];
        const bool second = INTERLEAVED ? (e & 1) != 0 : lane >= RC / 2;
        o[e] = x[e] * c[e] + (second ? other : -other) * s[e];
      }
      orr = pack<EPC>(o);
    }
    // Stores: the cache rows at the slot, then the dense rows.
    if (slot[u] >= 0) {
      char* dn = static_cast<char*>(a.cache_nope) + (int64_t)slot[u] * (kRank * EB);
#pragma unroll
      for (int k = 0; k < NC; ++k) store16(dn + (lane + kWave * k) * 16, on[k]);
      if (rope_lane) store16(static_cast<char*>(a.cache_rope) + (int64_t)slot[u] * (kRope * EB) + lane * 16, orr);
    }
    if (a.out_nope) {
      char* dn = static_cast<char*>(a.out_nope) + t * (kRank * EB);
#pragma unroll
      for (int k = 0; k < NC; ++k) store16(dn + (lane + kWave * k) * 16, on[k]);
      if (rope_lane) store16(static_cast<char*>(a.out_rope) + t * (kRope * EB) + lane * 16, orr);
    }
  }
}

hipError_t launch_latent_write(const LatentWriteArgs& a, hipStream_t stream) {
  if (a.num_tokens <= 0) return hipSuccess;
  constexpr int kTpw = 1;
  const int64_t waves = (a.num_tokens + kTpw - 1) / kTpw;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (a.bf16) {
    if (a.interleaved) latent_write_kernel<8, true, kTpw><<<grid, block, 0, stream>>>(a);
    else latent_write_kernel<8, false, kTpw><<<grid, block, 0, stream>>>(a);
  } else {
    if (a.interleaved) latent_write_kernel<4, true, kTpw><<<grid, block, 0, stream>>>(a);
    else latent_write_kernel<4, false, kTpw><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace pkv
