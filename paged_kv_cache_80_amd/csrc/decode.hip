// decode.hip -- paged decode (q_len = 1) on the vector ALUs, split over workgroups.
//
// Computes, for each sequence b and query head h,
//     out[b,h] = sum_j softmax_j(q[b,h] . k_j * scale) v_j
// over the keys j the newest position sees ("KV Cache notes": the attention
// formula and its per-token decode form; keys of the KV head h / (H/H_kv),
// section "MHA -> MQA -> GQA"), reading K/V rows through the block table
// ("KVCache optimisation skill", section 3.1).
//
// Work split.  One workgroup (4 waves) owns one (sequence, KV head, partition)
// where a partition is `blocks_per_part` consecutive table blocks; a call whose
// sequences would take at most 4 partitions runs one 16-wave workgroup per
// (sequence, KV head) instead, over the whole sequence.  All G query heads that
// share the KV head are processed together, so every K/V row is read from HBM
// once per step (the GQA sharing of the pages' repeat_kv, done at read time).
// Each 16-byte lane chunk holds 8 bf16 (or 4 f32) of a row; LPR = D / (elements
// per chunk) lanes cover one row, a wave covers 64/LPR rows per load and each
// lane keeps U rows of K and of V in flight per iteration.
//
// Online softmax (running max m, sum l, rescale by 2^(m_old - m_new)) is kept
// per lane over the rows that lane's row group saw; logits are in log2 units
// (scale * log2 e folded in) so every exponential is one v_exp_f32.  Row dot
// products are reduced across the LPR lanes with DPP moves; the end of a
// partition merges row groups with lane shuffles and waves through LDS.  A
// single partition writes the normalised output directly; otherwise the
// partial (m, l, o) goes to the workspace and decode_combine merges them.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
// A whole sequence per workgroup: 16 waves stream 4x the keys of a 4-wave
// partition per iteration and merge in LDS, so a call that would cut each
// sequence into at most 4 partitions runs as one kernel, with no partials and
// no combine.  Only where the per-wave state fits, unspilled, the 128 registers
// a lane has at 16 waves per CU: fp32 rows of up to 256 elements over the head
// group (4 elements a lane chunk), bf16 (8 a chunk) with one head per KV head.
constexpr int kWideWaves = 16;
constexpr bool wide_fits(int elem_bytes, int D, int GT) { return elem_bytes == 4 ? GT * D <= 256 : GT == 1; }
constexpr int kMaxBpp = 1024;  // table blocks per partition held in LDS

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

template <typename T>
struct QChunk;

// f32: 4 query values as floats.
template <>
struct QChunk<float> {
  float v[4];
  __device__ void load(const float* p) {
    const uint4 w = ld16(p);
    v[0] = __uint_as_float(w.x);
    v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z);
    v[3] = __uint_as_float(w.w);
  }
  __device__ void zero() { v[0] = v[1] = v[2] = v[3] = 0.f; }
  __device__ float dot(const uint4& k) const {
    float s = v[0] * __uint_as_float(k.x);
    s = fmaf(v[1], __uint_as_float(k.y), s);
    s = fmaf(v[2], __uint_as_float(k.z), s);
    s = fmaf(v[3], __uint_as_float(k.w), s);
    return s;
  }
};

// bf16: 8 query values kept as raw bf16 pairs; products are exact in f32 and
// accumulate in f32 (v_dot2_f32_bf16).
template <>
struct QChunk<uint16_t> {
  uint32_t w[4];
  __device__ void load(const uint16_t* p) {
    const uint4 x = ld16(p);
    w[0] = x.x;
    w[1] = x.y;
    w[2] = x.z;
    w[3] = x.w;
  }
  __device__ void zero() { w[0] = w[1] = w[2] = w[3] = 0u; }
  __device__ float dot(const uint4& k) const {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[0]),
                                              __builtin_bit_cast(bf16x2_t, k.x), 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[1]),
                                        __builtin_bit_cast(bf16x2_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[2]),
                                        __builtin_bit_cast(bf16x2_t, k.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[3]),
                                        __builtin_bit_cast(bf16x2_t, k.w), s, false);
    return s;
  }
};

// acc[e] += p * v[e] for the elements of one 16-byte V chunk.
__device__ __forceinline__ void axpy_chunk(float* acc, float p, const uint4& v, float) {
  acc[0] = fmaf(p, __uint_as_float(v.x), acc[0]);
  acc[1] = fmaf(p, __uint_as_float(v.y), acc[1]);
  acc[2] = fmaf(p, __uint_as_float(v.z), acc[2]);
  acc[3] = fmaf(p, __uint_as_float(v.w), acc[3]);
}
__device__ __forceinline__ void axpy_chunk(float* acc, float p, const uint4& v, uint16_t) {
  acc[0] = fmaf(p, bf16_lo(v.x), acc[0]);
  acc[1] = fmaf(p, bf16_hi(v.x), acc[1]);
  acc[2] = fmaf(p, bf16_lo(v.y), acc[2]);
  acc[3] = fmaf(p, bf16_hi(v.y), acc[3]);
  acc[4] = fmaf(p, bf16_lo(v.z), acc[4]);
  acc[5] = fmaf(p, bf16_hi(v.z), acc[5]);
  acc[6] = fmaf(p, bf16_lo(v.w), acc[6]);
  acc[7] = fmaf(p, bf16_hi(v.w), acc[7]);
}

__device__ __forceinline__ void store_out(void* out, int64_t i, float x, int32_t out_dtype) {
  if (out_dtype == PKV_BF16)
    static_cast<uint16_t*>(out)[i] = f32_to_bf16(x);
  else
    static_cast<float*>(out)[i] = x;
}

template <typename T, int D, int GT, int U, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_valu_kernel(DecodeArgs a) {
  constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane chunk
  constexpr int LPR = D / EPL;              // lanes per row
  constexpr int RPW = kWave / LPR;          // rows per wave load
  constexpr int CH = NW * RPW * U;          // tokens per iteration
  static_assert(LPR >= 1 && LPR <= kWave && (kWave % LPR) == 0, "row must fit a wave");

  __shared__ int32_t s_blk[kMaxBpp];
  __shared__ float s_m[NW][GT];
  __shared__ float s_l[NW][GT];
  __shared__ float s_acc[NW][GT][D];

  // The grid is (KV head, sequence) x partition with the KV head fastest.
  // Workgroups are dealt to the 8 XCDs round-robin in launch order, so KV head
  // g of every sequence runs on XCD (g + H_kv * b) mod 8: each XCD streams whole
  // heads of whole sequences, and ragged lengths cannot pile the work of short
  // sequences (which only have low partition indices) onto a few XCDs.
  const int g = blockIdx.x % a.num_kv_heads;
  const int b = blockIdx.x / a.num_kv_heads;
  const int part = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int c = lane % LPR;
  const int rg = lane / LPR;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t qrow0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;  // row b*H + h of head g*G

  const int32_t L = a.seq_lens[b];
  const KeySpan sp = decode_span(L, a.window, a.block_size_log2, a.blocks_per_part);
  if (part >= sp.np) {
    // An empty sequence in single-pass mode: partition 0 writes its zero rows.
    if (a.max_np == 1 && sp.np == 0 && part == 0)
      for (int i = tid; i < G * D; i += blockDim.x) store_out(a.out, qrow0 * D + i, 0.f, a.out_dtype);
    return;
  }
  const int bs_log2 = a.block_size_log2;
  const int blk0 = sp.first_blk + part * a.blocks_per_part;
  const int nblk = min(a.blocks_per_part, ((L - 1) >> bs_log2) - blk0 + 1);
  const int tok_begin = max(sp.lo, blk0 << bs_log2);
  const int tok_end = min(L, (blk0 + nblk) << bs_log2);

  const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks_per_seq + blk0;
  for (int i = tid; i < nblk; i += blockDim.x) s_blk[i] = bt[i];

  const T* __restrict__ kc = static_cast<const T*>(a.k_cache);
  const T* __restrict__ vc = static_cast<const T*>(a.v_cache);
  const T* __restrict__ q = static_cast<const T*>(a.q);

  QChunk<T> qc[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    if (h < G)
      qc[h].load(q + (qrow0 + h) * D + c * EPL);
    else
      qc[h].zero();
  }
  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  __syncthreads();

  const int64_t slot_stride = (int64_t)a.num_kv_heads * D;  // elements between consecutive slots
  const T* kbase = kc + (int64_t)g * D + c * EPL;
  const T* vbase = vc + (int64_t)g * D + c * EPL;
  const int bs_mask = (1 << bs_log2) - 1;

  for (int t0 = blk0 << bs_log2; t0 < tok_end; t0 += CH) {
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + (wave * U + u) * RPW + rg;
      ok[u] = t >= tok_begin && t < tok_end;
      const int tt = ok[u] ? t : tok_begin;  // masked rows re-read a valid row
      const int64_t slot = ((int64_t)s_blk[(tt >> bs_log2) - blk0] << bs_log2) + (tt & bs_mask);
      kr[u] = ld16(kbase + slot * slot_stride);
      vr[u] = ld16(vbase + slot * slot_stride);
    }
    float s[U][GT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float d = group_sum<LPR>(qc[h].dot(kr[u]));
        s[u][h] = ok[u] ? d * a.scale_log2e : kNegInf;
      }
    }
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][h]);
      const float mn = fmaxf(m[h], mx);
      const float alpha = rescale(m[h], mn);
      const float msub = mn == kNegInf ? 0.f : mn;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = exp2_fast(s[u][h] - msub);
        l[h] += p;
        axpy_chunk(acc[h], p, vr[u], T());
      }
      m[h] = mn;
    }
  }

  // Merge the row groups of this wave: lanes with equal chunk index c.
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float a1 = rescale(m[h], mn);
      const float a2 = rescale(mo, mn);
      l[h] = l[h] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * a1 + __shfl_xor(acc[h][e], off) * a2;
      m[h] = mn;
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][c * EPL + e] = acc[h][e];
      if (c == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // Merge the waves; one thread per (head, element).
  for (int i = tid; i < G * D; i += blockDim.x) {
    const int h = i / D;
    const int d = i - h * D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = rescale(s_m[w][h], M);
      Ls += s_l[w][h] * f;
      O += s_acc[w][h][d] * f;
    }
    const int64_t row = qrow0 + h;
    if (a.max_np == 1) {
      store_out(a.out, row * D + d, Ls > 0.f ? O / Ls : 0.f, a.out_dtype);
    } else {
      a.ws_o[(row * a.max_np + part) * D + d] = O;
      if (d == 0) {
        a.ws_ml[(row * a.max_np + part) * 2 + 0] = M;
        a.ws_ml[(row * a.max_np + part) * 2 + 1] = Ls;
      }
    }
  }
}

// One wave per (sequence, head): M = max_p m_p, L = sum_p l_p 2^(m_p - M),
// out = (sum_p o_p 2^(m_p - M)) / L; a sequence with no key gets a zero row.
// seq_lens == NULL (prefill rows): every one of the max_np partials was written
// (an empty one as m = -inf, l = 0, o = 0) and all are merged.
__global__ __launch_bounds__(kWave) void decode_combine_kernel(const float* __restrict__ ws_o,
                                                               const float* __restrict__ ws_ml,
                                                               const int32_t* __restrict__ seq_lens,
                                                               int32_t H, int32_t D, int32_t max_np,
                                                               int32_t bs_log2, int32_t bpp,
                                                               int32_t window, void* out,
                                                               int32_t out_dtype) {
  extern __shared__ float s_w[];  // [max_np] weights 2^(m_p - M)
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const KeySpan sp = seq_lens ? decode_span(seq_lens[row / H], window, bs_log2, bpp) : KeySpan{0, 0, 0, max_np};
  const float* ml = ws_ml + row * max_np * 2;
  float M = kNegInf;
  for (int p = lane; p < sp.np; p += kWave) M = fmaxf(M, ml[2 * p]);
  M = group_max<kWave>(M);
  float Ls = 0.f;
  for (int p = lane; p < sp.np; p += kWave) {
    const float f = rescale(ml[2 * p], M);
    s_w[p] = f;
    Ls += ml[2 * p + 1] * f;
  }
  Ls = group_sum<kWave>(Ls);
  __syncthreads();
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  const float* o = ws_o + row * max_np * D;
  for (int d = lane; d < D; d += kWave) {
    float O = 0.f;
    for (int p = 0; p < sp.np; ++p) O += o[(int64_t)p * D + d] * s_w[p];
    store_out(out, row * D + d, O * inv, out_dtype);
  }
}

template <typename T, int D, int GT>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int U = GT <= 2 ? 8 : 4;
  const dim3 grid(a.num_kv_heads * a.batch, a.max_np);
  if (a.valu_waves == kWideWaves) {
    if constexpr (wide_fits((int)sizeof(T), D, GT)) {
      decode_valu_kernel<T, D, GT, U, kWideWaves><<<grid, kWideWaves * kWave, 0, stream>>>(a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  decode_valu_kernel<T, D, GT, U, kWaves><<<grid, kWaves * kWave, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, int gt, hipStream_t stream) {
  switch (gt) {
    case 1: return launch_t<T, D, 1>(a, stream);
    case 2: return launch_t<T, D, 2>(a, stream);
    case 4: return launch_t<T, D, 4>(a, stream);
    case 8: return launch_t<T, D, 8>(a, stream);
    case 16:
      if constexpr (D <= 128) return launch_t<T, D, 16>(a, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

int group_template(int32_t group) {
  int gt = 1;
  while (gt < group) gt <<= 1;
  return gt;
}

}  // namespace

bool decode_valu_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return false;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return false;
  const int gt = group_template(group);
  return gt <= 16 && gt * head_dim <= 2048;
}

bool decode_valu_wide_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  return decode_valu_supported(dtype, head_dim, group) &&
         wide_fits(dtype == PKV_F32 ? 4 : 2, head_dim, group_template(group));
}

hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream) {
  const int gt = group_template(a.num_q_heads / a.num_kv_heads);
  if (a.blocks_per_part > kMaxBpp) return hipErrorInvalidValue;
  if (a.valu_waves != kWaves && !(a.valu_waves == kWideWaves && a.max_np == 1)) return hipErrorInvalidValue;
  if (a.dtype == PKV_BF16) {
    switch (a.head_dim) {
      case 64: return launch_d<uint16_t, 64>(a, gt, stream);
      case 128: return launch_d<uint16_t, 128>(a, gt, stream);
      case 256: return launch_d<uint16_t, 256>(a, gt, stream);
    }
  } else {
    switch (a.head_dim) {
      case 64: return launch_d<float, 64>(a, gt, stream);
      case 128: return launch_d<float, 128>(a, gt, stream);
      case 256: return launch_d<float, 256>(a, gt, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const float* ws_o, const float* ws_ml, const int32_t* seq_lens,
                                 int32_t batch, int32_t num_q_heads, int32_t v_dim, int32_t max_np,
                                 int32_t block_size_log2, int32_t blocks_per_part, int32_t window,
                                 void* out, int32_t out_dtype, hipStream_t stream) {
  const int64_t rows = (int64_t)batch * num_q_heads;
  if (rows == 0) return hipSuccess;
  decode_combine_kernel<<<(unsigned)rows, kWave, sizeof(float) * max_np, stream>>>(
      ws_o, ws_ml, seq_lens, num_q_heads, v_dim, max_np, block_size_log2, blocks_per_part, window,
      out, out_dtype);
  return hipGetLastError();
}

}  // namespace pkv
