// decode_mfma.hip -- paged GQA decode with the head group on the matrix cores.
//
// Same result as decode.hip (softmax(q.K^T * scale) V over the keys the newest
// position sees, query head h reading KV head h / G), for head groups large
// enough that the group is a dense contraction: G query heads x 32 keys x 128
// per tile.  On the vector ALUs every V element costs G FMAs (8 for the
// llama2-70B shape), which makes the VALU kernel issue-bound long before HBM
// is; here S^T = K.Q^T and O^T += V^T.P^T run on v_mfma_f32_16x16x32_bf16 with
// the G heads as MFMA columns (padded to 16), and the vector ALUs only run the
// online softmax.
//
// Work split and data path.  One wave per (sequence, KV head, partition of
// table blocks) -- the partitions are the split-K partitions of decode.hip and
// share its combine.  Per 32-key tile the wave loads K straight into MFMA
// A-operand registers (lane = key row, 8 dims at 32ks + 8lg) and V into
// registers in row order, and keeps the next tile in flight while it computes
// the current one (8 waves per CU, 16 KiB each).  V goes through one private
// LDS tile so the transposed operand of O^T += V^T.P^T can be read with
// ds_read_b64_tr_b16; its 16-byte chunks are XOR-swizzled by row & 1 so those
// reads have at most two-way bank conflicts.  All loads are ordinary
// compiler-tracked loads (an LDS-DMA stream was tried: at most ~96 KiB in
// flight per CU fits the LDS, against 128 KiB here).  Probabilities enter P.V
// as a hi + lo bf16 pair.
#include "mfma_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kD = 128;
constexpr int kKeyTile = 32;
constexpr int kRowBytes = kD * 2;                  // 256
constexpr int kTileBytes = kKeyTile * kRowBytes;   // 8 KiB per tensor per tile
constexpr int kMaxBpp = 256;                       // table blocks per partition held in LDS

__global__ __launch_bounds__(kWave, 8) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int KS = kD / 32;
  constexpr int DT = kD / 16;
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[kTileBytes];
  __shared__ int32_t s_blk[kMaxBpp];

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int H = a.num_q_heads;
  const int G = H / a.num_kv_heads;
  const bool cvalid = l16 < G;
  const int64_t qrow = (int64_t)b * H + (int64_t)g * G + (cvalid ? l16 : 0);

  const int32_t L = a.seq_lens[b];
  const KeySpan sp = decode_span(L, a.window, a.block_size_log2, a.blocks_per_part);
  if (part >= sp.np) {
    if (a.max_np == 1 && sp.np == 0 && part == 0 && cvalid) {
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
      for (int dt = 0; dt < DT; ++dt) store4(a.out, qrow * kD + 16 * dt + 4 * lg, z, a.out_dtype);
    }
    return;
  }
  const int bs_log2 = a.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int blk0 = sp.first_blk + part * a.blocks_per_part;
  const int nblk = min(a.blocks_per_part, ((L - 1) >> bs_log2) - blk0 + 1);
  const int tok_begin = max(sp.lo, blk0 << bs_log2);
  const int tok_end = min(L, (blk0 + nblk) << bs_log2);
  const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks_per_seq + blk0;
  for (int i = lane; i < nblk; i += kWave) s_blk[i] = bt[i];

  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  uint4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = cvalid ? ld16(q + qrow * kD + 32 * ks + 8 * lg) : make_uint4(0, 0, 0, 0);
  __syncthreads();

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache) + (int64_t)g * kD;
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache) + (int64_t)g * kD;
  const int64_t slot_stride = (int64_t)a.num_kv_heads * kD;

  auto slot_of = [&](int j) -> int64_t {
    j = min(max(j, tok_begin), tok_end - 1);
    return ((int64_t)s_blk[(j >> bs_log2) - blk0] << bs_log2) + (j & bs_mask);
  };
  // V rows of a tile: lane takes chunk (lane & 15) of rows (lane >> 4) + 4i.
  uint4 kr[2 * KS], vr[8];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) vr[i] = ld16(vc + slot_of(t0 + 4 * i + lg) * slot_stride + 8 * l16);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t base = slot_of(t0 + 16 * u + l16) * slot_stride;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kr[u * KS + ks] = ld16(kc + base + 32 * ks + 8 * lg);
    }
  };

  const int kq = l16 >> 2, q4 = l16 & 3;
  const int ra = 4 * lg + kq;
  const int v_off = ra * kRowBytes + 16 * ((q4 >> 1) ^ (ra & 1)) + 8 * (q4 & 1);

  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_zero();
  float m = kNegInf, l = 0.f;
  const float c2 = a.scale_log2e;
  const int t_first = tok_begin & ~(kKeyTile - 1);

  load_tile(t_first);
  for (int t0 = t_first; t0 < tok_end; t0 += kKeyTile) {
    // Stage this tile's V rows (chunk swizzled by row & 1) and keep its K.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + lg;
      *reinterpret_cast<uint4*>(v_lds + r * kRowBytes + 16 * (l16 ^ (r & 1))) = vr[i];
    }
    uint4 kcur[2 * KS];
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) kcur[i] = kr[i];
    if (t0 + kKeyTile < tok_end) load_tile(t0 + kKeyTile);

    f32x4_t s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[u] = mfma_bf16(kcur[u * KS + ks], qf[ks], ks == 0 ? f32x4_zero() : s[u]);
    }
    if (!(t0 >= tok_begin && t0 + kKeyTile <= tok_end)) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = t0 + 16 * u + 4 * lg + r;
          s[u][r] = (j >= tok_begin && j < tok_end) ? s[u][r] : kNegInf;
        }
    }
    float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    const float msc = mn == kNegInf ? 0.f : mn * c2;
    const float alpha = m == mn ? 1.f : exp2_fast(m * c2 - msc);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    float p8[8];
    float ls = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2_fast(fmaf(s[u][r], c2, -msc));
        p8[4 * u + r] = p;
        ls += p;
      }
    l = l * alpha + ls;
    m = mn;
    uint4 phi, plo;
    pack_p_split(p8, phi, plo);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint2 x0 = lds_tr16(reinterpret_cast<const uint16_t*>(v_lds + v_off + 32 * dt));
      const uint2 x1 = lds_tr16(reinterpret_cast<const uint16_t*>(v_lds + v_off + 16 * kRowBytes + 32 * dt));
      const uint4 af = make_uint4(x0.x, x0.y, x1.x, x1.y);
      o[dt] = mfma_bf16(af, phi, o[dt]);
      o[dt] = mfma_bf16(af, plo, o[dt]);
    }
  }

  float lsum = l;
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (!cvalid) return;
  if (a.max_np == 1) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float v[4] = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
      store4(a.out, qrow * kD + 16 * dt + 4 * lg, v, a.out_dtype);
    }
  } else {
    float* wo = a.ws_o + (qrow * a.max_np + part) * kD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float v[4] = {o[dt][0], o[dt][1], o[dt][2], o[dt][3]};
      store4(wo, 16 * dt + 4 * lg, v, PKV_F32);
    }
    if (lg == 0) {
      a.ws_ml[(qrow * a.max_np + part) * 2 + 0] = m * c2;
      a.ws_ml[(qrow * a.max_np + part) * 2 + 1] = lsum;
    }
  }
}

}  // namespace

bool decode_mfma_supported(int32_t dtype, int32_t head_dim, int32_t group, int32_t blocks_per_part) {
  return dtype == PKV_BF16 && head_dim == kD && group >= 1 && group <= 16 && blocks_per_part <= kMaxBpp;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  if (a.blocks_per_part > kMaxBpp) return hipErrorInvalidValue;
  const dim3 grid(a.max_np, a.num_kv_heads, a.batch);
  decode_mfma_kernel<<<grid, kWave, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
