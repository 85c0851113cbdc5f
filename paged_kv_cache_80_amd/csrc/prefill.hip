// prefill.hip -- chunked causal prefill over a paged KV cache on bf16 MFMA.
//
// New row i of sequence b (n_b rows, L_b keys including them) sits at
// position p = L_b - n_b + i and attends to keys j <= p (and j > p - W with a
// window): the bottom-right alignment of the "KV Cache notes" minimal
// implementation and sparse_mode 3 of the skill page's appendix C.  The new
// rows must already be in the cache (the write precedes attention on every
// layer, skill page section 3.6).
//
// Work split.  One workgroup (4 waves) owns 128 "columns" of one (sequence,
// KV head): a column is one (query row, query head) pair, ordered position-major
// so the G heads sharing the KV head sit side by side and share each K/V tile.
// Each wave owns two 16-column tiles.  The workgroup walks 64-key tiles: K is
// staged row-major in LDS, V transposed (keys contiguous per dimension) so both
// products read 16- or 8-byte LDS fragments.  S^T = K.Q^T and O^T += V^T.P^T run
// on v_mfma_f32_16x16x32_bf16 with fp32 accumulation; probabilities enter P.V as
// a hi + lo bf16 pair (split_bf16) so rounding P costs no accuracy.  The online
// softmax (running max in log2 units, v_exp_f32) is per column, which is fixed
// per lane; the max over a tile's keys needs only two cross-lane steps.
#include "mfma_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kColTiles = 2;                     // 16-column tiles per wave
constexpr int kCols = kWaves * kColTiles * 16;   // columns per workgroup
constexpr int kKeyTile = 64;                     // keys per LDS tile
constexpr int kKPad = 8;                         // bf16 padding per K row
constexpr int kVPad = 4;                         // bf16 padding per V^T row

template <int D>
__global__ __launch_bounds__(kWaves * kWave) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int KS = D / 32;  // 32-wide contraction steps of Q.K
  constexpr int DT = D / 16;  // 16-row tiles of O^T
  constexpr int NU = kKeyTile / 16;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kKeyTile][D + kKPad];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D][kKeyTile + kVPad];

  const int qt = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const int H = a.num_q_heads;
  const int G = H / a.num_kv_heads;
  const int q0 = a.cu_seqlens_q[b];
  const int n = a.cu_seqlens_q[b + 1] - q0;
  const int L = a.seq_lens_kv[b];
  const int ncols = n * G;
  const int col0 = qt * kCols;
  if (col0 >= ncols) return;

  // This lane's columns.
  bool cvalid[kColTiles];
  int cpos[kColTiles];
  int64_t crow[kColTiles];
  uint4 qf[kColTiles][KS];
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    const int gc = col0 + (wave * kColTiles + ct) * 16 + l16;
    cvalid[ct] = gc < ncols;
    const int i = cvalid[ct] ? gc / G : 0;
    const int hl = gc - (gc / G) * G;
    cpos[ct] = L - n + i;
    crow[ct] = (int64_t)(q0 + i) * H + (int64_t)g * G + (cvalid[ct] ? hl : 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ct][ks] = cvalid[ct] ? ld16(q + crow[ct] * D + 32 * ks + 8 * lg) : make_uint4(0, 0, 0, 0);
  }

  // Keys any column of this workgroup can see.
  const int last_col = min(ncols - 1, col0 + kCols - 1);
  const int p_lo = L - n + col0 / G;
  const int p_hi = L - n + last_col / G;
  const int key_lo = a.window > 0 ? max(0, p_lo - a.window + 1) : 0;
  const int key_hi = p_hi + 1;
  const int t_begin = key_lo / kKeyTile;
  const int t_end = (key_hi + kKeyTile - 1) / kKeyTile;

  f32x4_t o[kColTiles][DT];
  float m[kColTiles], l[kColTiles];
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    m[ct] = kNegInf;
    l[ct] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[ct][dt] = f32x4_zero();
  }

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks_per_seq;
  const int bs_log2 = a.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int64_t slot_stride = (int64_t)a.num_kv_heads * D;
  const int64_t head_off = (int64_t)g * D;

  for (int tile = t_begin; tile < t_end; ++tile) {
    const int j0 = tile * kKeyTile;
    __syncthreads();  // the previous tile is no longer read
    // K tile, row-major: 16 lanes per key row (coalesced 16-byte chunks).
    for (int idx = tid; idx < kKeyTile * (D / 8); idx += kWaves * kWave) {
      const int r = idx / (D / 8);
      const int c = idx - r * (D / 8);
      const int j = j0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j >= key_lo && j < key_hi) {
        const int64_t slot = ((int64_t)bt[j >> bs_log2] << bs_log2) + (j & bs_mask);
        v = ld16(kc + slot * slot_stride + head_off + 8 * c);
      }
      *reinterpret_cast<uint4*>(&k_lds[r][8 * c]) = v;
    }
    // V tile, transposed: a lane takes two keys' chunk and writes 8 key pairs.
    for (int idx = tid; idx < (kKeyTile / 2) * (D / 8); idx += kWaves * kWave) {
      const int pr = idx % (kKeyTile / 2);
      const int c = idx / (kKeyTile / 2);
      const int j = j0 + 2 * pr;
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
      if (j >= key_lo && j < key_hi) {
        const int64_t slot = ((int64_t)bt[j >> bs_log2] << bs_log2) + (j & bs_mask);
        v0 = ld16(vc + slot * slot_stride + head_off + 8 * c);
      }
      if (j + 1 >= key_lo && j + 1 < key_hi) {
        const int64_t slot = ((int64_t)bt[(j + 1) >> bs_log2] << bs_log2) + ((j + 1) & bs_mask);
        v1 = ld16(vc + slot * slot_stride + head_off + 8 * c);
      }
      uint32_t w[8];
      interleave_pairs(v0, v1, w);
#pragma unroll
      for (int e = 0; e < 8; ++e) *reinterpret_cast<uint32_t*>(&vt_lds[8 * c + e][2 * pr]) = w[e];
    }
    __syncthreads();

    // S^T = K . Q^T
    f32x4_t s[kColTiles][NU];
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct)
#pragma unroll
      for (int u = 0; u < NU; ++u) s[ct][u] = f32x4_zero();
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 af = lds16(&k_lds[16 * u + l16][32 * ks + 8 * lg]);
#pragma unroll
        for (int ct = 0; ct < kColTiles; ++ct) s[ct][u] = mfma_bf16(af, qf[ct][ks], s[ct][u]);
      }
    }

    // Online softmax per column.
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) {
      float mt = kNegInf;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + 16 * u + 4 * lg + r;
          const bool vis = cvalid[ct] && j <= cpos[ct] && (a.window == 0 || j > cpos[ct] - a.window);
          const float x = vis ? s[ct][u][r] * a.scale_log2e : kNegInf;
          s[ct][u][r] = x;
          mt = fmaxf(mt, x);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m[ct], mt);
      const float alpha = rescale(m[ct], mn);
      const float msub = mn == kNegInf ? 0.f : mn;
      float ls = 0.f;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = exp2_fast(s[ct][u][r] - msub);
          s[ct][u][r] = p;
          ls += p;
        }
      }
      l[ct] = l[ct] * alpha + ls;
      m[ct] = mn;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[ct][dt] *= alpha;
    }

    // O^T += V^T . P^T, 32 keys per step, P as hi + lo bf16.
#pragma unroll
    for (int kk = 0; kk < kKeyTile / 32; ++kk) {
      uint4 phi[kColTiles], plo[kColTiles];
#pragma unroll
      for (int ct = 0; ct < kColTiles; ++ct) {
        float p8[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p8[r] = s[ct][2 * kk][r];
          p8[4 + r] = s[ct][2 * kk + 1][r];
        }
        pack_p(p8, phi[ct], plo[ct]);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 x0 = lds8(&vt_lds[16 * dt + l16][32 * kk + 4 * lg]);
        const uint2 x1 = lds8(&vt_lds[16 * dt + l16][32 * kk + 16 + 4 * lg]);
        const uint4 af = make_uint4(x0.x, x0.y, x1.x, x1.y);
#pragma unroll
        for (int ct = 0; ct < kColTiles; ++ct) {
          o[ct][dt] = mfma_bf16(af, phi[ct], o[ct][dt]);
          o[ct][dt] = mfma_bf16(af, plo[ct], o[ct][dt]);
        }
      }
    }
  }

  // Normalise and store: lane holds column l16, dimensions 16*dt + 4*lg + r.
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    float ls = l[ct];
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if (!cvalid[ct]) continue;
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float v[4] = {o[ct][dt][0] * inv, o[ct][dt][1] * inv, o[ct][dt][2] * inv, o[ct][dt][3] * inv};
      store4(a.out, crow[ct] * D + 16 * dt + 4 * lg, v, a.out_dtype);
    }
  }
}

}  // namespace

bool prefill_mfma_supported(int32_t dtype, int32_t head_dim) {
  return dtype == PKV_BF16 && (head_dim == 64 || head_dim == 128);
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t cols = (int64_t)a.max_q_len * G;
  const int64_t tiles = (cols + kCols - 1) / kCols;
  if (tiles == 0 || a.batch == 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles, a.num_kv_heads, a.batch);
  switch (a.head_dim) {
    case 64: prefill_mfma_kernel<64><<<grid, kWaves * kWave, 0, stream>>>(a); break;
    case 128: prefill_mfma_kernel<128><<<grid, kWaves * kWave, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
