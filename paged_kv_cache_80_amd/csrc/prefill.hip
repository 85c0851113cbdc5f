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
// Each wave owns two 16-column tiles and keeps their q in registers.
//
// Data path per 64-key tile.  K and V rows are copied straight from the paged
// cache into LDS with global_load_lds (no register staging), double-buffered so
// the next tile streams in while the current one is computed.  One wave load
// moves 1 KiB = four 256-byte rows; it takes rows r, r+16, r+32, r+48 so that a
// 16-row fragment read walks consecutive 1 KiB groups, padded by 32 bytes: the
// padding at which neither fragment read has a bank conflict (measured:
// SQ_LDS_BANK_CONFLICT is 0 at 32 bytes, nonzero at 0, 16, 48, 64 and 128).  Every fragment address is one lane constant plus an
// immediate offset.  S^T = K.Q^T reads K fragments with ds_read_b128;
// O^T += V^T.P^T reads the transposed V operand straight from the row-major
// tile with ds_read_b64_tr_b16.  Both products run on v_mfma_f32_16x16x32_bf16
// with fp32 accumulation; probabilities enter P.V as a hi + lo bf16 pair so
// rounding P costs no accuracy.  The online softmax works in log2 units
// (scale*log2(e) folded into one FMA before v_exp_f32), reduces a column over
// the four 16-lane rows with permlane swaps, and raises a column's reference
// maximum -- rescaling its accumulators -- only when a logit passes it by more
// than 2^8; tiles wholly inside every column's visible range skip the mask.
#include <type_traits>

#include "mfma_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kColTiles = 2;                     // 16-column tiles per wave
constexpr int kCols = kWaves * kColTiles * 16;   // columns per workgroup
constexpr int kKeyTile = 64;                     // keys per LDS tile
constexpr int kMaxTableLds = kPrefillMaxTableBlocks;  // block-table entries staged in LDS
static_assert(kCols == kPrefillColumns && kKeyTile == kPrefillKeyTile, "host sizing");
constexpr float kRescaleLog2 = 8.f;              // lazy-rescale threshold (log2 units)
constexpr float kRaiseSum = 256.f;               // 2^kRescaleLog2: a lane sum at most this has no p above it

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;       // rows one wave load moves
  static constexpr int kGroups = kKeyTile / kRowsPerLoad;     // wave loads per tile and tensor
  static constexpr int kGroupBytes = 1024 + 32;               // one load's rows plus padding
  static constexpr int kBytes = kGroups * kGroupBytes;        // one tensor, one buffer
  // Byte offset of (row, byte) inside a tile: load g holds rows g, g+kGroups, ...
  static constexpr int off(int row, int byte) {
    return (row % kGroups) * kGroupBytes + (row / kGroups) * kRowBytes + byte;
  }
};

// FEW, the narrow variant (split calls, and calls whose columns fit in one
// full-width workgroup, as a few query rows per sequence do): one 16-column tile
// per wave instead of two, so a call's columns spread over twice as many waves,
// and waves without a column skip the arithmetic.  SPLIT: the keys are cut into
// partitions (blockIdx.y) that leave partials for the combine.  Both are
// template flags so that the full-width, unsplit kernel keeps their branches out
// of its schedule.
template <int D, bool FEW, bool SPLIT>
__global__ __launch_bounds__(kWaves * kWave, 2) void prefill_mfma_kernel(PrefillArgs a) {
  using T = Tile<D>;
  constexpr int CT = FEW ? 1 : kColTiles;  // 16-column tiles per wave
  constexpr int COLS = kWaves * CT * 16;  // columns per workgroup
  constexpr int KS = D / 32;                       // 32-wide contraction steps of Q.K
  constexpr int DT = D / 16;                       // 16-row tiles of O^T
  constexpr int NU = kKeyTile / 16;
  constexpr int LPW = T::kGroups / kWaves;         // wave loads per wave and tensor
  // Fragment addresses split into a lane constant plus an immediate when 16-row
  // steps map whole groups onto whole groups.
  static_assert(T::kGroups % kWaves == 0 && (16 % T::kGroups == 0 || T::kGroups % 16 == 0), "tile layout");
  __shared__ __attribute__((aligned(16))) unsigned char k_lds[2 * T::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[2 * T::kBytes];
  __shared__ int32_t s_bt[kMaxTableLds];

  // Workgroups are dealt to the 8 XCDs round-robin by launch order; renumber them
  // so the query tiles of one (sequence, KV head) -- which read the same K/V
  // tiles -- run on one XCD and share its L2.
  const int nwg = gridDim.x;                // a multiple of 8
  const int w = blockIdx.x;
  const int logical = (w & 7) * (nwg >> 3) + (w >> 3);
  const int qt = logical % a.q_tiles;
  const int gb = logical / a.q_tiles;
  if (gb >= a.num_kv_heads * a.batch) return;  // padding workgroup
  const int g = gb % a.num_kv_heads;
  const int b = gb / a.num_kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const int H = a.num_q_heads;
  const int G = H / a.num_kv_heads;
  const int q0 = a.cu_seqlens_q[b];
  const int n = a.cu_seqlens_q[b + 1] - q0;
  const int L = a.seq_lens_kv[b];
  const int ncols = n * G;
  const int col0 = qt * COLS;
  if (col0 >= ncols) return;

  // This lane's columns and their q fragments.
  bool cvalid[CT];
  int cpos[CT];
  int64_t crow[CT];
  uint4 qf[CT][KS];
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int gc = col0 + (wave * CT + ct) * 16 + l16;
    cvalid[ct] = gc < ncols;
    const int i = cvalid[ct] ? gc / G : 0;
    const int hl = cvalid[ct] ? gc - i * G : 0;
    cpos[ct] = L - n + i;
    crow[ct] = (int64_t)(q0 + i) * H + (int64_t)g * G + hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ct][ks] = cvalid[ct] ? ld16(q + crow[ct] * D + 32 * ks + 8 * lg) : make_uint4(0, 0, 0, 0);
  }

  retire_loads();  // q fragments are in registers before any tile is in flight
  // Keys any column of this workgroup can see.
  const int last_col = min(ncols - 1, col0 + COLS - 1);
  const int p_lo = L - n + col0 / G;
  const int p_hi = L - n + last_col / G;
  const int key_lo = a.window > 0 ? max(0, p_lo - a.window + 1) : 0;
  const int key_hi = p_hi + 1;
  if constexpr (!SPLIT) {
    if (key_hi <= key_lo) return;  // malformed lengths (n > L): nothing visible
  }
  int t_begin = key_lo / kKeyTile;
  int t_end = (key_hi + kKeyTile - 1) / kKeyTile;
  if constexpr (SPLIT) {
    // This workgroup's key partition; with nothing visible in it (or malformed
    // lengths) the workgroup leaves empty partials (m = -inf, l = 0, o = 0).
    const int p0 = (int)blockIdx.y * a.part_tiles;
    if (key_hi <= key_lo) t_end = t_begin;
    t_begin = max(t_begin, p0);
    t_end = max(t_begin, min(t_end, p0 + a.part_tiles));
    if (t_begin >= t_end) {
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if (!cvalid[ct]) continue;
        const int64_t pr = crow[ct] * a.max_np + blockIdx.y;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) store4(a.ws_o, pr * D + 16 * dt + 4 * lg, z, PKV_F32);
        if (lg == 0) {
          a.ws_ml[2 * pr] = kNegInf;
          a.ws_ml[2 * pr + 1] = 0.f;
        }
      }
      return;
    }
  }

  const int bs_log2 = a.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks_per_seq;
  const int blk_lo = key_lo >> bs_log2;
  const int nblk = ((key_hi - 1) >> bs_log2) - blk_lo + 1;
  // nblk <= max_blocks_per_seq <= kMaxTableLds (checked by the host).
  for (int i = tid; i < nblk; i += kWaves * kWave) s_bt[i] = bt[blk_lo + i];
  __syncthreads();

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache) + (int64_t)g * D;
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache) + (int64_t)g * D;
  const int64_t slot_stride = (int64_t)a.num_kv_heads * D;
  // Lane constants of the loads and of the two fragment reads.
  const int ld_row = lane / (D / 8);       // row within one wave load
  const int ld_chunk = lane % (D / 8);     // 16-byte chunk of that row
  const int64_t ld_lane_off = (int64_t)T::kGroups * ld_row * slot_stride + 8 * ld_chunk;
  const uint32_t ld_lane_bytes = (uint32_t)(2 * ld_lane_off);  // < 2^32: rows of at most 64 KiB (checked by the host)
  const int qk_lane = T::off(l16, 16 * lg);
  const int tr_row = 4 * lg + (l16 >> 2);  // tile row of this lane's transposed read
  const int tr_lane = T::off(tr_row, 8 * (l16 & 3));

  // Copy one 64-key tile of K and V into buffer BUF.  Keys outside
  // [key_lo, key_hi) re-read a visible row: they are masked, and a finite row
  // keeps 0 * v = 0 (padding table entries may point at a NaN-filled block).
  auto issue_tile = [&](auto bufc, int tile) {
    constexpr int BUF = decltype(bufc)::value;
    const int j0 = tile * kKeyTile;
    if (j0 >= key_lo && j0 + kKeyTile <= key_hi && bs_log2 >= 6) {
      // The tile lies in one block and every row is visible: one block lookup,
      // a wave-uniform base in SGPRs, lane offsets fixed for the whole kernel.
      const int phys = __builtin_amdgcn_readfirstlane(s_bt[(j0 >> bs_log2) - blk_lo]);
      const int64_t row0 = ((int64_t)phys << bs_log2) + (j0 & bs_mask);
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int grp = wave * LPW + i;
        const int64_t base = (row0 + grp) * slot_stride;
        load_lds16_s(kc + base, ld_lane_bytes, k_lds + BUF * T::kBytes + grp * T::kGroupBytes);
        load_lds16_s(vc + base, ld_lane_bytes, v_lds + BUF * T::kBytes + grp * T::kGroupBytes);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int grp = wave * LPW + i;
      const int j = min(max(j0 + grp + T::kGroups * ld_row, key_lo), key_hi - 1);
      const int lb = j >> bs_log2;
      const int phys = s_bt[lb - blk_lo];
      const int64_t off = (((int64_t)phys << bs_log2) + (j & bs_mask)) * slot_stride + 8 * ld_chunk;
      load_lds16(kc + off, k_lds + BUF * T::kBytes + grp * T::kGroupBytes);
      load_lds16(vc + off, v_lds + BUF * T::kBytes + grp * T::kGroupBytes);
    }
  };

  f32x4_t o[CT][DT];
  float mref[CT], l[CT];  // mref: reference maximum in log2 units
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    mref[ct] = kNegInf;
    l[ct] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[ct][dt] = f32x4_zero();
  }
  const float c2 = a.scale_log2e;

  // One V^T fragment (16 dimensions x 32 keys) for O^T += V^T . P^T.
  auto read_v = [&](const unsigned char* vb, int kk, int dt) {
    const uint2 x0 = lds_tr16(reinterpret_cast<const uint16_t*>(vb + T::off(32 * kk, 32 * dt)));
    const uint2 x1 = lds_tr16(reinterpret_cast<const uint16_t*>(vb + T::off(32 * kk + 16, 32 * dt)));
    return make_uint4(x0.x, x0.y, x1.x, x1.y);
  };

  // Every LDS fragment is read one step ahead of the MFMAs that use it (K rows
  // u+1 while rows u multiply, the first V fragments during the softmax, V keys
  // kk+1 while keys kk multiply); the scheduling barriers keep the compiler from
  // sinking the reads back next to their use, where each would stall for the
  // full LDS latency.
  auto compute_tile = [&](auto bufc, int tile) {
    constexpr int BUF = decltype(bufc)::value;
    const unsigned char* kb = k_lds + BUF * T::kBytes + qk_lane;
    const unsigned char* vb = v_lds + BUF * T::kBytes + tr_lane;
    const int j0 = tile * kKeyTile;

    // S^T = K . Q^T
    f32x4_t s[CT][NU];
    uint4 kf[2][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[0][ks] = *reinterpret_cast<const uint4*>(kb + T::off(0, 64 * ks));
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (u + 1 < NU) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kf[(u + 1) & 1][ks] = *reinterpret_cast<const uint4*>(kb + T::off(16 * (u + 1), 64 * ks));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          s[ct][u] = mfma_bf16(kf[u & 1][ks], qf[ct][ks], ks == 0 ? f32x4_zero() : s[ct][u]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    uint4 vf[2][DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[0][dt] = read_v(vb, 0, dt);
    __builtin_amdgcn_sched_barrier(0);

    // Online softmax per column.  The reference maximum is raised only when a
    // logit exceeds it by more than 2^8 in probability; in between,
    // probabilities up to 256 accumulate against the stale reference, which is
    // exact (O and l share it) and skips the O rescale on almost every tile.
    const bool full = j0 >= key_lo && j0 + kKeyTile - 1 <= p_lo && (a.window == 0 || j0 > p_hi - a.window);
    uint4 phi[CT][kKeyTile / 32], plo[CT][kKeyTile / 32];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if (!full) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = j0 + 16 * u + 4 * lg + r;
            const bool vis = j <= cpos[ct] && (a.window == 0 || j > cpos[ct] - a.window);
            s[ct][u][r] = vis ? s[ct][u][r] : kNegInf;
          }
        }
      }
      // Probabilities against the current reference, and this lane's sum of them.
      // No lane's sum above 2^8 means no probability above 2^8, i.e. no logit past
      // the reference by more than the rescale threshold: the raise test needs the
      // column maximum (a max chain and a cross-row exchange) only when some lane's
      // sum says it might -- the first visible tile, a new peak -- and then the
      // probabilities are taken again against the raised reference.  The decision
      // is the one the maximum alone would take.
      auto probs = [&](float mb, float& ls) {
        ls = 0.f;
#pragma unroll
        for (int kk = 0; kk < kKeyTile / 32; ++kk) {
          float p8[8];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float p = exp2_fast(fmaf(s[ct][2 * kk + h][r], c2, -mb));
              p8[4 * h + r] = p;
              ls += p;
            }
          pack_p_split(p8, phi[ct][kk], plo[ct][kk]);
        }
      };
      float ls;
      probs(mref[ct] == kNegInf ? 0.f : mref[ct], ls);
      if (__any(mref[ct] == kNegInf || !(ls <= kRaiseSum))) {  // !(<=): a NaN or inf sum too
        // A running chain of pairs, so that each step is one v_max3_f32.
        float mt = s[ct][0][0];
#pragma unroll
        for (int e = 1; e + 1 < 4 * NU; e += 2)
          mt = fmaxf(fmaxf(mt, s[ct][e / 4][e % 4]), s[ct][(e + 1) / 4][(e + 1) % 4]);
        mt = fmaxf(mt, s[ct][NU - 1][3]);
        const float mts = row4_max(mt) * c2;
        const bool raise = mts > mref[ct] + kRescaleLog2;
        if (__any(raise)) {
          const float alpha = raise ? exp2_fast(mref[ct] - mts) : 1.f;  // mref = -inf gives 0
          if (raise) mref[ct] = mts;
          l[ct] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[ct][dt] *= alpha;
        }
        probs(mref[ct] == kNegInf ? 0.f : mref[ct], ls);  // no visible key yet: every p is 0
      }
      l[ct] += ls;
    }
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T . P^T, 32 keys per step, P as hi + lo bf16.
#pragma unroll
    for (int kk = 0; kk < kKeyTile / 32; ++kk) {
      if (kk + 1 < kKeyTile / 32) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vf[(kk + 1) & 1][dt] = read_v(vb, kk + 1, dt);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          o[ct][dt] = mfma_bf16(vf[kk & 1][dt], phi[ct][kk], o[ct][dt]);
          o[ct][dt] = mfma_bf16(vf[kk & 1][dt], plo[ct][kk], o[ct][dt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // A wave whose columns all lie past the last one copies its share of every
  // tile but skips the arithmetic.
  const bool wave_cols = col0 + wave * CT * 16 < ncols;
  issue_tile(B0{}, t_begin);  // t_begin < t_end here
  for (int tile = t_begin; tile < t_end; tile += 2) {
    wait_vmem();
    __syncthreads();  // buffer 0 holds `tile`; nobody reads buffer 1 any more
    if (tile + 1 < t_end) issue_tile(B1{}, tile + 1);
    if constexpr (FEW) {
      if (wave_cols) compute_tile(B0{}, tile);
    } else {
      compute_tile(B0{}, tile);
    }
    if (tile + 1 < t_end) {
      wait_vmem();
      __syncthreads();  // buffer 1 holds tile+1; nobody reads buffer 0 any more
      if (tile + 2 < t_end) issue_tile(B0{}, tile + 2);
      if constexpr (FEW) {
        if (wave_cols) compute_tile(B1{}, tile + 1);
      } else {
        compute_tile(B1{}, tile + 1);
      }
    }
  }

  if (SPLIT) {
    // Partials of this key partition: unnormalised o, the reference maximum
    // (log2 units) and the sum; a column that saw no key here leaves (-inf, 0, 0).
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const float ls = row4_sum(l[ct]);
      if (!cvalid[ct]) continue;
      const int64_t pr = crow[ct] * a.max_np + blockIdx.y;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float v[4] = {o[ct][dt][0], o[ct][dt][1], o[ct][dt][2], o[ct][dt][3]};
        store4(a.ws_o, pr * D + 16 * dt + 4 * lg, v, PKV_F32);
      }
      if (lg == 0) {
        a.ws_ml[2 * pr] = mref[ct];
        a.ws_ml[2 * pr + 1] = ls;
      }
    }
    return;
  }
  // Normalise and store: lane holds column l16, dimensions 16*dt + 4*lg + r.
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const float ls = row4_sum(l[ct]);
    if (!cvalid[ct]) continue;
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float v[4] = {o[ct][dt][0] * inv, o[ct][dt][1] * inv, o[ct][dt][2] * inv, o[ct][dt][3] * inv};
      store4(a.out, crow[ct] * D + 16 * dt + 4 * lg, v, a.out_dtype);
    }
  }
}

template <int D>
void launch_variant(const PrefillArgs& a, dim3 grid, bool narrow, bool split, hipStream_t stream) {
  // A split call always takes the narrow variant (the wide split one does not fit
  // its registers); the grid's column tiles were sized for it.
  const dim3 blk(kWaves * kWave);
  if (split) prefill_mfma_kernel<D, true, true><<<grid, blk, 0, stream>>>(a);
  else if (narrow) prefill_mfma_kernel<D, true, false><<<grid, blk, 0, stream>>>(a);
  else prefill_mfma_kernel<D, false, false><<<grid, blk, 0, stream>>>(a);
}

}  // namespace

bool prefill_mfma_supported(int32_t dtype, int32_t head_dim) {
  return dtype == PKV_BF16 && (head_dim == 64 || head_dim == 128);
}

hipError_t launch_prefill_mfma(const PrefillArgs& a_in, hipStream_t stream) {
  PrefillArgs a = a_in;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t cols = (int64_t)a.max_q_len * G;
  // Split calls, and calls whose columns fit in one full-width workgroup, take the
  // narrow variant (FEW: one 16-column tile per wave, waves without a column skip
  // the arithmetic); its workgroups hold half as many columns.
  const bool split = a.max_np > 1;
  const bool narrow = split || cols < kCols;
  const int64_t width = narrow ? kCols / 2 : kCols;
  const int64_t tiles = (cols + width - 1) / width;
  if (tiles == 0 || a.batch == 0) return hipSuccess;
  const int64_t total = tiles * a.num_kv_heads * a.batch;
  const int64_t padded = (total + 7) / 8 * 8;
  if (padded > 0x7fffffff || a.max_np < 1 || a.max_np > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)padded, (unsigned)a.max_np);
  a.q_tiles = (int32_t)tiles;
  switch (a.head_dim) {
    case 64: launch_variant<64>(a, grid, narrow, split, stream); break;
    case 128: launch_variant<128>(a, grid, narrow, split, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
