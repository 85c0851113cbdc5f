// mla.hip -- MLA absorbed-form decode over a paged latent cache on bf16 MFMA.
//
// The cache holds, per token, the compressed latent c (kv_lora_rank = 512) and
// a separate rotary part c_r (64).  With the projections absorbed, every query
// head h scores a key as q_nope[h].c + q_rope[h].c_r and the value is c itself
// ("KVCache optimisation skill", mode 3: key = value = cache_nope, rope passed
// separately; "KV Cache notes", MLA section: one latent shared by all heads).
// So all H query heads read the same 1152-byte row per token: Q-tile x key-tile
// is a dense contraction (H x 576 by 576 x keys, then H x keys by keys x 512).
//
// Work split.  One workgroup per (sequence, key partition, group of up to 128
// heads); each wave owns 16 heads and keeps their q (576 bf16) in registers and
// their O^T (512 x 16 fp32) in accumulators.  32-key tiles of the latent are
// copied straight into LDS with global_load_lds through a ring of slots, one row per
// wave instruction (rows padded so fragment reads spread over the banks); the
// rope rows sit in a second, chunk-swizzled tile.  The same row-major latent
// tile feeds S^T = C.Q^T (ds_read_b128) and, through ds_read_b64_tr_b16, the
// transposed operand of O^T += C^T.P^T -- no second copy.  Partials (m, l, o)
// of each partition go to the workspace and the split-K combine of decode.hip
// merges them, exactly as for standard decode.
#include <algorithm>

#include "mfma_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kD = 512;        // latent width (value width)
constexpr int kR = 64;         // rope width
constexpr int kKeyTile = 32;
constexpr int kRowPad = 16;    // bf16 padding per latent row in LDS (32 bytes)
constexpr int kRow = kD + kRowPad;
constexpr int kMaxBpp = 1024;  // table blocks per partition held in LDS
// Fragment reads issued ahead of their MFMAs (Q.K steps, P.V row tiles): two
// each is what the 8-wave kernel's registers hold next to q and O.
constexpr int kQkAhead = 2;
constexpr int kPvAhead = 2;
// A column's reference maximum (log2 units) is raised only when a score exceeds
// it by more than this; in between, probabilities up to 2^8 accumulate against
// the stale reference, which is exact (o and l share it) and skips the O
// rescale on almost every tile.
constexpr float kRescaleLog2 = 8.f;
constexpr float kRaiseSum = 256.f;  // 2^kRescaleLog2: a lane sum at most this has no p above it

__device__ __forceinline__ int rope_swz(int r) { return r & 7; }

// Wait for the oldest of this wave's in-flight tiles, `ahead` newer tiles
// (each NL loads) staying in flight.
template <int NL, int MAXA>
__device__ __forceinline__ void wait_tile(int ahead) {
  if constexpr (MAXA >= 2) {
    if (ahead >= 2) { wait_vm<2 * NL>(); return; }
  }
  if constexpr (MAXA >= 1) {
    if (ahead == 1) { wait_vm<NL>(); return; }
  }
  wait_vm<0>();
}

// NW waves of 16 heads; NBUF key tiles in an LDS ring (kLead of them in flight);
// QD / PD fragment reads in flight ahead of the Q.K / P.V MFMAs.
template <int NW, int NBUF, int QD, int PD>
__global__ __launch_bounds__(NW * kWave, 8 / NW) void mla_decode_kernel(MlaArgs a) {
  constexpr int KS = (kD + kR) / 32;  // 18 contraction steps (16 latent + 2 rope)
  constexpr int DT = kD / 16;         // 32 row tiles of O^T
  constexpr int NT = NW * kWave;
  constexpr int kRopeLoads = kKeyTile * kR / (8 * kWave);  // 4 wave loads of eight rope rows
  constexpr int kRows = kKeyTile / NW;                     // latent rows per wave and tile
  // Wave loads per tile: rope load k goes to wave k % NW.
  constexpr int NL_LO = kRows + (kRopeLoads + NW - 1) / NW;  // waves < kRopeLoads % NW (or all)
  constexpr int NL_HI = kRows + kRopeLoads / NW;
  static_assert(kKeyTile % NW == 0 && NBUF >= 2 && NBUF <= 4, "tile split");
  // Tiles in flight beyond the current one.  The 4-slot ring keeps two, so a slot
  // is refilled two barriers after its last read; against three in flight it
  // measured 0-2 % faster on MLA decode and equal on the multi-token decode and
  // the chunked prefill.
  constexpr int kLead = NBUF >= 4 ? NBUF - 2 : NBUF - 1;
  __shared__ __attribute__((aligned(16))) uint16_t c_lds[NBUF][kKeyTile][kRow];
  __shared__ __attribute__((aligned(16))) uint16_t r_lds[NBUF][kKeyTile][kR];
  __shared__ int32_t s_blk[kMaxBpp];

  int part = blockIdx.x;
  int hg = blockIdx.y;
  int zi = blockIdx.z;
  if (a.cu_seqlens_q) {
    // Prefill: workgroups are dealt to the 8 XCDs round robin by launch order.
    // Renumber them so that each XCD takes a contiguous run of query rows --
    // neighbouring rows of one sequence read the same latent tiles and then
    // share that XCD's L2.  The grid is padded to a multiple of 8.
    const int nwg = gridDim.x * gridDim.y * gridDim.z;
    const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int logical = (lin & 7) * (nwg >> 3) + (lin >> 3);
    part = logical % gridDim.x;
    hg = (logical / gridDim.x) % gridDim.y;
    zi = logical / (gridDim.x * gridDim.y);
    if (zi >= a.rows - a.row0) return;  // padding workgroup
  }
  const int row = a.row0 + zi;  // query row: the sequence (decode) or a row of q (prefill)
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int H = a.num_q_heads;
  const int head = (hg * NW + wave) * 16 + l16;
  const int64_t qrow = (int64_t)row * H + head;

  // Decode: row b attends to the L = seq_lens[b] keys of sequence b.  Prefill:
  // row i of sequence b (cu[b] <= row < cu[b+1], n = cu[b+1] - cu[b] new rows)
  // sits at position seq_lens[b] - n + i and attends to the keys up to it, i.e.
  // it is a decode of length seq_lens[b] - n + i + 1 over sequence b's table.
  int b = row;
  int32_t L;
  if (a.cu_seqlens_q) {
    const int32_t* cu = a.cu_seqlens_q;
    int lo_b = 0, hi_b = a.batch - 1;  // the last b with cu[b] <= row
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if (cu[mid] <= row) lo_b = mid; else hi_b = mid - 1;
    }
    b = lo_b;
    L = a.seq_lens[b] - (cu[b + 1] - cu[b]) + (row - cu[b]) + 1;
  } else {
    L = a.seq_lens[b];
  }
  const KeySpan sp = decode_span(L, a.window, a.block_size_log2, a.blocks_per_part);
  if (part >= sp.np) {
    if (a.max_np == 1 && sp.np == 0 && part == 0) {
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
  for (int i = tid; i < nblk; i += NT) s_blk[i] = bt[i];

  const uint16_t* qn = static_cast<const uint16_t*>(a.q);
  const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope);
  uint4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = ks < kD / 32 ? ld16(qn + qrow * kD + 32 * ks + 8 * lg)
                          : ld16(qr + qrow * kR + 32 * (ks - kD / 32) + 8 * lg);
  retire_loads();  // q fragments are in registers before any tile is in flight
  __syncthreads();  // s_blk ready

  const uint16_t* cn = static_cast<const uint16_t*>(a.c_nope);
  const uint16_t* cr = static_cast<const uint16_t*>(a.c_rope);
  const int rope_row = lane >> 3;                                      // row within a rope load
  const uint32_t rope_voff = 16 * ((lane & 7) ^ rope_swz(rope_row));  // 8-row steps keep r & 7

  // Copy key tile t0 into ring slot buf.  Keys outside [tok_begin, tok_end)
  // re-read a visible row: they are masked, and a finite row keeps 0 * c = 0
  // (spare table entries may point at a NaN-filled block).
  auto issue_tile = [&](int t0, int buf) {
    if (t0 >= tok_begin && t0 + kKeyTile <= tok_end && bs_log2 >= 5) {
      // One block holds the whole tile and every row is visible: scalar bases.
      const int phys = __builtin_amdgcn_readfirstlane(s_blk[(t0 >> bs_log2) - blk0]);
      const int64_t row0 = ((int64_t)phys << bs_log2) + (t0 & bs_mask);
      const uint16_t* cb = cn + row0 * kD;
      const uint16_t* rb = cr + row0 * kR;
#pragma unroll
      for (int k = 0; k < kRows; ++k) {
        const int i = wave + k * NW;
        load_lds16_s(cb, (uint32_t)(i * kD * 2) + 16 * lane, &c_lds[buf][i][0]);
      }
#pragma unroll
      for (int k = 0; k < kRopeLoads; ++k)
        if (k % NW == wave) load_lds16_s(rb, (uint32_t)((8 * k + rope_row) * kR * 2) + rope_voff, &r_lds[buf][8 * k][0]);
      return;
    }
    auto slot_of = [&](int j) -> int64_t {
      j = min(max(j, tok_begin), tok_end - 1);
      return ((int64_t)s_blk[(j >> bs_log2) - blk0] << bs_log2) + (j & bs_mask);
    };
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int i = wave + k * NW;
      load_lds16(cn + slot_of(t0 + i) * kD + 8 * lane, &c_lds[buf][i][0]);
    }
#pragma unroll
    for (int k = 0; k < kRopeLoads; ++k)
      if (k % NW == wave)
        load_lds16(cr + slot_of(t0 + 8 * k + rope_row) * kR + rope_voff / 2, &r_lds[buf][8 * k][0]);
  };

  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_zero();
  float mref = kNegInf, l = 0.f;  // reference maximum in log2 units, running sum
  const float c2 = a.scale_log2e;
  const int q4 = l16 & 3;
  const int ra = 4 * lg + (l16 >> 2);  // rows of this lane's transposed reads
  const int rb = ra + 16;

  const int t_first = tok_begin & ~(kKeyTile - 1);
  const int ntiles = (tok_end - t_first + kKeyTile - 1) / kKeyTile;
#pragma unroll
  for (int k = 0; k < kLead; ++k)
    if (k < ntiles) issue_tile(t_first + k * kKeyTile, k);

  for (int it = 0; it < ntiles; ++it) {
    const int t0 = t_first + it * kKeyTile;
    const int buf = it % NBUF;
    const int ahead = min(kLead - 1, ntiles - 1 - it);
    if (wave < kRopeLoads % NW || kRopeLoads % NW == 0)
      wait_tile<NL_LO, kLead - 1>(ahead);
    else
      wait_tile<NL_HI, kLead - 1>(ahead);
    __syncthreads();  // tile it is visible; slot (it + kLead) % NBUF was last read before it
    if (it + kLead < ntiles) issue_tile(t0 + kLead * kKeyTile, (it + kLead) % NBUF);

    // S^T = C.Q^T over 18 contraction steps for both 16-key halves, the steps
    // of the two halves interleaved; each fragment is read QD steps ahead of
    // its MFMA (scheduling barriers keep the read there), so the LDS latency
    // overlaps the MFMAs instead of stalling every step.
    constexpr int NF = 2 * KS;
    auto c_frag = [&](int f) {
      const int ks = f >> 1, r = 16 * (f & 1) + l16;
      return ks < kD / 32 ? lds16(&c_lds[buf][r][32 * ks + 8 * lg])
                          : lds16(&r_lds[buf][r][8 * ((4 * (ks - kD / 32) + lg) ^ rope_swz(r))]);
    };
    f32x4_t s[2] = {f32x4_zero(), f32x4_zero()};
    uint4 cf[QD + 1];
#pragma unroll
    for (int f = 0; f < QD; ++f) cf[f] = c_frag(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f + QD < NF) cf[(f + QD) % (QD + 1)] = c_frag(f + QD);
      __builtin_amdgcn_sched_barrier(0);
      s[f & 1] = mfma_bf16(cf[f % (QD + 1)], qf[f >> 1], s[f & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!(t0 >= tok_begin && t0 + kKeyTile <= tok_end)) {
#pragma unroll
      for (int u = 0; u < kKeyTile / 16; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = t0 + 16 * u + 4 * lg + r;
          s[u][r] = (j >= tok_begin && j < tok_end) ? s[u][r] : kNegInf;
        }
    }
    // Probabilities against the current reference and this lane's sum of them; the
    // column maximum (to raise the reference) is formed only when some lane's sum
    // exceeds 2^8 -- which any probability above 2^8 implies -- and the
    // probabilities are then taken again.
    float p8[8];
    float ls;
    auto probs = [&](float mb) {
      ls = 0.f;
#pragma unroll
      for (int u = 0; u < kKeyTile / 16; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = exp2_fast(fmaf(s[u][r], c2, -mb));
          p8[4 * u + r] = p;
          ls += p;
        }
    };
    probs(mref == kNegInf ? 0.f : mref);
    if (__any(mref == kNegInf || !(ls <= kRaiseSum))) {  // !(<=): a NaN or inf sum too
      float mt = kNegInf;
#pragma unroll
      for (int u = 0; u < kKeyTile / 16; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s[u][r]);
      const float mts = row4_max(mt) * c2;
      const bool raise = mts > mref + kRescaleLog2;
      if (__any(raise)) {
        const float alpha = raise ? exp2_fast(mref - mts) : 1.f;  // mref = -inf gives 0
        if (raise) mref = mts;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      }
      probs(mref == kNegInf ? 0.f : mref);  // no finite score yet: every p is 0
    }
    l += ls;
    uint4 phi, plo;
    pack_p_split(p8, phi, plo);
    // O^T += C^T.P^T: the transposed fragment of row tile dt is read PD tiles ahead.
    auto v_frag = [&](int dt) {
      const uint2 x0 = lds_tr16(&c_lds[buf][ra][16 * dt + 4 * q4]);
      const uint2 x1 = lds_tr16(&c_lds[buf][rb][16 * dt + 4 * q4]);
      return make_uint4(x0.x, x0.y, x1.x, x1.y);
    };
    uint4 vf[PD + 1];
#pragma unroll
    for (int dt = 0; dt < PD; ++dt) vf[dt] = v_frag(dt);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (dt + PD < DT) vf[(dt + PD) % (PD + 1)] = v_frag(dt + PD);
      __builtin_amdgcn_sched_barrier(0);
      o[dt] = mfma_bf16(vf[dt % (PD + 1)], phi, o[dt]);
      o[dt] = mfma_bf16(vf[dt % (PD + 1)], plo, o[dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  const float lsum = row4_sum(l);
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
      a.ws_ml[(qrow * a.max_np + part) * 2 + 0] = mref;  // log2 units, like the VALU decode
      a.ws_ml[(qrow * a.max_np + part) * 2 + 1] = lsum;
    }
  }
}

}  // namespace

bool mla_decode_supported(int32_t dtype, int32_t head_dim, int32_t rope_dim, int32_t num_q_heads) {
  return dtype == PKV_BF16 && head_dim == kD && rope_dim == kR && num_q_heads % 16 == 0;
}

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t stream) {
  const int tiles16 = a.num_q_heads / 16;
  if (a.batch == 0 || a.rows == 0) return hipSuccess;
  if (a.blocks_per_part > kMaxBpp) return hipErrorInvalidValue;
  // Up to 8 waves (128 heads) per workgroup; the head groups tile H exactly.
  int nw = 8;
  while (tiles16 % nw) nw >>= 1;
  // Query rows go in launches of at most 65528 (the grid's z limit, rounded
  // down to a multiple of 8); prefill pads each launch to a multiple of 8
  // workgroups for the XCD renumbering (extra rows exit at once).
  for (int32_t r0 = 0; r0 < a.rows; r0 += 65528) {
    MlaArgs c = a;
    c.row0 = r0;
    int32_t nz = std::min<int32_t>(65528, a.rows - r0);
    if (a.cu_seqlens_q) {
      const int64_t per_z = (int64_t)a.max_np * (tiles16 / nw);
      while ((per_z * nz) % 8) ++nz;
    }
    const dim3 grid(a.max_np, tiles16 / nw, (unsigned)nz);
    switch (nw) {
      // One 8-wave workgroup per CU can hold a 4-deep ring (152 KiB of LDS);
      // smaller workgroups keep two slots so that several fit on a CU.
      case 8: mla_decode_kernel<8, 4, kQkAhead, kPvAhead><<<grid, 8 * kWave, 0, stream>>>(c); break;
      case 4: mla_decode_kernel<4, 2, kQkAhead, kPvAhead><<<grid, 4 * kWave, 0, stream>>>(c); break;
      case 2: mla_decode_kernel<2, 2, kQkAhead, kPvAhead><<<grid, 2 * kWave, 0, stream>>>(c); break;
      default: mla_decode_kernel<1, 2, kQkAhead, kPvAhead><<<grid, 1 * kWave, 0, stream>>>(c); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pkv
