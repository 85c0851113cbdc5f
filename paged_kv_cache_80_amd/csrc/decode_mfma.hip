// decode_mfma.hip -- paged decode on the matrix cores with a stream split.
//
// Same result as decode.hip (softmax(q.K^T * scale) V over the keys the newest
// position sees, query head h reading KV head h / G: "KV Cache notes", the
// attention formula, its decode form and the MHA -> MQA -> GQA section), for
// bf16 caches with 128-wide heads.  The G query heads that share a KV head are
// the columns of the MFMA tiles (padded to 16): S^T = K.Q^T and O^T += V^T.P^T
// run on v_mfma_f32_16x16x32_bf16 per 32-key tile, so the vector ALUs only run
// the online softmax and a KV row is read from HBM once for all G heads.
//
// Work split (stream split).  The 32-key tiles of all sequences are laid end to
// end as one list of C tile columns (a column is one tile position of one
// sequence, for all H_kv heads).  The launch holds exactly the waves that are
// resident at once, taken as NG groups of H_kv waves; group x takes the
// contiguous run of columns [C x / NG, C (x+1) / NG) and its wave g streams KV
// head g of those columns.  Every wave streams the same number of tiles however
// ragged the lengths are, with no partition size to trade tail imbalance against
// start-up cost; waves are dealt to the 8 XCDs round robin, so every XCD streams
// the same share; and the H_kv waves of a group read the same slot rows (one
// row holds every head of a token) at about the same time, which keeps DRAM
// pages open.  A run crosses sequence ends.  A sequence that the group holds
// whole is normalised and stored by its waves; otherwise the wave stores the
// partial (m, l, O) of the piece of sequence b it holds as piece (x + b)
// H_kv + g (a group boundary and a sequence boundary never produce the same
// x + b), and stream_combine merges the pieces of each output row.  Both kernels need the
// per-sequence column prefix of seq_lens: each decode workgroup scans it into
// LDS at start (workgroup 0 also stores it for the combine), or, for batches
// of 2048 sequences and more, a small scan kernel writes it first.
//
// Data path.  Each wave owns two LDS slots of one tile (K and V, 16 KiB) and
// streams tile k + 1 into one while it computes tile k from the other.  The
// copies are global_load_lds DMAs: 16 lanes read one 256-byte head row, a wave
// instruction four whole rows, the way they lie in memory (loading K straight
// into the MFMA operand layout would put 16 different rows on consecutive
// lanes and make the L1 serve every lane separately), and no register holds a
// tile in flight.  A DMA writes lane l's 16 bytes at 16 l of its 1 KiB LDS
// destination, so the swizzles of the slot layout are applied on the source
// side: the lane that fills chunk position p of row r reads logical chunk
// p ^ swz(r).  The slots are re-read as MFMA operands: K with ds_read_b128 (its
// chunks XOR-swizzled by row & 15 so the 16 rows of an operand read fall in
// distinct banks), V transposed with ds_read_b64_tr_b16 (chunks swizzled by
// 2 * (row & 7) for the same reason).  Four waves per CU with one tile in flight
// each keep HBM saturated for plain streams, and that is what 128 KiB of slots
// per workgroup allows.
//
// Online softmax.  Logits are in log2 units (scale * log2 e folded into one
// FMA before v_exp_f32).  A column's reference maximum is raised only when a
// tile's maximum exceeds it by more than 2^8 in probability; in between,
// probabilities up to 256 accumulate against the stale reference, which is
// exact (O and l share it) and skips the O rescale on almost every tile.
// Probabilities enter P.V as a hi + lo bf16 pair (p = hi + lo + r, |r| < 2^-15
// p), so rounding P costs no accuracy.
//
// INT8 caches (I8).  A tile then holds 32 rows of 128 int8 codes per tensor
// (4 KiB) plus the 32 K and 32 V scales of the tile's keys (256 bytes, one more
// DMA).  Codes become bf16 in registers after the LDS read (exact: at most 8
// significant bits), so the same MFMAs run: S^T = Kq.Q^T is scaled per key by
// its K scale, and the V scales fold into P before the hi/lo split
// (sum_j p_j s_j v_j = (p . s) . Vq).  V^T operands come from the byte
// transposing read ds_read_b64_tr_b8, which hands a lane 8 consecutive keys of
// one dim; to match, the K operand rows are ordered so that S^T lane (n, lg)
// holds keys 8 lg .. 8 lg + 7 (tile u row m is key 8 (m / 4) + 4 u + m % 4).
#include "mfma_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kD = 128;
constexpr int kKeyTile = 32;
constexpr int kTileLog2 = 5;
constexpr int kRowBytes = kD * 2;                 // 256: one head row of K or V
constexpr int kWaves = 4;                         // independent waves per workgroup (bf16)
constexpr int kWavesI8 = 8;                       // int8: half-size slots leave LDS for twice the waves
constexpr float kRescaleLog2 = 8.f;
constexpr float kRaiseSum = 256.f;  // 2^kRescaleLog2: a lane sum at most this has no p above it

// Tile geometry per cache type: bytes of one head row, of one tensor of a tile,
// of a whole LDS slot (K, V and, for int8, the tile's 32 + 32 scales), and the
// DMA instructions that fill a slot.
template <bool I8>
struct Geo {
  static constexpr int kRow = I8 ? kD : 2 * kD;
  static constexpr int kTile = kKeyTile * kRow;
  static constexpr int kSlot = 2 * kTile + (I8 ? 2 * kKeyTile * 4 : 0);
  static constexpr int kDma = I8 ? 9 : 16;
};
constexpr int kLdsPrefix = 2048;                   // batch + 1 up to this: prefix scanned in LDS
constexpr int kStreamCols = kStreamMtColumns;      // columns of a multi-token decode piece (two tiles)

// 16-byte chunk swizzles of row r in the staged K and V tiles.
__device__ __forceinline__ int kswz(int r) { return r & 15; }
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 7); }
// int8 tiles (8 chunks per 128-byte row).  K operand rows of tile u are
// r = 8 (l16 / 4) + 4 u + l16 % 4; with j = l16 = 4 (r / 8) + r % 4 the chunk
// position is c ^ ((j / 2) ^ 4 (j % 2)): lanes 0..7 of a 16-byte read hit 8
// distinct positions and lanes 0..15 distinct (row parity, position) pairs, so
// the read is conflict-free with 8 or with 16 lanes served per cycle.  V rows
// of a transposing read (8 consecutive rows, two such groups per half wave)
// take position dt ^ (r % 8) ^ (r / 8 % 2).
__device__ __forceinline__ int kswz8(int r) {
  const int j = 4 * ((r >> 3) & 3) + (r & 3);
  return (j >> 1) ^ ((j & 1) << 2);
}
__device__ __forceinline__ int vswz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Scalar (SMEM) load of a value that is uniform across the wave and read-only
// for the whole kernel.  Vector loads retire in order, so a vector load of
// such metadata would make every wait for it also wait for the tiles in flight.
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Keys some query of a sequence of length L sees, when its last n keys are query
// rows (n = 1: decode): row i sits at position L - n + i and sees (pos - W, pos]
// with a window W, so together they see [lo, L), lo = L - n + 1 - W.
__device__ __forceinline__ int32_t visible_lo(int32_t L, int32_t window, int32_t n) {
  return (window > 0 && L - n + 1 > window) ? L - n + 1 - window : 0;
}
// 32-key tiles covering [lo, L), aligned to absolute positions (none without a row).
__device__ __forceinline__ int32_t seq_tiles(int32_t L, int32_t window, int32_t n) {
  if (L <= 0 || n <= 0) return 0;
  return ((L - 1) >> kTileLog2) - (visible_lo(L, window, n) >> kTileLog2) + 1;
}
// Query rows of sequence b: one per sequence in decode, n_b from cu_seqlens_q
// in multi-token decode.
__device__ __forceinline__ int32_t seq_rows(const int32_t* cu, int32_t b) { return cu ? cu[b + 1] - cu[b] : 1; }

// Wave groups that share the C columns: every resident group, or fewer when a
// target number of tiles per wave is given (split_tiles > 0), and never more
// groups than columns (a group without a column would only leave an empty slot
// for the combine to skip).
__device__ __forceinline__ int64_t stream_groups(int64_t C, int32_t resident_waves, int32_t Hkv,
                                                 int32_t split_tiles) {
  int64_t ng = resident_waves / Hkv;  // >= 1: the host checks H_kv <= resident waves
  if (split_tiles > 0) ng = min(ng, max<int64_t>(1, (C + split_tiles - 1) / split_tiles));
  return max<int64_t>(1, min(ng, C));
}
// The group whose run [C x / NG, C (x+1) / NG) holds column t.
__device__ __forceinline__ int64_t group_of_column(int64_t t, int64_t C, int64_t ng) {
  return ((t + 1) * ng - 1) / C;
}

// prefix[b] = sum of seq_tiles over sequences < b (prefix[B] = all columns).
// One workgroup of 1024 threads scans 1024 sequences per step.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ seq_lens,
                                                           const int32_t* __restrict__ cu, int32_t B, int32_t window,
                                                           int32_t* __restrict__ prefix) {
  __shared__ int32_t s_scan[1024];
  const int tid = threadIdx.x;
  int32_t run = 0;
  if (tid == 0) prefix[0] = 0;
  for (int32_t base = 0; base < B; base += 1024) {
    const int32_t b = base + tid;
    s_scan[tid] = b < B ? seq_tiles(seq_lens[b], window, seq_rows(cu, b)) : 0;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
      const int32_t add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    if (b < B) prefix[b + 1] = run + s_scan[tid];
    run += s_scan[1023];
    __syncthreads();
  }
}

// Position of a wave in the column list: sequence b, tile k of its n tiles.
struct Cursor {
  int32_t b, k, n;
  int32_t lo, L;     // keys [lo, L) of sequence b that some query row sees
  int32_t t_first;   // first key of tile 0 (lo rounded down to a tile)
  int32_t nq, q0;    // query rows of sequence b and the first one's index
};

// ONE_BLOCK: the block size is 32 or more, so a 32-key tile never straddles
// two blocks; otherwise it is 16 and a tile spans two.
// LDS_PREFIX: every workgroup scans seq_lens into its own LDS copy of the
// column prefix (batch + 1 <= kLdsPrefix) and workgroup 0 also stores it for
// the combine; otherwise tile_prefix_kernel has written it to the workspace.
// MT: multi-token decode -- sequence b has n_b query rows (cu_seqlens_q) at its
// last n_b positions, each seeing the keys up to its own position (bottom-right
// causal); the columns of a wave are then the (row, head) pairs of its KV head,
// row-major, in two 16-column tiles.
template <bool ONE_BLOCK, bool LDS_PREFIX, bool I8, bool MT>
__global__ __launch_bounds__((I8 ? kWavesI8 : kWaves) * kWave, 1) void decode_stream_kernel(DecodeArgs a) {
  constexpr int KS = kD / 32;  // contraction steps of q.k
  constexpr int DT = kD / 16;  // 16-row tiles of O^T
  constexpr int CT = MT ? 2 : 1;  // 16-column tiles per wave
  static_assert(!(MT && I8), "multi-token decode reads bf16 caches");
  constexpr int NW = I8 ? kWavesI8 : kWaves;
  using GT = Geo<I8>;
  __shared__ __attribute__((aligned(16))) unsigned char lds_buf[NW * 2 * GT::kSlot];
  __shared__ int32_t s_prefix[LDS_PREFIX ? kLdsPrefix : 1];
  __shared__ int32_t s_wave_sum[NW];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int B = a.batch;
  const int H = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int G = H / Hkv;
  if constexpr (LDS_PREFIX) {
    // Thread t owns sequences [kPerThread t, kPerThread (t + 1)): local sums,
    // a wave scan of the thread totals, then the waves' totals through LDS.
    constexpr int kPerThread = kLdsPrefix / (NW * kWave);
    int32_t incl[kPerThread], nrow[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {  // all loads first (clamped: B >= 1), then the sums
      const int bb = min(kPerThread * tid + j, B - 1);
      incl[j] = a.seq_lens[bb];
      nrow[j] = MT ? a.cu_seqlens_q[bb + 1] - a.cu_seqlens_q[bb] : 1;
    }
    int32_t run = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      run += kPerThread * tid + j < B ? seq_tiles(incl[j], a.window, nrow[j]) : 0;
      incl[j] = run;
    }
    int32_t x = run;  // inclusive scan of the thread totals over the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) s_wave_sum[wave] = x;
    __syncthreads();
    int32_t excl = x - run;
    for (int w2 = 0; w2 < wave; ++w2) excl += s_wave_sum[w2];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int b = kPerThread * tid + j;
      if (b < B) s_prefix[b + 1] = excl + incl[j];
    }
    if (tid == 0) s_prefix[0] = 0;
    __syncthreads();
    if (blockIdx.x == 0)
      for (int i = tid; i <= B; i += NW * kWave) a.tile_prefix[i] = s_prefix[i];
  }
  // prefix[i]: columns of the sequences before i (prefix[B] = all columns).
  auto prefix_at = [&](int i) -> int32_t {
    if constexpr (LDS_PREFIX) return __builtin_amdgcn_readfirstlane(s_prefix[i]);
    else return sload(a.tile_prefix + i);
  };

  const int64_t C = prefix_at(B);
  const int64_t NG = stream_groups(C, gridDim.x * NW, Hkv, a.split_tiles);
  const int64_t w = (int64_t)blockIdx.x * NW + wave;
  const int64_t grp = w / Hkv;  // wave-uniform
  const int g = (int)(w - grp * Hkv);
  if (grp >= NG) return;
  const int64_t c_beg = C * grp / NG, c_end = C * (grp + 1) / NG;
  if (c_beg >= c_end) return;

  // Locate the first column: the sequence b with prefix[b] <= c_beg < prefix[b+1].
  Cursor c0;
  {
    int lo_b = 0, hi_b = B - 1;
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if (prefix_at(mid) <= c_beg) lo_b = mid; else hi_b = mid - 1;
    }
    c0.b = lo_b;
    const int32_t p0 = prefix_at(lo_b);
    c0.n = prefix_at(lo_b + 1) - p0;
    c0.k = (int)(c_beg - p0);
    c0.L = sload(a.seq_lens + c0.b);
    c0.q0 = MT ? sload(a.cu_seqlens_q + c0.b) : c0.b;
    c0.nq = MT ? sload(a.cu_seqlens_q + c0.b + 1) - c0.q0 : 1;
    c0.lo = visible_lo(c0.L, a.window, c0.nq);
    c0.t_first = c0.lo & ~(kKeyTile - 1);
  }
  auto advance = [&](Cursor& c) {
    if (++c.k < c.n) return;
    c.k = 0;
    do {  // the next sequence with a visible key (the run ends before B)
      ++c.b;
      c.n = c.b < B ? prefix_at(c.b + 1) - prefix_at(c.b) : 1;
    } while (c.n == 0);
    if (c.b < B) {
      c.L = sload(a.seq_lens + c.b);
      c.q0 = MT ? sload(a.cu_seqlens_q + c.b) : c.b;
      c.nq = MT ? sload(a.cu_seqlens_q + c.b + 1) - c.q0 : 1;
      c.lo = visible_lo(c.L, a.window, c.nq);
      c.t_first = c.lo & ~(kKeyTile - 1);
    }
  };

  const int64_t row_elems = (int64_t)Hkv * kD;  // elements between consecutive slots
  const uint32_t row_bytes = (uint32_t)row_elems * (I8 ? 1 : 2);
  const int bs_log2 = a.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const uint16_t* kcache = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vcache = static_cast<const uint16_t*>(a.v_cache);
  const unsigned char* kcache8 = static_cast<const unsigned char*>(a.k_cache);
  const unsigned char* vcache8 = static_cast<const unsigned char*>(a.v_cache);

  // Lane constants.  DMA instruction i of a tensor fills rows 4i + lg; lane
  // (l16, lg) fills chunk position l16 and so reads logical chunk l16 ^ swz(r),
  // where r & 15 = 4(i & 3) + lg (K) and r & 7 = 4(i & 1) + lg (V).
  uint32_t k_src[4], v_src[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) k_src[i] = 16 * (l16 ^ kswz(4 * i + lg));
#pragma unroll
  for (int i = 0; i < 2; ++i) v_src[i] = 16 * (l16 ^ vswz(4 * i + lg));
  // K operand of step ks: key row 16u + l16, chunk 4ks + lg (row & 15 = l16).
  int kr_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kr_off[ks] = l16 * kRowBytes + 16 * ((4 * ks + lg) ^ l16);
  // V^T operand of 16-dim tile dt: row ra = 4lg + l16/4, 8 bytes at column
  // 16dt + 4(l16 & 3); row ra + 16 has the same swizzle.
  const int ra = 4 * lg + (l16 >> 2);
  int vr_off[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) vr_off[dt] = ra * kRowBytes + 32 * (dt ^ (ra & 7)) + 8 * (l16 & 3);
  // int8: DMA instruction i of K fills rows 8i + lane/8, chunk position lane % 8
  // (logical chunk (lane % 8) ^ kswz8(row)); V likewise with vswz8(row) = lane / 8.
  // K operand (tile u, step ks): row 8(l16/4) + 4u + l16%4, bytes 32ks + 8lg.
  // V^T operand of dim tile dt: the transposing read of row 8lg + l16/2, half
  // l16 % 2 of logical chunk dt.
  // The contraction order of q.k is permuted for int8: step ks of lane group lg
  // takes dims 16 (lg + 4 (ks / 2)) + 8 (ks % 2) .. + 8, so one 16-byte read of
  // chunk lg (or lg + 4) of a K row feeds two steps.
  uint32_t k_src8[4], v_src8[2] = {0, 0};
  int kr8_off[2][2], vr8_off[DT];
  if constexpr (I8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) k_src8[i] = 16 * ((lane & 7) ^ kswz8(8 * i + (lane >> 3)));
#pragma unroll
    for (int i = 0; i < 2; ++i) v_src8[i] = 16 * ((lane & 7) ^ vswz8(8 * i + (lane >> 3)));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * (l16 >> 2) + 4 * u + (l16 & 3);
        kr8_off[u][h] = r * GT::kRow + 16 * ((lg + 4 * h) ^ kswz8(r));
      }
    const int rv = 8 * lg + (l16 >> 1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vr8_off[dt] = rv * GT::kRow + 16 * (dt ^ vswz8(rv)) + 8 * (l16 & 1);
  }
  unsigned char* slots = lds_buf + wave * 2 * GT::kSlot;

  // Copy the tile at cursor c (16 DMAs: K rows then V rows) into slot `sl`.
  // Rows outside [lo, L) re-read a visible row of the tile: they are masked
  // later, and a finite row keeps 0 * v = 0 (table entries outside the visible
  // keys may point at a NaN-filled block).
  auto issue_tile = [&](const Cursor& c, int sl) {
    const int t0 = c.t_first + (c.k << kTileLog2);
    const int lo_r = max(c.lo - t0, 0);
    const int hi_r = min(c.L - t0, kKeyTile) - 1;
    const int32_t* bt = a.block_table + (int64_t)c.b * a.max_blocks_per_seq;
    const int64_t head_off = (int64_t)g * kD;
    unsigned char* kdst = slots + sl * GT::kSlot;
    unsigned char* vdst = kdst + GT::kTile;
    if constexpr (I8) {
      // 4 + 4 row DMAs (8 rows of 128 codes each) and one for the scales: lanes
      // 0..7 bring the K scales of keys 4l .. 4l + 3, lanes 8..15 the V scales.
      // Scales of keys outside [lo, L) are read too (in bounds: the tile's
      // block(s)) and masked out in compute; rows are clamped as below.
      unsigned char* sdst = vdst + GT::kTile;
      const int blk = t0 >> bs_log2;
      const float* scale_src = lane < 8 ? a.k_scale : a.v_scale;
      const int key = 4 * (lane & 7);
      if constexpr (ONE_BLOCK) {
        const int32_t phys = sload(bt + blk);
        const int64_t row0 = ((int64_t)phys << bs_log2) + (t0 & bs_mask);
        const unsigned char* kb = kcache8 + row0 * row_bytes + head_off;
        const unsigned char* vb = vcache8 + row0 * row_bytes + head_off;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t row = (uint32_t)min(max(8 * i + (lane >> 3), lo_r), hi_r) * row_bytes;
          load_lds16_s(kb, row + k_src8[i], kdst + 1024 * i);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t row = (uint32_t)min(max(8 * i + (lane >> 3), lo_r), hi_r) * row_bytes;
          load_lds16_s(vb, row + v_src8[i & 1], vdst + 1024 * i);
        }
        if (lane < 16)
          load_lds16(scale_src + ((((int64_t)phys * Hkv + g) << bs_log2) + (t0 & bs_mask) + key), sdst);
      } else {
        const int32_t e0 = sload(bt + blk);
        const int32_t e1 = ((blk + 1) << bs_log2) < c.L ? sload(bt + blk + 1) : e0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = t0 + min(max(8 * i + (lane >> 3), lo_r), hi_r);
          const int32_t phys = (j >> bs_log2) == blk ? e0 : e1;
          const int64_t slot = ((int64_t)phys << bs_log2) + (j & bs_mask);
          load_lds16(kcache8 + slot * row_bytes + head_off + k_src8[i], kdst + 1024 * i);
          load_lds16(vcache8 + slot * row_bytes + head_off + v_src8[i & 1], vdst + 1024 * i);
        }
        if (lane < 16) {
          // The lane's 4 keys lie in one 16-key block.  A block wholly before the
          // window start has a table entry that may hold anything (the null
          // block, or no block id at all): its lanes read the other block's
          // scales instead, which hold a visible key and are masked like the rest.
          const int j = t0 + key;
          const bool blk_visible = ((blk + 1) << bs_log2) > c.lo;
          const int32_t phys = ((j >> bs_log2) == blk && blk_visible) ? e0 : e1;
          load_lds16(scale_src + ((((int64_t)phys * Hkv + g) << bs_log2) + (j & bs_mask)), sdst);
        }
      }
    } else {
      // Append fused in: the sequence's newest key (row rn of this tile) comes
      // from k_new / v_new rather than the cache, and this wave -- the only one
      // that reads that row of KV head g -- stores it at its slot.  Nothing in
      // this kernel reads the slot, so the store needs no ordering.
      bool has_new = false;
      int rn = 0;
      if constexpr (!MT) {
        rn = c.L - 1 - t0;
        has_new = a.k_new != nullptr && rn >= 0 && rn < kKeyTile;
      }
      if (ONE_BLOCK && !has_new) {  // one table entry, a wave-uniform base and 32-bit lane offsets
        const int32_t phys = sload(bt + (t0 >> bs_log2));
        const int64_t row0 = ((int64_t)phys << bs_log2) + (t0 & bs_mask);
        const uint16_t* kb = kcache + row0 * row_elems + head_off;
        const uint16_t* vb = vcache + row0 * row_elems + head_off;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t row = (uint32_t)min(max(4 * i + lg, lo_r), hi_r) * row_bytes;
          load_lds16_s(kb, row + k_src[i & 3], kdst + 1024 * i);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t row = (uint32_t)min(max(4 * i + lg, lo_r), hi_r) * row_bytes;
          load_lds16_s(vb, row + v_src[i & 1], vdst + 1024 * i);
        }
      } else {
        // Per-lane addresses: 16-token blocks (the tile spans blocks blk and
        // blk + 1, the second only if it holds a visible key; both entries are
        // scalar reads), or the tile holding the newest key.
        const int blk = t0 >> bs_log2;
        const int32_t e0 = sload(bt + blk);
        const int32_t e1 = ((blk + 1) << bs_log2) < c.L ? sload(bt + blk + 1) : e0;
        const int64_t new_off = ((int64_t)c.b * a.num_kv_heads + g) * kD * 2;  // bytes
        const unsigned char* kn = has_new ? static_cast<const unsigned char*>(a.k_new) + new_off : nullptr;
        const unsigned char* vn = has_new ? static_cast<const unsigned char*>(a.v_new) + new_off : nullptr;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = min(max(4 * i + lg, lo_r), hi_r);
          const int j = t0 + r;
          const int32_t phys = (j >> bs_log2) == blk ? e0 : e1;
          const int64_t slot = ((int64_t)phys << bs_log2) + (j & bs_mask);
          const bool from_new = has_new && r == rn;
          const unsigned char* kr =
              from_new ? kn : reinterpret_cast<const unsigned char*>(kcache + slot * row_elems + head_off);
          const unsigned char* vr =
              from_new ? vn : reinterpret_cast<const unsigned char*>(vcache + slot * row_elems + head_off);
          load_lds16(kr + k_src[i & 3], kdst + 1024 * i);
          load_lds16(vr + v_src[i & 1], vdst + 1024 * i);
        }
        if (has_new && lane < 32) {
          const int j = c.L - 1;
          const int32_t phys = (j >> bs_log2) == blk ? e0 : e1;
          const int64_t slot = ((int64_t)phys << bs_log2) + (j & bs_mask);
          // The cache is the caller's writable memory; DecodeArgs carries it const
          // because no other path of this kernel writes it.
          uint16_t* dst = const_cast<uint16_t*>(lane < 16 ? kcache : vcache) + slot * row_elems + head_off;
          const unsigned char* src = lane < 16 ? kn : vn;
          st16(dst + 8 * l16, ld16(src + 16 * l16));
        }
      }
    }
  };

  // Column l16 of tile ct: query head g G + l16 (decode), or (row, head) pair
  // 16 ct + l16 of the sequence's rows x G heads (multi-token decode), whose row
  // sits at position cpos.
  bool cvalid[CT];
  int32_t cpos[CT];
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  uint4 qf[CT][KS];
  auto load_q = [&](const Cursor& c) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      int64_t qrow;
      if constexpr (MT) {
        const int col = 16 * ct + l16;
        const int i = col / G;
        cvalid[ct] = i < c.nq;
        cpos[ct] = c.L - c.nq + i;
        qrow = (int64_t)(c.q0 + (cvalid[ct] ? i : 0)) * H + (int64_t)g * G + (col - i * G);
      } else {
        cvalid[ct] = l16 < G;
        cpos[ct] = c.L - 1;
        qrow = (int64_t)c.q0 * H + (int64_t)g * G + l16;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = I8 ? 16 * (lg + 4 * (ks >> 1)) + 8 * (ks & 1) : 32 * ks + 8 * lg;
        qf[ct][ks] = cvalid[ct] ? ld16(qp + qrow * kD + d0) : make_uint4(0, 0, 0, 0);
      }
    }
  };

  f32x4_t o[CT][DT];
  float mref[CT], l[CT];  // column reference maximum (log2 units), lane partial sum
  auto reset = [&] {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[ct][dt] = f32x4_zero();
      mref[ct] = kNegInf;
      l[ct] = 0.f;
    }
  };
  // The piece of sequence c.b that this wave holds is complete.  A sequence
  // this group holds whole (its first and last columns in this run) is
  // normalised and stored here, and the combine skips its rows; a piece of a
  // split one is stored as piece (grp + b) H_kv + g (kStreamCols columns of a
  // piece in multi-token decode, G in decode).
  auto flush = [&](const Cursor& c) {
    const int64_t p0 = prefix_at(c.b);
    const bool whole = group_of_column(p0, C, NG) == group_of_column(p0 + c.n - 1, C, NG);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const float lsum = row4_sum(l[ct]);
      if (!cvalid[ct]) continue;
      if (whole) {
        int64_t orow;
        if constexpr (MT) {
          const int col = 16 * ct + l16;
          const int i = col / G;
          orow = (int64_t)(c.q0 + i) * H + (int64_t)g * G + (col - i * G);
        } else {
          orow = (int64_t)c.q0 * H + (int64_t)g * G + l16;
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const float v[4] = {o[ct][dt][0] * inv, o[ct][dt][1] * inv, o[ct][dt][2] * inv, o[ct][dt][3] * inv};
          store4(a.out, orow * kD + 16 * dt + 4 * lg, v, a.out_dtype);
        }
        continue;
      }
      const int64_t prow = MT ? ((grp + c.b) * Hkv + g) * kStreamCols + 16 * ct + l16 : ((grp + c.b) * Hkv + g) * G + l16;
      float* wo = a.ws_o + prow * kD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float v[4] = {o[ct][dt][0], o[ct][dt][1], o[ct][dt][2], o[ct][dt][3]};
        store4(wo, 16 * dt + 4 * lg, v, PKV_F32);
      }
      if (lg == 0) {
        a.ws_ml[prow * 2 + 0] = mref[ct];
        a.ws_ml[prow * 2 + 1] = lsum;
      }
    }
  };

  const float c2 = a.scale_log2e;
  // Compute the tile at cursor c from slot `sl`.
  auto compute_i8 = [&](const Cursor& c, int sl) {
    const int t0 = c.t_first + (c.k << kTileLog2);
    const unsigned char* kt = slots + sl * GT::kSlot;
    const unsigned char* vt = kt + GT::kTile;
    const float* sc = reinterpret_cast<const float*>(vt + GT::kTile);  // 32 K scales, then 32 V scales

    f32x4_t s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 kw = *reinterpret_cast<const uint4*>(kt + kr8_off[u][h]);
        s[u] = mfma_bf16(i8x8_to_bf16(make_uint2(kw.x, kw.y)), qf[0][2 * h], h == 0 ? f32x4_zero() : s[u]);
        s[u] = mfma_bf16(i8x8_to_bf16(make_uint2(kw.z, kw.w)), qf[0][2 * h + 1], s[u]);
      }
    }
    // Lane (n, lg) holds keys 8 lg + 4 u + e of tile u.
    float4 ksc[2], vsc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      ksc[u] = *reinterpret_cast<const float4*>(sc + 8 * lg + 4 * u);
      vsc[u] = *reinterpret_cast<const float4*>(sc + kKeyTile + 8 * lg + 4 * u);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s[u][0] *= ksc[u].x;
      s[u][1] *= ksc[u].y;
      s[u][2] *= ksc[u].z;
      s[u][3] *= ksc[u].w;
    }
    if (!(t0 >= c.lo && t0 + kKeyTile <= c.L)) {
      // Keys outside [lo, L): logit -inf and V scale 0 (their scales may be any
      // bits, a NaN included: selected away, never multiplied).
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float* vs = reinterpret_cast<float*>(&vsc[u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = t0 + 8 * lg + 4 * u + e;
          const bool ok = j >= c.lo && j < c.L;
          s[u][e] = ok ? s[u][e] : kNegInf;
          vs[e] = ok ? vs[e] : 0.f;
        }
      }
    }
    // Probabilities against the current reference first; the column maximum is
    // formed only when some lane's sum of them says it may be needed (see compute).
    float pv[8];
    float ls;
    auto probs = [&](float mb) {
      ls = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float* vs = reinterpret_cast<const float*>(&vsc[u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = exp2_fast(fmaf(s[u][e], c2, -mb));
          ls += p;
          pv[4 * u + e] = p * vs[e];
        }
      }
    };
    probs(mref[0] == kNegInf ? 0.f : mref[0]);
    if (__any(mref[0] == kNegInf || !(ls <= kRaiseSum))) {
      float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      mt = row4_max(mt);
      const float mts = mt * c2;
      const bool raise = mts > mref[0] + kRescaleLog2;
      if (__any(raise)) {
        const float alpha = raise ? exp2_fast(mref[0] - mts) : 1.f;
        if (raise) mref[0] = mts;
        l[0] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[0][dt] *= alpha;
      }
      probs(mref[0] == kNegInf ? 0.f : mref[0]);
    }
    l[0] += ls;
    uint4 phi, plo;
    pack_p_split(pv, phi, plo);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint4 af = i8x8_to_bf16(lds_tr8(vt + vr8_off[dt]));
      o[0][dt] = mfma_bf16(af, phi, o[0][dt]);
      o[0][dt] = mfma_bf16(af, plo, o[0][dt]);
    }
  };

  auto compute = [&](const Cursor& c, int sl) {
    const int t0 = c.t_first + (c.k << kTileLog2);
    const unsigned char* kt = slots + sl * GT::kSlot;
    const unsigned char* vt = kt + GT::kTile;

    f32x4_t s[CT][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 af = *reinterpret_cast<const uint4*>(kt + kr_off[ks] + u * 16 * kRowBytes);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) s[ct][u] = mfma_bf16(af, qf[ct][ks], ks == 0 ? f32x4_zero() : s[ct][u]);
      }
    }
    if constexpr (MT) {
      // Column (row at cpos) sees keys (cpos - W, cpos]; a tile every column sees
      // whole lies at or after the last row's window start and at or before the
      // first row's position.
      const int lo_all = a.window > 0 ? max(0, c.L - a.window) : 0;
      if (!(t0 >= lo_all && t0 + kKeyTile - 1 <= c.L - c.nq)) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = t0 + 16 * u + 4 * lg + e;
              const bool vis = j <= cpos[ct] && (a.window == 0 || j > cpos[ct] - a.window);
              s[ct][u][e] = vis ? s[ct][u][e] : kNegInf;
            }
      }
    } else {
      if (!(t0 >= c.lo && t0 + kKeyTile <= c.L)) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = t0 + 16 * u + 4 * lg + e;
            s[0][u][e] = (j >= c.lo && j < c.L) ? s[0][u][e] : kNegInf;
          }
      }
    }
    uint4 phi[CT], plo[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      // Probabilities against the current reference and this lane's sum of them.
      // No lane's sum above 2^8 means no probability above 2^8 (no logit past the
      // reference by more than the rescale threshold), so the column maximum --
      // a max chain and the cross-row exchange -- is formed only when some sum
      // says it may be needed (the first visible tile, a new peak); the
      // probabilities are then taken again against the raised reference.
      float p8[8];
      float ls;
      auto probs = [&](float mb) {
        ls = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = exp2_fast(fmaf(s[ct][u][e], c2, -mb));
            p8[4 * u + e] = p;
            ls += p;
          }
      };
      probs(mref[ct] == kNegInf ? 0.f : mref[ct]);
      if (__any(mref[ct] == kNegInf || !(ls <= kRaiseSum))) {  // !(<=): a NaN or inf sum too
        float mt = fmaxf(fmaxf(fmaxf(s[ct][0][0], s[ct][0][1]), fmaxf(s[ct][0][2], s[ct][0][3])),
                         fmaxf(fmaxf(s[ct][1][0], s[ct][1][1]), fmaxf(s[ct][1][2], s[ct][1][3])));
        mt = row4_max(mt);
        const float mts = mt * c2;
        const bool raise = mts > mref[ct] + kRescaleLog2;
        if (__any(raise)) {
          const float alpha = raise ? exp2_fast(mref[ct] - mts) : 1.f;  // mref = -inf gives 0
          if (raise) mref[ct] = mts;
          l[ct] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[ct][dt] *= alpha;
        }
        probs(mref[ct] == kNegInf ? 0.f : mref[ct]);  // no finite logit yet: every p is 0
      }
      l[ct] += ls;
      pack_p_split(p8, phi[ct], plo[ct]);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint2 x0 = lds_tr16(reinterpret_cast<const uint16_t*>(vt + vr_off[dt]));
      const uint2 x1 = lds_tr16(reinterpret_cast<const uint16_t*>(vt + vr_off[dt] + 16 * kRowBytes));
      const uint4 af = make_uint4(x0.x, x0.y, x1.x, x1.y);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        o[ct][dt] = mfma_bf16(af, phi[ct], o[ct][dt]);
        o[ct][dt] = mfma_bf16(af, plo[ct], o[ct][dt]);
      }
    }
  };

  // Columns c_beg .. c_end-1 in order: cc is the tile being computed, pc the
  // one streaming in.  A sequence change stores the finished piece and loads
  // the next q (its wait also drains the tile in flight: rarely more than once
  // or twice per wave).
  const int64_t ntl = c_end - c_beg;
  Cursor cc = c0, pc = c0;
  load_q(cc);
  reset();
  retire_loads();  // q is in before the first DMA: only tile copies are in flight below
  issue_tile(pc, 0);
  for (int64_t i = 0; i < ntl; ++i) {
    const int sl = (int)(i & 1);
    if (i + 1 < ntl) {
      advance(pc);
      issue_tile(pc, sl ^ 1);
      wait_vm<GT::kDma>();  // tile i has landed; tile i + 1's copies stay in flight
    } else {
      wait_vm<0>();
    }
    if constexpr (I8) compute_i8(cc, sl);
    else compute(cc, sl);
    if (i + 1 < ntl) {
      const Cursor prev = cc;
      advance(cc);
      if (cc.k == 0) {  // a sequence ends here: store its piece, start the next one
        flush(prev);
        reset();
        load_q(cc);
        retire_loads();  // the compiler then knows q is in: no wait for it inside the loop
      }
    }
  }
  flush(cc);
}

// One wave per output row (query row t of sequence b, query head h): merge the
// pieces of (b, h / G): M = max m_p, L = sum l_p 2^(m_p - M), out = sum o_p
// 2^(m_p - M) / L.  Lanes read the (m, l) of up to 64 pieces at once; a
// sequence with no visible key gets a zero row.  Decode: t = b and the piece
// column is h % G; multi-token decode (MT): b holds row t (cu_seqlens_q) and the
// column is (t - cu[b]) G + h % G.
template <bool MT>
__global__ __launch_bounds__(kWaves * kWave) void stream_combine_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int H = a.num_q_heads;
  if (row >= (int64_t)(MT ? a.total_q : a.batch) * H) return;
  const int t = (int)(row / H);
  const int h = (int)(row % H);
  const int Hkv = a.num_kv_heads;
  const int G = H / Hkv;
  const int g = h / G;
  int b = t, c = h % G;
  if constexpr (MT) {
    // b = the last sequence with cu[b] <= t, found 64 samples at a time: the
    // lanes read 64 evenly spaced entries of [lo, hi] at once and the range
    // shrinks to the gap between the last sample <= t and the first one past it
    // (a range of at most 64 entries is sampled whole, so one round trip ends it).
    const int32_t* cu = a.cu_seqlens_q;
    int lo = 0, hi = a.batch - 1;
    while (hi > lo) {
      const int64_t span = hi - lo + 1;
      const bool le = cu[lo + (int)(span * lane / kWave)] <= t;
      const uint64_t m = __ballot(le);  // a prefix of the lanes: cu never decreases
      const int k_last = 63 - __builtin_clzll(m);  // lane 0 samples lo, where cu[lo] <= t
      const int64_t next = ~m ? lo + span * __builtin_ctzll(~m) / kWave : hi + 1;
      lo = lo + (int)(span * k_last / kWave);
      hi = (int)next - 1;
    }
    b = lo;
    c += (t - cu[b]) * G;
  }
  const int64_t cols = MT ? kStreamCols : G;  // columns of a piece
  const int32_t* prefix = a.tile_prefix;
  const int32_t p0 = prefix[b];
  const int32_t n = prefix[b + 1] - p0;
  float O0 = 0.f, O1 = 0.f, inv = 0.f;
  if (n > 0) {
    const int64_t C = prefix[a.batch];
    const int64_t NG = stream_groups(C, a.resident_waves, Hkv, a.split_tiles);
    const int64_t xA = group_of_column(p0, C, NG), xB = group_of_column(p0 + n - 1, C, NG);
    if (xA == xB) return;  // one group held the sequence whole and stored its rows
    // Groups in [xA, xB] with an empty run (fewer columns than groups) store
    // nothing; every other one holds a piece of sequence b.
    auto piece_row = [&](int64_t x) { return ((x + b) * Hkv + g) * cols + c; };
    float M = kNegInf, Ls = 0.f;
    for (int64_t x0 = xA; x0 <= xB; x0 += kWave) {  // pass 1: the maximum
      const int64_t x = x0 + lane;
      if (x <= xB && C * x / NG != C * (x + 1) / NG) M = fmaxf(M, a.ws_ml[piece_row(x) * 2]);
    }
    M = group_max<kWave>(M);
    for (int64_t x0 = xA; x0 <= xB; x0 += kWave) {  // pass 2: weights, sum and O
      const int64_t x = x0 + lane;
      float f = 0.f;
      if (x <= xB && C * x / NG != C * (x + 1) / NG) {
        const int64_t pr = piece_row(x);
        f = rescale(a.ws_ml[pr * 2], M);
        Ls += a.ws_ml[pr * 2 + 1] * f;
      }
      // Eight pieces' loads in flight at a time: the loads are unconditional
      // (clamped to the last piece of the chunk, all inside the workspace) and a
      // zero weight -- an empty run whose slot holds stale data, or a piece
      // that cannot contribute -- selects nothing rather than multiplying.
      const int cnt = (int)min<int64_t>(kWave, xB - x0 + 1);
      for (int i0 = 0; i0 < cnt; i0 += 8) {
        float2 v[8];
        float w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = min(i0 + k, cnt - 1);
          w[k] = i0 + k < cnt ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(f), i)) : 0.f;
          v[k] = *reinterpret_cast<const float2*>(a.ws_o + piece_row(x0 + i) * kD + 2 * lane);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          O0 = w[k] != 0.f ? fmaf(v[k].x, w[k], O0) : O0;
          O1 = w[k] != 0.f ? fmaf(v[k].y, w[k], O1) : O1;
        }
      }
    }
    Ls = group_sum<kWave>(Ls);
    inv = Ls > 0.f ? 1.f / Ls : 0.f;
  }
  const int64_t oi = row * kD + 2 * lane;
  if (a.out_dtype == PKV_BF16) {
    const uint32_t wd = (uint32_t)f32_to_bf16(O0 * inv) | ((uint32_t)f32_to_bf16(O1 * inv) << 16);
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + oi) = wd;
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(a.out) + oi) = make_float2(O0 * inv, O1 * inv);
  }
}

}  // namespace

bool decode_mfma_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  return (dtype == PKV_BF16 || dtype == PKV_INT8) && head_dim == kD && group >= 1 && group <= 16;
}

int32_t decode_stream_resident_waves(int32_t cu_count, int32_t dtype) {
  return cu_count * (dtype == PKV_INT8 ? kWavesI8 : kWaves);
}

size_t decode_stream_workspace(int32_t batch, int32_t columns, int32_t num_kv_heads, int32_t resident_waves,
                               size_t* ws_o_offset, size_t* ws_ml_offset) {
  const size_t group = (size_t)columns;
  const size_t pieces = (size_t)resident_waves + (size_t)batch * num_kv_heads;
  const size_t prefix_bytes = (((size_t)batch + 1) * sizeof(int32_t) + 255) & ~size_t(255);
  const size_t o_bytes = (pieces * group * kD * sizeof(float) + 255) & ~size_t(255);
  *ws_o_offset = prefix_bytes;
  *ws_ml_offset = prefix_bytes + o_bytes;
  return prefix_bytes + o_bytes + pieces * group * 2 * sizeof(float);
}

hipError_t launch_decode_stream(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  const bool lds_prefix = (int64_t)a.batch + 1 <= kLdsPrefix;
  const bool mt = a.cu_seqlens_q != nullptr;
  if (mt && a.dtype != PKV_BF16) return hipErrorInvalidValue;
  if (!lds_prefix) {
    tile_prefix_kernel<<<1, 1024, 0, stream>>>(a.seq_lens, a.cu_seqlens_q, a.batch, a.window, a.tile_prefix);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool one_block = a.block_size_log2 >= kTileLog2;
  if (a.dtype == PKV_INT8) {
    const unsigned grid = (unsigned)(a.resident_waves / kWavesI8);
    const dim3 blk(kWavesI8 * kWave);
    if (lds_prefix && one_block) decode_stream_kernel<true, true, true, false><<<grid, blk, 0, stream>>>(a);
    else if (lds_prefix) decode_stream_kernel<false, true, true, false><<<grid, blk, 0, stream>>>(a);
    else if (one_block) decode_stream_kernel<true, false, true, false><<<grid, blk, 0, stream>>>(a);
    else decode_stream_kernel<false, false, true, false><<<grid, blk, 0, stream>>>(a);
  } else if (mt) {
    const unsigned grid = (unsigned)(a.resident_waves / kWaves);
    const dim3 blk(kWaves * kWave);
    if (lds_prefix && one_block) decode_stream_kernel<true, true, false, true><<<grid, blk, 0, stream>>>(a);
    else if (lds_prefix) decode_stream_kernel<false, true, false, true><<<grid, blk, 0, stream>>>(a);
    else if (one_block) decode_stream_kernel<true, false, false, true><<<grid, blk, 0, stream>>>(a);
    else decode_stream_kernel<false, false, false, true><<<grid, blk, 0, stream>>>(a);
  } else {
    const unsigned grid = (unsigned)(a.resident_waves / kWaves);
    const dim3 blk(kWaves * kWave);
    if (lds_prefix && one_block) decode_stream_kernel<true, true, false, false><<<grid, blk, 0, stream>>>(a);
    else if (lds_prefix) decode_stream_kernel<false, true, false, false><<<grid, blk, 0, stream>>>(a);
    else if (one_block) decode_stream_kernel<true, false, false, false><<<grid, blk, 0, stream>>>(a);
    else decode_stream_kernel<false, false, false, false><<<grid, blk, 0, stream>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)(mt ? a.total_q : a.batch) * a.num_q_heads;
  const unsigned cgrid = (unsigned)((rows + kWaves - 1) / kWaves);
  if (mt) stream_combine_kernel<true><<<cgrid, kWaves * kWave, 0, stream>>>(a);
  else stream_combine_kernel<false><<<cgrid, kWaves * kWave, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
