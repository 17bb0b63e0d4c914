// Fused Markov-bias product: matrix-core product of W1 rows with W2 -> add U_k
// and scale by 1/T -> per-(row, vocabulary tile) reduction.
//
// The Markov head (Blog, "Markov sequential head"; KB section 2) adds the bias
// row W1[x_{k-1}, :] W2 to the backbone logits U_k.  For a batch of rows this is
// an [M, r] x [r, V] product whose only consumer is a vocabulary-wide
// reduction, so z never goes to HBM: per row and 128-column vocabulary tile the
// kernel emits one partial.
//
//   Draft epilogue  (m_t, s_t) = (max_v z, sum_v exp(z - m_t)) of the tile
//   Verify epilogue (sum_v min(p, q), sum_v (p - q)_+) of the tile, with
//                   q = exp(z - m_q)/S_q from the draft's statistics and
//                   p = exp(t/T - m_p)/S_p from the target row statistics
#pragma once
#include <type_traits>

#include "common.h"

namespace dspark {

constexpr int kChunks = 4;            // target-row statistics are kept per quarter row

// Combined statistics of one target row from its kChunks partials, in chunk
// order.  Every consumer calls this, so all see the same (m_p, S_p).
__device__ __forceinline__ float2 combine_chunk_stats(const float2 *cs) {
  float m = cs[0].x;
#pragma unroll
  for (int c = 1; c < kChunks; ++c) m = fmaxf(m, cs[c].x);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) s += cs[c].y * (cs[c].x == -INFINITY ? 0.0f : fexp(cs[c].x - m));
  return make_float2(m, s);
}

struct BiasTileParams {
  int R, gamma, V, r, n_tiles;
  float invT;
  const void *U;        // [R][gamma][V]
  const void *W1;       // [V][r]
  const void *W2;       // column-major r x V
  const int32_t *x0;    // [R]
  const int32_t *x;     // [R][gamma]
  int32_t *err;
  // draft: rows are requests at position k
  int k;
  float2 *tile_stats;   // [R][n_tiles]
  // verify: rows are the compacted verified drafts
  const int32_t *ell, *row_offset;
  int rows_capacity;
  const void *P;            // [rows_capacity][V]
  const float2 *p_chunks;   // [rows_capacity][kChunks]
  const float *q_stats;     // [R][gamma][2]
  float2 *pair_partials;    // [R*gamma][n_tiles] (sum min, sum residual)
  const int4 *row_map;      // [R*gamma] (rho, k, x_{k-1}, target row) of compact row i
  // transition rows W1[x_{k-1}] of the product's rows, contiguous: [R][r]
  // (draft, row = request) or [R*gamma][r] (verify, row = compact row);
  // or, where a_tokens is set (draft), row i is W1[a_tokens[i]] read in place
  const void *A;
  const int32_t *a_tokens;
};

enum class Epi { kDraft, kVerify };

// ------------------------------------------------------------------------
// Row-stationary streaming tile kernel.
//
// A workgroup of NW waves takes a row group of product rows (each wave RB
// blocks of 32 rows) and a contiguous range of vocabulary tiles.  Each wave
// keeps the A operand of its rows (all of K) in registers for the whole range;
// W2 streams through in blocks of 32 columns: loaded into registers ahead of
// use, written to one half of a double-buffered LDS stage (a padded column
// pitch keeps the operand reads free of bank conflicts), and read by all
// waves.  U (and P) row segments stream into a register ring two blocks
// ahead.  The epilogue works on 16 consecutive columns of one row per lane:
// the draft step puts W2 first in the product (columns in the order
// block_col_of_m), so each lane's accumulator already holds them; the verify
// pass puts the rows first and transposes its accumulator through the wave's
// own LDS scratch (its longer epilogue ran faster that way).  U is added, the
// block is folded into running per-row sums, and the partials of finished
// tiles are buffered in LDS and written every kFlushTiles tiles.
//
// The loop body covers one tile (4 blocks) with a fixed instruction sequence
// (loads past the range are clamped), so the waits the compiler inserts count
// only the loads they need.
constexpr int kRowsPerWave = 32;                        // product rows of one wave
constexpr int kBlockCols = 32;                          // W2 columns per block
constexpr int kBlocksPerTile = kTileN / kBlockCols;     // 4
constexpr int kColPieces = kMaxRank * 2 / 16;           // 16-byte pieces per W2 column (max)
constexpr int kColPitch = kColPieces + 1;               // pieces per LDS column: one of padding
constexpr int kStageBytes = kBlockCols * kColPitch * 16;  // one W2 block in LDS: 16.5 KB
constexpr int kScratchPitch = 36;                       // floats per scratch row (rows first)
constexpr int kFlushTiles = 8;                          // tile partials kept in LDS

// the A operand of one wave's 32 rows, all K
template <typename T> struct AFrag;
template <> struct AFrag<bf16_t> {
  static constexpr int kSteps = kMaxRank / 16;
  u16x8 v[kSteps];
};
template <> struct AFrag<float> {
  static constexpr int kSteps = 64;
  float v[kSteps];
};

// Rows past the last real row read a clamped real row (finite values whose
// outputs are discarded).
__device__ __forceinline__ void load_afrag(const bf16_t *Arow, int r, AFrag<bf16_t> &a,
                                           int ks_static) {
  const int lane = threadIdx.x & (kWave - 1);
  const bf16_t *ptr = Arow + (lane >> 5) * 8;
  const u16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < AFrag<bf16_t>::kSteps; ++ks) {
    const bool in = ks_static > 0 ? ks < ks_static : ks * 16 < r;
    const int kk = in ? ks * 16 : 0;
    const u16x8 t = *reinterpret_cast<const u16x8 *>(ptr + kk);
    a.v[ks] = in ? t : zero;
  }
}
__device__ __forceinline__ void load_afrag(const float *Arow, int r, AFrag<float> &a,
                                           int ks_static) {
  const int lane = threadIdx.x & (kWave - 1);
  const float *ptr = Arow + (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < AFrag<float>::kSteps; ++ks) {
    const bool in = ks_static > 0 ? ks < ks_static : ks * 2 < r;
    const float t = ptr[in ? ks * 2 : 0];
    a.v[ks] = in ? t : 0.0f;
  }
}

// 16-byte piece pc of the W2 column in LDS slot m of a block.  Lane l reads
// slot l % 32 for its operand: with W2 first a block is stored in matrix-row
// order (column c in slot block_m_of_col(c)), rows first in column order.  The
// pitch of kColPitch (odd) pieces puts the same piece of 16 consecutive slots
// in 16 different bank groups, and keeps every offset within a column affine.
__device__ __forceinline__ int w2_slot(int m, int pc) { return m * kColPitch + pc; }
template <bool kW2First> __device__ __forceinline__ int w2_slot_of_col(int c) {
  return kW2First ? block_m_of_col(c) : c;
}

template <bool kW2First>
__device__ __forceinline__ floatx16 mfma16(const u16x8 &w2, const u16x8 &rows, const floatx16 &c) {
  if constexpr (kW2First)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w2),
                                                   __builtin_bit_cast(bf16x8, rows), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, rows),
                                                   __builtin_bit_cast(bf16x8, w2), c, 0, 0, 0);
}

// Product of one W2 block from LDS with one wave's 32 rows (A operand in
// registers).  K advances in increasing order from a zero accumulator with the
// same instruction and operand order as mma_rows<kW2First>: the same element
// comes out of the same instruction sequence.  With W2 first (the draft step)
// every W2 read of the block is issued before the products: interleaved two
// at a time, the LDS latency was exposed between pairs.  Rows first (the
// verify pass, eight waves per workgroup) keeps each read next to its product,
// which measured faster there.
template <int KS, bool kW2First>
__device__ __forceinline__ void mma_block(const AFrag<bf16_t> &a, const unsigned char *stage,
                                          int r, floatx16 &acc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int m = lane & 31;  // LDS slot of this lane's W2 column
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  if constexpr (KS > 0 && kW2First) {
    u16x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      b[ks] = *reinterpret_cast<const u16x8 *>(stage + 16 * w2_slot(m, 2 * ks + (lane >> 5)));
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma16<kW2First>(b[ks], a.v[ks], acc);
  } else {
#pragma unroll
    for (int ks = 0; ks < (KS > 0 ? KS : AFrag<bf16_t>::kSteps); ++ks) {
      if (KS > 0 || ks * 16 < r) {
        const u16x8 b = *reinterpret_cast<const u16x8 *>(
            stage + 16 * w2_slot(m, 2 * ks + (lane >> 5)));
        acc = mfma16<kW2First>(b, a.v[ks], acc);
      }
    }
  }
}
template <int KS, bool kW2First>
__device__ __forceinline__ void mma_block(const AFrag<float> &a, const unsigned char *stage,
                                          int r, floatx16 &acc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int m = lane & 31;  // LDS slot of this lane's W2 column
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < (KS > 0 ? KS : AFrag<float>::kSteps); ++ks) {
    if (KS > 0 || ks * 2 < r) {
      const int k = 2 * ks + (lane >> 5);
      const float b = *reinterpret_cast<const float *>(stage + 16 * w2_slot(m, 0) + 4 * k);
      if constexpr (kW2First)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a.v[ks], acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[ks], b, acc, 0, 0, 0);
    }
  }
}

// exchange with the neighbouring lane (l ^ 1)
__device__ __forceinline__ float pair_swap(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
// exchange with the lane holding the other half of the row (l ^ 32)
__device__ __forceinline__ float half_swap(float x) {
  const int lane = threadIdx.x & (kWave - 1);
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(x)));
}

// log2 of a probability exp(x / T - m) / S from a logit x before the
// temperature and the row's (m, S): x / T - m in one rounding (so an entry
// near the maximum keeps full relative precision), then scaled to base 2.
// The verify pass and the residual draw form every per-entry quantity with
// this function, so they agree element by element.
__device__ __forceinline__ float log2_prob(float x, float invT, float m, float log2S) {
  return fmaf(fmaf(x, invT, -m), kLog2e, -log2S);
}

// NW waves per workgroup, each with RB blocks of 32 product rows: a row group
// of 32 NW RB rows shares every W2 block it loads.  One workgroup per compute
// unit (a wave may use up to 512 registers).
template <typename T, Epi E, int KS, int NW, int RB>
__global__ __launch_bounds__(NW * kWave, 1) void stream_tile_kernel(BiasTileParams p) {
  constexpr bool kVerify = E == Epi::kVerify;
  constexpr bool kW2First = !kVerify;  // operand order of the product
  constexpr int kThreads = NW * kWave;
  constexpr int kRowGroup = NW * RB * kRowsPerWave;
  constexpr int kPer = 16 / (int)sizeof(T);   // elements per 16-byte piece
  constexpr int kSegV = 16 / kPer;            // pieces per 16-column row segment
  constexpr int kTpc = kThreads / kBlockCols;  // threads per W2 column of a block
  constexpr int kWPieces = kColPieces / kTpc;  // W2 pieces per thread per block
  __shared__ __align__(16) unsigned char w2s[2][kStageBytes];
  __shared__ __align__(16) float scratch[kW2First ? 1 : NW][kW2First ? 1 : 32 * kScratchPitch];
  __shared__ float2 pbuf[kRowGroup][kFlushTiles];  // partials of the last tiles, by row
  __shared__ int pout[kRowGroup];                  // output row of each row, -1 for none

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int V = p.V, n_tiles = p.n_tiles;
  const int r = KS > 0 ? KS * (sizeof(T) == 2 ? 16 : 2) : p.r;
  const int npieces = r * (int)sizeof(T) / 16;  // W2 pieces per column, <= 32
  const float invT = p.invT, cl = invT * kLog2e;

  int n_rows = p.R;
  if constexpr (kVerify) {
    n_rows = p.row_offset[p.R] - p.R;  // sum of ell
    if (n_rows > p.R * p.gamma) n_rows = p.R * p.gamma;
  }
  if (n_rows <= 0) return;
  const int n_rg = (n_rows + kRowGroup - 1) / kRowGroup;
  // Work: (row group, vocabulary tile) items; one workgroup per compute unit.
  int t0, t1;
  if (kVerify && n_rg > 1 && n_rg <= (int)gridDim.x / kXcds && gridDim.x % kXcds == 0) {
    // Workgroups are dealt to the XCDs in turn (workgroup b on XCD b % 8), and
    // each XCD has its own L2.  Groups of n_rg workgroups on one XCD take the
    // same tile range, one row group each, so each W2 block comes from HBM
    // about once per group rather than once per row group (fetched bytes
    // 639 -> 539 MB on a long-block round); workgroups left over on an XCD
    // stay idle.
    const int per_xcd = (int)gridDim.x / kXcds;
    const int x = (int)blockIdx.x % kXcds, li = (int)blockIdx.x / kXcds;
    const int groups = per_xcd / n_rg;
    const int g = li / n_rg, rg = li - g * n_rg;
    if (g >= groups) {
      t0 = t1 = 0;
    } else {
      const int nr = kXcds * groups, ri = g * kXcds + x;  // tile range of the group
      t0 = rg * n_tiles + (int)((int64_t)ri * n_tiles / nr);
      t1 = rg * n_tiles + (int)((int64_t)(ri + 1) * n_tiles / nr);
    }
  } else {
    // equal contiguous ranges, row-group major
    const int total = n_rg * n_tiles;
    const int per = (total + (int)gridDim.x - 1) / (int)gridDim.x;
    t0 = (int)blockIdx.x * per;
    t1 = min(total, t0 + per);
  }

  const T *Ab = reinterpret_cast<const T *>(p.A);
  const T *W2 = reinterpret_cast<const T *>(p.W2);
  const T *U = reinterpret_cast<const T *>(p.U);
  const T *P = reinterpret_cast<const T *>(p.P);
  float *ws = scratch[kW2First ? 0 : wave];
  // epilogue row within a 32-row block, its first column within the block, and
  // whether this lane is the first of the two that hold the row
  const int erow_w = kW2First ? lane & 31 : lane >> 1;
  const int ec0 = kW2First ? (lane >> 5) * 16 : (lane & 1) * 16;
  const bool row_lead = kW2First ? (lane >> 5) == 0 : (lane & 1) == 0;
  bool bad_entry = false;

  // per row block of this wave: block b = rb * NW + wave of the row group
  struct RowState {
    bool live, wave_live;
    int slot;                  // row of the group, for pbuf and pout
    const T *Urow, *Prow;
    float mq, lq, mp, lp;      // (m, log2 S) of q and p (verify)
    float run_m, run_s;        // draft: max of acc + u, sum of exp over the tile
    float run_min, run_res;    // verify: sum min(p, q), sum (p - q)_+
  };

  while (t0 < t1) {
    __syncthreads();  // the previous range's flush is done with pbuf and pout
    const int rg = t0 / n_tiles, tile0 = t0 - rg * n_tiles;
    const int ntile = min(n_tiles - tile0, t1 - t0);
    t0 += ntile;
    const int nblk = ntile * kBlocksPerTile;
    const int cb0 = tile0 * kBlocksPerTile;  // first column block

    AFrag<T> af[RB];
    RowState rs[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rbase = rg * kRowGroup + (rb * NW + wave) * kRowsPerWave;
      // the A rows (product row = lane % 32 of the block)
      const int arow = min(rbase + (lane & 31), n_rows - 1);
      const T *aptr = Ab + (int64_t)arow * r;
      if (p.a_tokens != nullptr) {
        int tok = p.a_tokens[arow];
        if (tok < 0 || tok >= V) {
          flag_error(p.err, kErrToken);
          tok = tok < 0 ? 0 : V - 1;
        }
        aptr = reinterpret_cast<const T *>(p.W1) + (int64_t)tok * r;
      }
      load_afrag(aptr, r, af[rb], KS);
      // this lane's epilogue row: source rows and statistics
      RowState &s = rs[rb];
      const int erow = rbase + erow_w;
      s.slot = (rb * NW + wave) * kRowsPerWave + erow_w;
      s.live = erow < n_rows;
      s.wave_live = rbase < n_rows;  // uniform per wave
      int rho = 0, k = 1, prow = 0;
      if constexpr (kVerify) {
        const int4 e = p.row_map[s.live ? erow : 0];  // written by the target-row statistics pass
        const bool bad = e.x < 0 || e.x >= p.R || e.y < 1 || e.y > p.gamma || e.w < 0 ||
                         e.w >= p.rows_capacity;
        bad_entry |= s.live && bad;
        s.live = s.live && !bad;
        if (s.live) { rho = e.x; k = e.y; prow = e.w; }
      } else {
        if (s.live) { rho = erow; k = p.k; }
      }
      if (row_lead) pout[s.slot] = s.live ? erow : -1;
      s.Urow = U + ((int64_t)rho * p.gamma + (k - 1)) * V;
      s.Prow = P + (int64_t)prow * V;
      s.mq = s.lq = s.mp = s.lp = 0.0f;
      if constexpr (kVerify) {
        const int64_t qi = (int64_t)rho * p.gamma + k - 1;
        s.mq = p.q_stats[2 * qi];
        s.lq = log2_fast(p.q_stats[2 * qi + 1]);
        const float2 ps = combine_chunk_stats(p.p_chunks + (int64_t)prow * kChunks);
        s.mp = ps.x;
        s.lp = log2_fast(ps.y);
      }
      s.run_m = -INFINITY;
      s.run_s = s.run_min = s.run_res = 0.0f;
    }

    // ---- loads of block j (clamped past the range)
    // native vectors, so that the stages stay in registers
    struct WRegs { u32x4 w[kWPieces]; };
    struct URegs { u32x4 u[RB][kSegV]; u32x4 t[RB][kVerify ? kSegV : 1]; };
    // W2 pieces of a block: thread t takes column t / kTpc and pieces
    // (t % kTpc) + kTpc i (pieces past the column's npieces repeat its last)
    const int wc = tid / kTpc, wp = tid % kTpc;
    auto load_w = [&](WRegs &wr, int j) __attribute__((always_inline)) {
      const int col = min((cb0 + min(j, nblk - 1)) * kBlockCols + wc, V - 1);
      const T *src = W2 + (int64_t)col * r;
#pragma unroll
      for (int i = 0; i < kWPieces; ++i)
        wr.w[i] = *reinterpret_cast<const u32x4 *>(src + min(wp + kTpc * i, npieces - 1) * kPer);
    };
    auto store_w = [&](int stage, const WRegs &wr) __attribute__((always_inline)) {
      unsigned char *dst = w2s[stage] + 16 * w2_slot(w2_slot_of_col<kW2First>(wc), wp);
#pragma unroll
      for (int i = 0; i < kWPieces; ++i)
        if (KS > 0 ? kTpc * i < npieces : wp + kTpc * i < npieces)
          *reinterpret_cast<u32x4 *>(dst + 16 * kTpc * i) = wr.w[i];
    };
    auto load_u = [&](URegs &ur, int j) __attribute__((always_inline)) {
      const int cb = cb0 + min(j, nblk - 1);
      // a 16-byte piece is all in or all out of [0, V) (V % 8 == 0).  Plain
      // loads: a 128-byte line serves two consecutive blocks of a row, so it
      // must stay in L2 until the next block's load.
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < kSegV; ++i) {
          const int col = min(cb * kBlockCols + ec0 + i * kPer, V - kPer);
          ur.u[rb][i] = *reinterpret_cast<const u32x4 *>(rs[rb].Urow + col);
          if constexpr (kVerify) ur.t[rb][i] = *reinterpret_cast<const u32x4 *>(rs[rb].Prow + col);
        }
    };

    // ---- epilogue of block j for row block rb: (rows first: transpose the
    //      product through the wave's scratch), add U, fold into the running
    //      sums
    auto epilogue = [&](int j, int rb, const floatx16 &acc, const URegs &ur,
                        auto mask_tag) __attribute__((always_inline)) {
      constexpr bool kMask = decltype(mask_tag)::value;
      RowState &s = rs[rb];
      if constexpr (!kW2First) {
        wave_sync();  // the previous block's reads of the scratch are done
#pragma unroll
        for (int e = 0; e < 16; ++e)
          ws[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * kScratchPitch + (lane & 31)] = acc[e];
        wave_sync();  // the other lanes' accumulators are in the scratch
      }
      const float *srow = ws + erow_w * kScratchPitch + ec0;
      // product values of columns c..c+3 of this lane's row
      auto prod4 = [&](int c) __attribute__((always_inline)) {
        if constexpr (kW2First) {
          floatx4 c4;
          c4[0] = acc[c]; c4[1] = acc[c + 1]; c4[2] = acc[c + 2]; c4[3] = acc[c + 3];
          return c4;
        } else {
          return *reinterpret_cast<const floatx4 *>(srow + c);
        }
      };
      const int col0 = (cb0 + j) * kBlockCols + ec0;
      if constexpr (!kVerify) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const floatx4 c4 = prod4(4 * q);
          v[4 * q] = c4[0]; v[4 * q + 1] = c4[1]; v[4 * q + 2] = c4[2]; v[4 * q + 3] = c4[3];
        }
#pragma unroll
        for (int i = 0; i < kSegV; ++i) {
          float u[kPer];
          unpack16(ur.u[rb][i], (T *)nullptr, u);
#pragma unroll
          for (int q = 0; q < kPer; ++q) v[i * kPer + q] += u[q];  // v = acc + u
        }
        float bm = -INFINITY;
#pragma unroll
        for (int c = 0; c < 16; ++c) bm = fmaxf(bm, (kMask && col0 + c >= V) ? -INFINITY : v[c]);
        const float mn = fmaxf(s.run_m, bm);
        if (!kMask || mn != -INFINITY) {
          // exp(z - z_max) = 2^((v - v_max) log2(e) / T): v - v_max keeps the
          // precision of the terms near the maximum
          float sb = 0.0f;
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const float e = exp2_fast((v[c] - mn) * cl);
            sb += (kMask && col0 + c >= V) ? 0.0f : e;
          }
          s.run_s = fmaf(s.run_s, exp2_fast((s.run_m - mn) * cl), sb);
          s.run_m = mn;
        }
      } else {
        // one 16-byte piece (kPer columns) of U and P at a time
#pragma unroll
        for (int i = 0; i < kSegV; ++i) {
          float u[kPer], t[kPer];
          unpack16(ur.u[rb][i], (T *)nullptr, u);
          unpack16(ur.t[rb][i], (T *)nullptr, t);
#pragma unroll
          for (int q4 = 0; q4 < kPer; q4 += 4) {
            const floatx4 c4 = prod4(i * kPer + q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int q = q4 + e, c = i * kPer + q;
              const float a = log2_prob(t[q], invT, s.mp, s.lp);          // log2 p
              const float b = log2_prob(c4[e] + u[q], invT, s.mq, s.lq);  // log2 q, v = acc + u
              const float mn = exp2_fast(fminf(a, b));
              const float pe = exp2_fast(a);
              const bool in = !kMask || col0 + c < V;
              s.run_min += in ? mn : 0.0f;
              s.run_res += in ? pe - mn : 0.0f;
            }
          }
        }
      }
    };
    // ---- end of a tile: combine the two lanes of each row into the LDS
    //      partial buffer, reset; every kFlushTiles tiles the buffer goes out
    auto tile_end = [&](int tl) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        RowState &s = rs[rb];
        float2 o;
        if constexpr (!kVerify) {
          const float om = kW2First ? half_swap(s.run_m) : pair_swap(s.run_m);
          const float os = kW2First ? half_swap(s.run_s) : pair_swap(s.run_s);
          const float M = fmaxf(s.run_m, om);
          float S = 0.0f;
          if (M != -INFINITY)
            S = s.run_s * exp2_fast((s.run_m - M) * cl) + os * exp2_fast((om - M) * cl);
          o = make_float2(M * invT, S);  // max z = (max of acc + u) / T, exactly
          s.run_m = -INFINITY;
          s.run_s = 0.0f;
        } else {
          const float omin = kW2First ? half_swap(s.run_min) : pair_swap(s.run_min);
          const float ores = kW2First ? half_swap(s.run_res) : pair_swap(s.run_res);
          o = make_float2(s.run_min + omin, s.run_res + ores);
          s.run_min = s.run_res = 0.0f;
        }
        if (row_lead) pbuf[s.slot][tl % kFlushTiles] = o;
      }
    };
    auto flush = [&](int tl) __attribute__((always_inline)) {
      __syncthreads();
      const int n = tl % kFlushTiles + 1, ft = tile0 + tl + 1 - n;
      float2 *out = kVerify ? p.pair_partials : p.tile_stats;
      for (int i = tid; i < kRowGroup * n; i += kThreads) {
        const int row = i / n, t = i - row * n;
        const int orow = pout[row];
        if (orow >= 0) out[(int64_t)orow * n_tiles + ft + t] = pbuf[row][t];
      }
    };

    // ---- pipeline.  The product of block j + 1 is issued before the
    //      epilogue of block j, so the matrix cores work while the vector ALU
    //      reduces: at step j block j + 1 is in LDS stage (j + 1) & 1, W2 of
    //      block j + 2 is in registers and goes to stage j & 1 (free since the
    //      product of block j), and that register set is refilled with block
    //      j + 4; U (P) of block j is used and its set refilled with j + 2.
    WRegs wr0, wr1;
    URegs ur0, ur1;
    floatx16 acc0[RB], acc1[RB];
    __syncthreads();  // the previous range is done with both LDS stages
    load_w(wr0, 0);
    load_w(wr1, 1);
    load_u(ur0, 0);
    load_u(ur1, 1);
    store_w(0, wr0);
    store_w(1, wr1);
    load_w(wr0, 2);
    load_w(wr1, 3);
    __syncthreads();  // blocks 0 and 1 in LDS
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      if (rs[rb].wave_live) mma_block<KS, kW2First>(af[rb], w2s[0], r, acc0[rb]);
    auto step = [&](int j, bool masked, WRegs &wst, URegs &ucur, floatx16 (&acc_j)[RB],
                    floatx16 (&acc_n)[RB]) __attribute__((always_inline)) {
      __syncthreads();  // block j + 1 in stage (j + 1) & 1; stage j & 1 is free
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (rs[rb].wave_live) mma_block<KS, kW2First>(af[rb], w2s[(j + 1) & 1], r, acc_n[rb]);
      store_w(j & 1, wst);  // block j + 2
      load_w(wst, j + 4);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (!rs[rb].wave_live) {
        } else if (masked) {
          epilogue(j, rb, acc_j[rb], ucur, std::true_type{});
        } else {
          epilogue(j, rb, acc_j[rb], ucur, std::false_type{});
        }
      }
      load_u(ucur, j + 2);
    };
    // draft: no branch between the product of block j + 1 and the epilogue of
    // block j (every wave runs both; a wave without live rows works on
    // clamped rows and its results are dropped), so the scheduler can put a
    // few epilogue instructions after each matrix instruction: they issue
    // while the matrix core works (25.0 vs 26.4 us per draft step)
    auto step_d = [&](int j, auto mask_tag, WRegs &wst, URegs &ucur, floatx16 (&acc_j)[RB],
                      floatx16 (&acc_n)[RB]) __attribute__((always_inline)) {
      __syncthreads();  // block j + 1 in stage (j + 1) & 1; stage j & 1 is free
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        mma_block<KS, kW2First>(af[rb], w2s[(j + 1) & 1], r, acc_n[rb]);
      store_w(j & 1, wst);  // block j + 2
      load_w(wst, j + 4);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) epilogue(j, rb, acc_j[rb], ucur, mask_tag);
      load_u(ucur, j + 2);
#pragma unroll
      for (int i = 0; i < 16 * RB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix instruction
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // then six vector ALU
      }
    };
    if constexpr (kVerify) {
      // blocks in pairs (the register sets alternate with the block's parity)
      // with the tile's end checked after each block: half the code of the
      // tile-unrolled loop below, which matters for the larger verify
      // epilogue (measured 133 -> 126 us on a long-block round)
      for (int j = 0; j < nblk; j += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int jb = j + h;
          if (h == 0) step(jb, (cb0 + jb + 1) * kBlockCols > V, wr0, ur0, acc0, acc1);
          else step(jb, (cb0 + jb + 1) * kBlockCols > V, wr1, ur1, acc1, acc0);
          if ((jb + 1) % kBlocksPerTile == 0) {
            const int tl = jb / kBlocksPerTile;
            tile_end(tl);
            if (tl % kFlushTiles == kFlushTiles - 1 || tl == ntile - 1) flush(tl);
          }
        }
      }
    } else {
      // full tiles, then the range's last tile alone where it passes V
      const bool mask_last = (int64_t)(tile0 + ntile) * kTileN > V;
      const int nfull = ntile - (mask_last ? 1 : 0);
      for (int tl = 0; tl < nfull; ++tl) {
        const int j = tl * kBlocksPerTile;
        step_d(j, std::false_type{}, wr0, ur0, acc0, acc1);
        step_d(j + 1, std::false_type{}, wr1, ur1, acc1, acc0);
        step_d(j + 2, std::false_type{}, wr0, ur0, acc0, acc1);
        step_d(j + 3, std::false_type{}, wr1, ur1, acc1, acc0);
        tile_end(tl);
        if (tl % kFlushTiles == kFlushTiles - 1 || tl == ntile - 1) flush(tl);
      }
      if (mask_last) {
        const int tl = ntile - 1, j = tl * kBlocksPerTile;
        step_d(j, std::true_type{}, wr0, ur0, acc0, acc1);
        step_d(j + 1, std::true_type{}, wr1, ur1, acc1, acc0);
        step_d(j + 2, std::true_type{}, wr0, ur0, acc0, acc1);
        step_d(j + 3, std::true_type{}, wr1, ur1, acc1, acc0);
        tile_end(tl);
        flush(tl);
      }
    }
  }
  if (bad_entry) flag_error(p.err, kErrLength);
}

// Workgroups of a stream_tile_kernel launch: at most max_groups (one per
// compute unit), each with the same number of (row group, tile) items.
inline int stream_tile_grid(int total_items, int max_groups) {
  if (total_items <= 0) return 1;
  const int per = (total_items + max_groups - 1) / max_groups;
  return (total_items + per - 1) / per;
}

// v = acc + U (before the temperature) of one row over one vocabulary tile,
// formed by the same instruction sequence as stream_tile_kernel with the same
// operand order: W2 columns from global memory (W2 first: in the order
// block_col_of_m), the row's A operand from LDS (ldsArow: r elements) read by
// every row position of the block, the result taken from position
// row_in_block = the row's index mod 32, where stream_tile_kernel had it; K in
// increasing order from a zero accumulator.  Called by all 256 threads; wave w
// produces columns 32w..32w+31 of the tile.  Writes v (or -inf past V) to
// vout[0..127].
// KS > 0 fixes the number of K steps at compile time (see mma_rows).
template <typename T, bool kW2First, int KS = 0>
__device__ __forceinline__ void recompute_tile_v(const T *ldsArow, const T *W2, const T *Urow,
                                                 int V, int r, int tile, int row_in_block,
                                                 float *vout) {
  constexpr int kPer = 16 / (int)sizeof(T);  // elements per 16-byte piece
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int b0 = tile * kTileN + wave * 32;  // first column of this wave's block
  if constexpr (kW2First) {
    // lanes row_in_block and row_in_block + 32 end with columns
    // b0 + 16 (l / 32) .. +15; their U pieces (a 16-byte piece is all in or
    // all out of [0, V)) are in flight with the W2 loads
    const int c0 = b0 + (lane >> 5) * 16;
    u32x4 ur[16 / kPer];
#pragma unroll
    for (int i = 0; i < 16 / kPer; ++i)
      ur[i] = *reinterpret_cast<const u32x4 *>(Urow + min(c0 + i * kPer, V - kPer));
    BFrag<T> bfr;
    load_bfrag(W2, V, r, b0 + block_col_of_m(lane & 31), bfr);
    floatx16 acc[1];
    mma_rows<true, 1, KS>(ldsArow, 0, 0, r, bfr, acc);
    if ((lane & 31) == row_in_block) {
#pragma unroll
      for (int i = 0; i < 16 / kPer; ++i) {
        float u[kPer];
        unpack16(ur[i], (T *)nullptr, u);
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int c = i * kPer + q;
          vout[wave * 32 + (lane >> 5) * 16 + c] = c0 + c < V ? acc[0][c] + u[q] : -INFINITY;
        }
      }
    }
  } else {
    // lane l (l % 32 = the column) holds the row in register
    // acc_reg_of_row(row_in_block) of lane half acc_half_of_row(row_in_block)
    const int col = b0 + (lane & 31);
    const float u = Elem<T>::at(Urow, min(col, V - 1));  // in flight with the W2 loads
    BFrag<T> bfr;
    load_bfrag(W2, V, r, col, bfr);
    floatx16 acc[1];
    mma_rows<false, 1, KS>(ldsArow, 0, 0, r, bfr, acc);
    const int reg = acc_reg_of_row(row_in_block);
    if ((lane >> 5) == acc_half_of_row(row_in_block)) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (e == reg) a = acc[0][e];
      vout[wave * 32 + (lane & 31)] = col < V ? a + u : -INFINITY;
    }
  }
}

}  // namespace dspark
