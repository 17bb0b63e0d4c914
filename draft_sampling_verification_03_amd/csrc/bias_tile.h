// Fused Markov-bias tile kernel: gather W1 rows -> matrix-core product with W2
// -> add U_k and scale by 1/T -> per-(row, vocabulary tile) reduction.
//
// The Markov head (Blog, "Markov sequential head"; KB section 2) adds the bias
// row W1[x_{k-1}, :] W2 to the backbone logits U_k.  For a batch of rows this is
// an [M, r] x [r, V] product whose only consumer is a vocabulary-wide
// reduction, so z never goes to HBM: a workgroup owns one 128-column
// vocabulary tile, keeps it on chip and emits one partial per row.
//
//   Draft epilogue  (m_t, s_t) = (max_v z, sum_v exp(z - m_t)) of the tile
//   Verify epilogue (sum_v min(p, q), sum_v (p - q)_+) of the tile, with
//                   q = exp(z - m_q)/S_q from the draft's statistics and
//                   p = exp(t/T - m_p)/S_p from the target row statistics
//
// Work split.  Each of the 4 waves owns 32 of the 128 columns; it loads the r
// coefficients of its 32 W2 columns into registers once (all K at a time, so
// one memory round trip) and keeps them for every row tile the workgroup
// visits: W2 crosses HBM once per launch.  Row tiles of TM rows (all requests
// for the draft, the compacted verified drafts for verification) are walked
// in a loop; per row tile the gathered W1 rows go to LDS, every wave multiplies
// all TM rows by its columns, the accumulators are transposed through the same
// LDS for a row-wise epilogue, and the U (and P) row segments that epilogue
// reads are prefetched into registers before the matrix-core work starts.
#pragma once
#include "common.h"

namespace dspark {

constexpr int kLdsBytesPerRow = 528;  // max(r_max + 8 bf16, r_max + 4 fp32, 132 fp32)
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
  // (draft, row = request) or [R*gamma][r] (verify, row = compact row)
  const void *A;
};

enum class Epi { kDraft, kVerify };

template <typename T, int TM, Epi E>
__global__ __launch_bounds__(kBlock, 2) void bias_tile_kernel(BiasTileParams p) {
  constexpr int WMB = TM / 32;                // 32-row blocks per wave
  constexpr int kG = kBlock / TM;             // threads per epilogue row
  constexpr int kSeg = TM * kTileN / kBlock;  // columns per thread in the epilogue
  constexpr int kPer = 16 / (int)sizeof(T);   // elements per 16-byte piece
  constexpr int kVec = kSeg / kPer;           // 16-byte pieces per segment
  constexpr int kPitchC = kTileN + 4;         // fp32 pitch of the transposed tile
  constexpr int kMaxA = TM * 32 / kBlock;     // gathered 16-byte pieces per thread (r max)
  constexpr bool kVerify = E == Epi::kVerify;
  __shared__ __align__(16) unsigned char smem[TM * kLdsBytesPerRow];
  __shared__ int row_prev[TM];  // token whose W1 row feeds the row (-1: padding row)
  __shared__ int row_req[TM];   // request of the row
  __shared__ int row_pos[TM];   // draft position k of the row (0: skipped)
  __shared__ int row_out[TM];   // output row index
  __shared__ int row_prow[TM];  // verify: target row of the row

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int nt = blockIdx.x;
  const int V = p.V, r = p.r;

  int n_rows_total;
  if constexpr (!kVerify) {
    n_rows_total = p.R;
  } else {
    n_rows_total = p.row_offset[p.R] - p.R;  // sum of ell
    if (n_rows_total > p.R * p.gamma) n_rows_total = p.R * p.gamma;
  }
  const int n_mt = n_rows_total > 0 ? (n_rows_total + TM - 1) / TM : 0;
  if ((int)blockIdx.y >= n_mt) return;  // uniform across the workgroup

  // the wave's 32 W2 columns, all of K, kept for every row tile
  BFrag<T> bfr;
  load_bfrag(reinterpret_cast<const T *>(p.W2), V, r, nt * kTileN + wave * 32, bfr);

  T *ldsA = reinterpret_cast<T *>(smem);
  float *ldsC = reinterpret_cast<float *>(smem);
  const int a_pitch = lds_pitch<T>(r);
  const int erow = tid / kG;         // epilogue row of the tile
  const int c0 = (tid % kG) * kSeg;  // first column of the thread's segment
  const int vbase = nt * kTileN + c0;
  const int pieces = r * (int)sizeof(T) / 16;  // 16-byte pieces per W1 row, <= 32

  for (int mt = blockIdx.y; mt < n_mt; mt += gridDim.y) {
    __syncthreads();  // the previous tile's epilogue is done with LDS
    // ---- row info: none for the draft (row = request), one load of the
    //      compact-row map (written by the target-row statistics pass) to verify
    if (tid < TM) {
      const int i = mt * TM + tid;
      int prev = -1, rho = 0, k = 0, prow = 0;
      if (i < n_rows_total) {
        if constexpr (!kVerify) {
          rho = i;
          k = p.k;
          prev = 0;  // the row's W1[x_{k-1}] is A[i]
        } else {
          const int4 e = p.row_map[i];  // (rho, k, prev, target row), checked when written
          rho = e.x; k = e.y; prev = e.z; prow = e.w;
          if (rho < 0 || rho >= p.R || k < 1 || k > p.gamma || prev < 0 || prev >= V ||
              prow < 0 || prow >= p.rows_capacity) {
            flag_error(p.err, kErrLength);
            prev = -1; rho = 0; k = 0; prow = 0;
          }
        }
      }
      row_prev[tid] = prev;
      row_req[tid] = rho;
      row_pos[tid] = k;
      row_out[tid] = i;
      row_prow[tid] = prow;
    }
    __syncthreads();

    // ---- A rows of this tile from the contiguous transition-row buffer: every
    //      load in flight before the first store; clamped addresses, masked
    //      values (zero rows for padding)
    {
      const int total = TM * pieces;
      const T *Ab = reinterpret_cast<const T *>(p.A);
      const int last_row = n_rows_total - 1;
      uint4 av[kMaxA];
#pragma unroll
      for (int j = 0; j < kMaxA; ++j) {
        const int idx = min(tid + j * kBlock, total - 1);
        const int row = idx / pieces, pc = idx - row * pieces;
        const int gi = min(mt * TM + row, last_row);
        const uint4 v = *reinterpret_cast<const uint4 *>(Ab + (int64_t)gi * r + pc * kPer);
        av[j] = row_prev[row] >= 0 ? v : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < kMaxA; ++j) {
        const int idx = tid + j * kBlock;
        if (idx < total) {
          const int row = idx / pieces, pc = idx - row * pieces;
          *reinterpret_cast<uint4 *>(ldsA + row * a_pitch + pc * kPer) = av[j];
        }
      }
    }

    // ---- prefetch the epilogue's U (and P) row segments: their latency
    //      overlaps the matrix-core work
    const int k = row_pos[erow];
    const bool live = row_prev[erow] >= 0 && k >= 1;
    const int rho = row_req[erow];
    const T *Urow =
        reinterpret_cast<const T *>(p.U) + ((int64_t)rho * p.gamma + (k >= 1 ? k - 1 : 0)) * V;
    const T *Prow = reinterpret_cast<const T *>(p.P) + (int64_t)row_prow[erow] * V;
    uint4 upre[kVec], ppre[kVerify ? kVec : 1];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int v0 = min(vbase + j * kPer, V - kPer);  // V % 8 == 0: pieces are all in or out
      const uint4 u = *reinterpret_cast<const uint4 *>(Urow + v0);
      upre[j] = u;
      if constexpr (kVerify) ppre[j] = *reinterpret_cast<const uint4 *>(Prow + v0);
    }
    __syncthreads();

    floatx16 acc[WMB];
    mma_rows<WMB>(ldsA, a_pitch, 0, r, bfr, acc);
    __syncthreads();  // A no longer needed: the LDS takes the transposed tile
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = mb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        ldsC[row * kPitchC + wave * 32 + (lane & 31)] = acc[mb][e];
      }
    __syncthreads();

    // ---- row-wise epilogue on the thread's kSeg consecutive columns
    if constexpr (!kVerify) {
      // two passes over the segment (max, then sum of exp); z is formed by the
      // same expression both times instead of being held in registers
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        float u[kPer];
        unpack16(upre[j], (T *)nullptr, u);
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int col = j * kPer + q;
          const float zz = (ldsC[erow * kPitchC + c0 + col] + u[q]) * p.invT;
          mx = fmaxf(mx, (vbase + col < V) ? zz : -INFINITY);
        }
      }
      mx = group_max<kG>(mx);
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        float u[kPer];
        unpack16(upre[j], (T *)nullptr, u);
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int col = j * kPer + q;
          const float zz = (ldsC[erow * kPitchC + c0 + col] + u[q]) * p.invT;
          s += (vbase + col < V) ? fexp(zz - mx) : 0.0f;
        }
      }
      s = group_sum<kG>(s);
      if (live && (tid % kG) == 0)
        p.tile_stats[(int64_t)row_out[erow] * p.n_tiles + nt] = make_float2(mx, s);
    } else {
      float mq = 0.0f, rq = 0.0f, mp = 0.0f, rp = 0.0f;
      if (live) {
        const int64_t qi = (int64_t)rho * p.gamma + k - 1;
        mq = p.q_stats[2 * qi];
        rq = 1.0f / p.q_stats[2 * qi + 1];
        const float2 ps = combine_chunk_stats(p.p_chunks + (int64_t)row_prow[erow] * kChunks);
        mp = ps.x;
        rp = 1.0f / ps.y;
      }
      float smin = 0.0f, sres = 0.0f;
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        float u[kPer], t[kPer];
        unpack16(upre[j], (T *)nullptr, u);
        unpack16(ppre[j], (T *)nullptr, t);
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int col = j * kPer + q;
          const float zz = (ldsC[erow * kPitchC + c0 + col] + u[q]) * p.invT;
          const float qv = fexp(zz - mq) * rq;
          const float pv = fexp(t[q] * p.invT - mp) * rp;
          const bool in = vbase + col < V;
          smin += in ? fminf(pv, qv) : 0.0f;
          sres += in ? fmaxf(pv - qv, 0.0f) : 0.0f;
        }
      }
      smin = group_sum<kG>(smin);
      sres = group_sum<kG>(sres);
      if (live && (tid % kG) == 0)
        p.pair_partials[(int64_t)row_out[erow] * p.n_tiles + nt] = make_float2(smin, sres);
    }
  }
}

// Draft product, software-pipelined over 32-row tiles.  One workgroup owns one
// 128-column vocabulary tile for all R rows: each wave keeps its 32 W2 columns
// in registers; the A rows of tile t+1 (from the contiguous transition-row
// buffer, into the other half of a double-buffered LDS area) and its U row
// segments (into a second register set) are loaded while tile t is multiplied
// and reduced.  Arithmetic per element is that of bias_tile_kernel's draft
// epilogue: z = (acc + U) * (1/T), max, then sum of exp(z - max).
template <typename T>
__global__ __launch_bounds__(kBlock, 3) void draft_tile_kernel(BiasTileParams p) {
  constexpr int TM = 32;
  constexpr int kG = kBlock / TM;             // 8 threads per epilogue row
  constexpr int kSeg = TM * kTileN / kBlock;  // 16 columns per thread
  constexpr int kPer = 16 / (int)sizeof(T);
  constexpr int kVec = kSeg / kPer;           // 16-byte U pieces per thread
  constexpr int kPitchC = kTileN + 4;
  constexpr int kMaxA = TM * 32 / kBlock;     // 16-byte A pieces per thread (r max)
  __shared__ __align__(16) unsigned char abuf[2][TM * kLdsBytesPerRow];
  __shared__ __align__(16) float cbuf[TM * kPitchC];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int nt = blockIdx.x, V = p.V, r = p.r, R = p.R;
  const int n_mt = (R + TM - 1) / TM;
  const int pieces = r * (int)sizeof(T) / 16;
  const int total = TM * pieces;
  const int a_pitch = lds_pitch<T>(r);
  const T *Ab = reinterpret_cast<const T *>(p.A);
  const T *U = reinterpret_cast<const T *>(p.U);
  const int erow = tid / kG, c0 = (tid % kG) * kSeg, vbase = nt * kTileN + c0;

  BFrag<T> bfr;
  load_bfrag(reinterpret_cast<const T *>(p.W2), V, r, nt * kTileN + wave * 32, bfr);

  // loads of one row tile: A pieces (masked for padding rows) and U segments
  auto load_tile = [&](int mt, uint4 (&av)[kMaxA], uint4 (&uv)[kVec]) {
#pragma unroll
    for (int j = 0; j < kMaxA; ++j) {
      const int idx = min(tid + j * kBlock, total - 1);
      const int row = idx / pieces, pc = idx - row * pieces;
      const int gi = min(mt * TM + row, R - 1);
      av[j] = *reinterpret_cast<const uint4 *>(Ab + (int64_t)gi * r + pc * kPer);
      if (mt * TM + row >= R) av[j] = make_uint4(0, 0, 0, 0);
    }
    const int rho = min(mt * TM + erow, R - 1);
    const T *Urow = U + ((int64_t)rho * p.gamma + (p.k - 1)) * V;
    // a 16-byte piece is all in or all out of [0, V) (V % 8 == 0): clamp the
    // address of out-of-range pieces, whose values the epilogue masks
#pragma unroll
    for (int j = 0; j < kVec; ++j)
      uv[j] = ld_stream(Urow + min(vbase + j * kPer, V - kPer));
  };
  auto store_a = [&](int buf, const uint4 (&av)[kMaxA]) {
    T *dst = reinterpret_cast<T *>(abuf[buf]);
#pragma unroll
    for (int j = 0; j < kMaxA; ++j) {
      const int idx = tid + j * kBlock;
      if (idx < total) {
        const int row = idx / pieces, pc = idx - row * pieces;
        *reinterpret_cast<uint4 *>(dst + row * a_pitch + pc * kPer) = av[j];
      }
    }
  };

  uint4 a_next[kMaxA], u_cur[kVec], u_next[kVec];
  load_tile(0, a_next, u_cur);
  store_a(0, a_next);
  for (int mt = 0; mt < n_mt; ++mt) {
    __syncthreads();  // A of tile mt in LDS; the previous epilogue is done with cbuf
    const bool more = mt + 1 < n_mt;
    if (more) load_tile(mt + 1, a_next, u_next);
    floatx16 acc[1];
    mma_rows<1>(reinterpret_cast<const T *>(abuf[mt & 1]), a_pitch, 0, r, bfr, acc);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      cbuf[row * kPitchC + wave * 32 + (lane & 31)] = acc[0][e];
    }
    if (more) store_a((mt + 1) & 1, a_next);
    __syncthreads();
    // epilogue of tile mt: two passes (max, then sum of exp) over 16 columns
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      float u[kPer];
      unpack16(u_cur[j], (T *)nullptr, u);
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int col = j * kPer + q;
        const float zz = (cbuf[erow * kPitchC + c0 + col] + u[q]) * p.invT;
        mx = fmaxf(mx, (vbase + col < V) ? zz : -INFINITY);
      }
    }
    mx = group_max<kG>(mx);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      float u[kPer];
      unpack16(u_cur[j], (T *)nullptr, u);
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int col = j * kPer + q;
        const float zz = (cbuf[erow * kPitchC + c0 + col] + u[q]) * p.invT;
        s += (vbase + col < V) ? fexp(zz - mx) : 0.0f;
      }
    }
    s = group_sum<kG>(s);
    const int rho = mt * TM + erow;
    if (rho < R && (tid % kG) == 0)
      p.tile_stats[(int64_t)rho * p.n_tiles + nt] = make_float2(mx, s);
#pragma unroll
    for (int j = 0; j < kVec; ++j) u_cur[j] = u_next[j];
  }
}

// Verify product, software-pipelined over 32-row tiles of the compacted verified
// drafts.  Per tile t the workgroup, with its W2 columns resident: loads the
// compact-row map entry of tile t+1 (one per epilogue row) while multiplying
// tile t; issues tile t+1's A rows, U and P row segments and row statistics
// while reducing tile t; epilogue arithmetic is bias_tile_kernel's verify
// epilogue (sum min(p, q), sum (p - q)_+ per row and tile).
template <typename T>
__global__ __launch_bounds__(kBlock, 2) void verify_tile_kernel(BiasTileParams p) {
  constexpr int TM = 32;
  constexpr int kG = kBlock / TM;             // 8 threads per epilogue row
  constexpr int kSeg = TM * kTileN / kBlock;  // 16 columns per thread
  constexpr int kPer = 16 / (int)sizeof(T);
  constexpr int kVec = kSeg / kPer;
  constexpr int kPitchC = kTileN + 4;
  constexpr int kMaxA = TM * 32 / kBlock;
  __shared__ __align__(16) unsigned char abuf[2][TM * kLdsBytesPerRow];
  __shared__ __align__(16) float cbuf[TM * kPitchC];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int nt = blockIdx.x, V = p.V, r = p.r;
  int n_rows = p.row_offset[p.R] - p.R;  // sum of ell
  if (n_rows > p.R * p.gamma) n_rows = p.R * p.gamma;
  const int n_mt = n_rows > 0 ? (n_rows + TM - 1) / TM : 0;
  if ((int)blockIdx.y >= n_mt) return;
  const int pieces = r * (int)sizeof(T) / 16;
  const int total = TM * pieces;
  const int a_pitch = lds_pitch<T>(r);
  const T *Ab = reinterpret_cast<const T *>(p.A);
  const T *U = reinterpret_cast<const T *>(p.U);
  const T *P = reinterpret_cast<const T *>(p.P);
  const int erow = tid / kG, c0 = (tid % kG) * kSeg, vbase = nt * kTileN + c0;
  const int step = gridDim.y;

  BFrag<T> bfr;
  load_bfrag(reinterpret_cast<const T *>(p.W2), V, r, nt * kTileN + wave * 32, bfr);

  // compact-row map entry of this thread's epilogue row in tile mt, checked
  auto load_map = [&](int mt) -> int4 {
    const int i = mt * TM + erow;
    int4 e = make_int4(-1, 0, 0, 0);
    if (mt < n_mt && i < n_rows) {
      e = p.row_map[i];
      if (e.x < 0 || e.x >= p.R || e.y < 1 || e.y > p.gamma || e.w < 0 || e.w >= p.rows_capacity) {
        flag_error(p.err, kErrLength);
        e.x = -1;
      }
    }
    return e;
  };
  // loads of tile mt: A pieces (masked for padding rows), U and P segments of
  // the thread's row, and the row's draft and target statistics
  struct Stage {
    uint4 u[kVec], t[kVec];
    float mq, rq, mp, rp;
  };
  auto load_tile = [&](int mt, int4 e, uint4 (&av)[kMaxA], Stage &s) {
#pragma unroll
    for (int j = 0; j < kMaxA; ++j) {
      const int idx = min(tid + j * kBlock, total - 1);
      const int row = idx / pieces, pc = idx - row * pieces;
      const int gi = min(mt * TM + row, n_rows - 1);
      av[j] = *reinterpret_cast<const uint4 *>(Ab + (int64_t)gi * r + pc * kPer);
      if (mt * TM + row >= n_rows) av[j] = make_uint4(0, 0, 0, 0);
    }
    const bool live = e.x >= 0;
    const int rho = live ? e.x : 0, k = live ? e.y : 1, prow = live ? e.w : 0;
    const T *Urow = U + ((int64_t)rho * p.gamma + (k - 1)) * V;
    const T *Prow = P + (int64_t)prow * V;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int v = min(vbase + j * kPer, V - kPer);  // all-in or all-out pieces (V % 8 == 0)
      s.u[j] = ld_stream(Urow + v);
      s.t[j] = ld_stream(Prow + v);
    }
    const int64_t qi = (int64_t)rho * p.gamma + k - 1;
    s.mq = p.q_stats[2 * qi];
    s.rq = 1.0f / p.q_stats[2 * qi + 1];
    const float2 ps = combine_chunk_stats(p.p_chunks + (int64_t)prow * kChunks);
    s.mp = ps.x;
    s.rp = 1.0f / ps.y;
  };
  auto store_a = [&](int buf, const uint4 (&av)[kMaxA]) {
    T *dst = reinterpret_cast<T *>(abuf[buf]);
#pragma unroll
    for (int j = 0; j < kMaxA; ++j) {
      const int idx = tid + j * kBlock;
      if (idx < total) {
        const int row = idx / pieces, pc = idx - row * pieces;
        *reinterpret_cast<uint4 *>(dst + row * a_pitch + pc * kPer) = av[j];
      }
    }
  };

  int mt = blockIdx.y;
  uint4 a_next[kMaxA];
  Stage cur, nxt;
  int4 e_cur = load_map(mt);
  load_tile(mt, e_cur, a_next, cur);
  store_a(0, a_next);
  int buf = 0;
  for (; mt < n_mt; mt += step) {
    __syncthreads();  // A of tile mt in LDS; the previous epilogue is done with cbuf
    const bool more = mt + step < n_mt;
    const int4 e_next = load_map(mt + step);
    floatx16 acc[1];
    mma_rows<1>(reinterpret_cast<const T *>(abuf[buf]), a_pitch, 0, r, bfr, acc);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      cbuf[row * kPitchC + wave * 32 + (lane & 31)] = acc[0][e];
    }
    if (more) load_tile(mt + step, e_next, a_next, nxt);
    __syncthreads();
    // epilogue of tile mt
    float smin = 0.0f, sres = 0.0f;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      float u[kPer], t[kPer];
      unpack16(cur.u[j], (T *)nullptr, u);
      unpack16(cur.t[j], (T *)nullptr, t);
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int col = j * kPer + q;
        const float zz = (cbuf[erow * kPitchC + c0 + col] + u[q]) * p.invT;
        const float qv = fexp(zz - cur.mq) * cur.rq;
        const float pv = fexp(t[q] * p.invT - cur.mp) * cur.rp;
        const bool in = vbase + col < V;
        smin += in ? fminf(pv, qv) : 0.0f;
        sres += in ? fmaxf(pv - qv, 0.0f) : 0.0f;
      }
    }
    smin = group_sum<kG>(smin);
    sres = group_sum<kG>(sres);
    const int i = mt * TM + erow;
    if (e_cur.x >= 0 && (tid % kG) == 0)
      p.pair_partials[(int64_t)i * p.n_tiles + nt] = make_float2(smin, sres);
    if (more) {
      store_a(buf ^ 1, a_next);
      cur = nxt;
    }
    e_cur = e_next;
    buf ^= 1;
  }
}

// Recompute z for one row and one vocabulary tile with the same matrix-core
// sequence and epilogue arithmetic as bias_tile_kernel.  Called by all 256
// threads; wave w produces columns 32w..32w+31 of the tile.  ldsArow holds
// W1[prev] (r elements); the row sits at position `row_in_block` (= its row
// index mod 32) of its 32-row block, which is where bias_tile_kernel computed
// it.  Writes z (or -inf past V) to zout[0..127].
template <typename T>
__device__ __forceinline__ void recompute_tile_z(const T *ldsArow, const T *W2, const T *Urow,
                                                 int V, int r, int tile, int row_in_block,
                                                 float invT, float *zout) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  BFrag<T> bfr;
  load_bfrag(W2, V, r, tile * kTileN + wave * 32, bfr);
  floatx16 acc[1];
  mma_rows<1>(ldsArow, 0, 0, r, bfr, acc);
  const int reg = acc_reg_of_row(row_in_block);
  if ((lane >> 5) == acc_half_of_row(row_in_block)) {
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (e == reg) a = acc[0][e];
    const int col = tile * kTileN + wave * 32 + (lane & 31);
    float z = -INFINITY;
    if (col < V) z = (a + Elem<T>::at(Urow, col)) * invT;
    zout[wave * 32 + (lane & 31)] = z;
  }
}

}  // namespace dspark
