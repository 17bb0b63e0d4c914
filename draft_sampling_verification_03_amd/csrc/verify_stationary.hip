// W2-stationary verify product: the per-tile (sum min(p, q), sum (p - q)_+)
// partials of every verified draft, with W2 held on chip.
//
// Verification recomputes the draft's logits z_k = U_k + W1[x_{k-1}] W2 of
// every verified position (Blog, "One-token exactness": the draft's q must be
// the one the draw came from) and meets them with the target's p (Blog,
// "Total variation label").  Here each workgroup (one per compute unit) owns
// a fixed range of at most NT whole 128-column vocabulary tiles, keeps their
// W2 columns for the whole launch (wave w: block w of every tile; the first
// NT - 1 tiles in registers, the last in LDS), and streams every verified row
// past them: for each 32-row block of compact rows, the transition rows come
// to LDS, and each wave multiplies its W2 blocks with them on the matrix cores
// (bf16 32x32x16, W2 first, K ascending from zero: the draft's instruction
// sequence, so z is bit-identical to the draft's) and reduces its 32 columns
// of each row to the two partials in the epilogue.  A row's U_k and P
// segments arrive as 1280-byte runs (the workgroup's five tiles), prefetched
// one row block ahead in a register ring, instead of 64-byte pieces of 512
// rows at a time.  A small pass before it gathers each verified row's q and
// p statistics into one record, so that the product needs a single load per
// row besides its U_k and P.
#include "bias_tile.h"
#include "kernels.h"
#include "trace.h"

namespace dspark {

namespace {

constexpr int kSKS = kMaxRank / 16;   // K steps (r = 256)
constexpr int kSPitch = kMaxRank + 8;  // LDS pitch of a transition row (bf16 elements)

struct VStatParams {
  int R, gamma, V, n_tiles, rows_capacity;
  float invT;
  const bf16_t *U;             // [R][gamma][V]
  const bf16_t *W2;            // column-major 256 x V
  const bf16_t *P;             // [rows_capacity][V]
  const bf16_t *A;             // [R*gamma][256]: transition rows of the compact rows
  const int32_t *row_offset;   // [R + 1]
  const float2 *p_chunks;      // [rows_capacity][kChunks]
  const float *q_stats;        // [R][gamma][2]
  const int4 *row_map;         // [R*gamma]: (rho, k, x_{k-1}, target row)
  float4 *row_stats;           // [R*gamma]: (m_q, log2 S_q, m_p, log2 S_p)
  float2 *pair_partials;       // [R*gamma][n_tiles]
  int32_t *err;
};

// Number of verified drafts (compact rows), sum of ell, from the row offsets.
__device__ __forceinline__ int compact_rows(const VStatParams &p) {
  const int n = p.row_offset[p.R] - p.R;
  return n > p.R * p.gamma ? p.R * p.gamma : n;
}

// A compact-row entry that does not name a verified draft of the batch.
__device__ __forceinline__ bool bad_entry(const VStatParams &p, const int4 e) {
  return e.x < 0 || e.x >= p.R || e.y < 1 || e.y > p.gamma || e.w < 0 || e.w >= p.rows_capacity;
}

// Statistics of every compact row in the form the product's epilogue takes
// them, so that a row's epilogue inputs are one load away from its index:
// q_k's (m, log2 S) from the draft, p's from the target row's chunk partials.
__global__ __launch_bounds__(kBlock) void verify_row_stats_kernel(VStatParams p) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i >= compact_rows(p)) return;
  const int4 e = p.row_map[i];
  if (bad_entry(p, e)) {
    flag_error(p.err, kErrLength);
    p.row_stats[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    return;
  }
  const int64_t qi = (int64_t)e.x * p.gamma + e.y - 1;
  const float2 ps = combine_chunk_stats(p.p_chunks + (int64_t)e.w * kChunks);
  p.row_stats[i] = make_float4(p.q_stats[2 * qi], log2_fast(p.q_stats[2 * qi + 1]), ps.x, log2_fast(ps.y));
}

template <int NT>
struct VStatLds {
  bf16_t rows[2][kRowsPerWave * kSPitch];  // transition rows of two row blocks
  u32x4 w2l[kSKS * 4 * kWave];             // W2 of the last tile slot, per lane
  float2 part[kRowsPerWave][NT][4];        // (sum min, sum residual) per row, slot, wave
  int live[2][kRowsPerWave];               // the row's entry is valid (row block parity)
};

// Where a lane's row of a row block comes from: its U_k row (rho gamma + k - 1)
// and its target row.
struct RowIx {
  int qi, prow;
  bool live;
};

template <int NT, bool kMask>
__global__ __launch_bounds__(kBlock, 1) void verify_stationary_kernel(VStatParams p) {
  __shared__ __align__(16) VStatLds<NT> sh;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int G = gridDim.x, g = blockIdx.x;
  const int V = p.V, nT = p.n_tiles;
  const int t0 = (int)((int64_t)g * nT / G), t1 = (int)((int64_t)(g + 1) * nT / G);
  const int ntl = t1 - t0;  // <= NT (checked by the host)
  const float invT = p.invT;
  const int m = lane & 31, half = lane >> 5;

  const int n_rows = compact_rows(p);
  if (n_rows <= 0) return;
  const int nrb = (n_rows + kRowsPerWave - 1) / kRowsPerWave;

  // ---- W2 of this wave's blocks: slots 0 .. NT - 2 in registers (pinned in
  //      the accumulation registers, which the products read directly), the
  //      last slot in LDS; a slot past the range or a column past V reads a
  //      clamped column whose results are dropped
  constexpr int kRegTiles = NT - 1;
  u16x8 w2r[kRegTiles][kSKS];
  {
    // every load in flight before the first pin (a pin consumes its value,
    // so a pin after each load made the loads one round trip each)
    u16x8 w2f[kSKS];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int col = min((t0 + i) * kTileN + wave * kBlockCols + block_col_of_m(m), V - 1);
      const bf16_t *src = p.W2 + (int64_t)col * kMaxRank + half * 8;
#pragma unroll
      for (int ks = 0; ks < kSKS; ++ks) {
        const u16x8 v = *reinterpret_cast<const u16x8 *>(src + ks * 16);
        if (i < kRegTiles) w2r[i < kRegTiles ? i : 0][ks] = v;
        else w2f[ks] = v;
      }
    }
#pragma unroll
    for (int i = 0; i < kRegTiles; ++i)
#pragma unroll
      for (int ks = 0; ks < kSKS; ++ks) asm volatile("" : "+a"(w2r[i][ks]));
#pragma unroll
    for (int ks = 0; ks < kSKS; ++ks)
      sh.w2l[(ks * 4 + wave) * kWave + lane] = __builtin_bit_cast(u32x4, w2f[ks]);
  }

  // ---- the lane's row of row block rb (its index clamped past n_rows)
  auto row_index = [&](int rb, int mm) __attribute__((always_inline)) {
    return min(rb * kRowsPerWave + mm, n_rows - 1);
  };
  auto decode = [&](int rb, int mm, const int4 e) __attribute__((always_inline)) {
    RowIx x;
    x.live = rb * kRowsPerWave + mm < n_rows && !bad_entry(p, e);
    x.qi = x.live ? e.x * p.gamma + e.y - 1 : 0;
    x.prow = x.live ? e.w : 0;
    return x;
  };

  // ---- U and P of item (row, tile slot i): this lane's 16 columns, each
  //      8-column piece clamped on its own (a piece is wholly inside or
  //      outside [0, V) because V % 8 == 0)
  struct UPPiece { u32x4 ua, ub, pa, pb; };
  auto load_up = [&](const RowIx &x, int i, int hf) __attribute__((always_inline)) {
    const int c0 = (t0 + i) * kTileN + wave * kBlockCols + hf * 16;
    const int ca = kMask ? min(c0, V - 8) : min(c0, V - 16);
    const int cb = kMask ? min(c0 + 8, V - 8) : ca + 8;
    const bf16_t *Urow = p.U + (int64_t)x.qi * V, *Prow = p.P + (int64_t)x.prow * V;
    UPPiece u;
    u.ua = *reinterpret_cast<const u32x4 *>(Urow + ca);
    u.ub = *reinterpret_cast<const u32x4 *>(Urow + cb);
    u.pa = *reinterpret_cast<const u32x4 *>(Prow + ca);
    u.pb = *reinterpret_cast<const u32x4 *>(Prow + cb);
    return u;
  };

  // ---- transition rows of row block rb: thread t loads 16-byte piece t % 32
  //      of rows t / 32 + 8 j (rows past n_rows read the last one; they are
  //      not live)
  constexpr int kPieces = kMaxRank * 2 / 16;
  constexpr int kAIt = kRowsPerWave * kPieces / kBlock;  // 4
  auto load_rows = [&](int rb, u32x4 (&v)[kAIt], int t) __attribute__((always_inline)) {
    const int off = (t % kPieces) * 8, row0 = t / kPieces;
#pragma unroll
    for (int j = 0; j < kAIt; ++j) {
      const int i = min(rb * kRowsPerWave + row0 + j * (kBlock / kPieces), n_rows - 1);
      v[j] = *reinterpret_cast<const u32x4 *>(p.A + (int64_t)i * kMaxRank + off);
    }
  };
  auto store_rows = [&](int buf, const u32x4 (&v)[kAIt], int t) __attribute__((always_inline)) {
    const int off = (t % kPieces) * 8, row0 = t / kPieces;
#pragma unroll
    for (int j = 0; j < kAIt; ++j)
      *reinterpret_cast<u32x4 *>(sh.rows[buf] + (row0 + j * (kBlock / kPieces)) * kSPitch + off) = v[j];
  };

  // ---- row block 0: rows, statistics and the U/P ring; the entry of row
  //      block 1.  Loads stay ordered so that no wait for a recent load
  //      (returns are counted in issue order) is also a wait for the ring:
  //      an entry is loaded a block before its indices are needed, the
  //      statistics a block before the epilogue reads them.
  {
    u32x4 v[kAIt];
    load_rows(0, v, tid);
    store_rows(0, v, tid);
  }
  const RowIx x0 = decode(0, m, p.row_map[row_index(0, m)]);
  float4 cur = p.row_stats[row_index(0, m)];
  if (wave == 0 && lane < kRowsPerWave) sh.live[0][lane] = x0.live;
  int4 e_next = p.row_map[row_index(1, m)];
  UPPiece ring[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) ring[i] = load_up(x0, i, half);
  __syncthreads();

  for (int rb = 0; rb < nrb; ++rb) {
    const int buf = rb & 1;
    const bool has_next = rb + 1 < nrb;
    // the thread's index, opaque to the compiler once per row block:
    // addresses derived from it are formed again in every block instead of
    // being held across the loop (where they went to scratch, and every
    // reload waited for all loads in flight, the U/P ring included)
    int tid_b = tid;
    asm volatile("" : "+v"(tid_b));
    const int m_b = tid_b & 31, half_b = (tid_b >> 5) & 1;
    // row block rb + 1: indices from the entry loaded a block ago; its
    // statistics, transition rows and the entry of rb + 2 go in flight now
    const RowIx nx = decode(rb + 1, m_b, e_next);
    e_next = p.row_map[row_index(rb + 2, m_b)];
    const float4 nst = p.row_stats[row_index(rb + 1, m_b)];
    u32x4 arow_next[kAIt];
    load_rows(has_next ? rb + 1 : rb, arow_next, tid_b);

    u16x8 bfr[kSKS];
    {
      const bf16_t *rowp = sh.rows[buf] + m_b * kSPitch + half_b * 8;
#pragma unroll
      for (int ks = 0; ks < kSKS; ++ks) bfr[ks] = *reinterpret_cast<const u16x8 *>(rowp + ks * 16);
    }
    auto mma = [&](int i) __attribute__((always_inline)) {
      floatx16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
      if (i < NT - 1) {
#pragma unroll
        for (int ks = 0; ks < kSKS; ++ks) acc = mfma16<true>(w2r[i < NT - 1 ? i : 0][ks], bfr[ks], acc);
      } else {
#pragma unroll
        for (int ks = 0; ks < kSKS; ++ks)
          acc = mfma16<true>(__builtin_bit_cast(u16x8, sh.w2l[(ks * 4 + wave) * kWave + (tid_b & 63)]),
                             bfr[ks], acc);
      }
      return acc;
    };
    // the epilogue of item i: (sum min(p, q), sum (p - q)_+) of the lane's 16
    // columns, merged with the other 16 of the row (lane l ^ 32)
    auto epilogue = [&](int i, const floatx16 &acc) __attribute__((always_inline)) {
      float u[16], t[16];
      unpack16(ring[i].ua, (bf16_t *)nullptr, u);
      unpack16(ring[i].ub, (bf16_t *)nullptr, u + 8);
      unpack16(ring[i].pa, (bf16_t *)nullptr, t);
      unpack16(ring[i].pb, (bf16_t *)nullptr, t + 8);
      ring[i] = load_up(nx, i, half_b);  // the same slot, one row block later
      const int c0 = (t0 + i) * kTileN + wave * kBlockCols + half_b * 16;
      float smin = 0.0f, sres = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float a = log2_prob(t[c], invT, cur.z, cur.w);            // log2 p
        const float b = log2_prob(acc[c] + u[c], invT, cur.x, cur.y);   // log2 q, z T = acc + u
        const float mn = exp2_fast(fminf(a, b));
        const float pe = exp2_fast(a);
        const bool in = !kMask || c0 + c < V;
        smin += in ? mn : 0.0f;
        sres += in ? pe - mn : 0.0f;
      }
      // both lanes of a row form the same sums (addition is commutative)
      smin += half_swap(smin);
      sres += half_swap(sres);
      sh.part[m_b][i][wave] = make_float2(smin, sres);
    };
    floatx16 acc0 = mma(0), acc1;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (i + 1 < NT) {
        if (i & 1) acc0 = mma(i + 1);
        else acc1 = mma(i + 1);
      }
      epilogue(i, (i & 1) ? acc1 : acc0);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix instruction
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // then six vector ALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the same for the stores that end the block
    int tid_t = tid;
    asm volatile("" : "+v"(tid_t));
    if (has_next) {
      store_rows(buf ^ 1, arow_next, tid_t);
      if (tid_t < kRowsPerWave) sh.live[buf ^ 1][tid_t] = nx.live;
    }
    __syncthreads();  // the block's partials and the next block's rows are in LDS

    // ---- the block's tile partials (fixed wave order) to global memory
    for (int q = tid_t; q < kRowsPerWave * ntl; q += kBlock) {
      const int row = q / ntl, i = q - row * ntl;
      const int ci = rb * kRowsPerWave + row;
      if (sh.live[buf][row]) {
        float2 o = sh.part[row][i][0];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          o.x += sh.part[row][i][w].x;
          o.y += sh.part[row][i][w].y;
        }
        p.pair_partials[(int64_t)ci * nT + t0 + i] = o;
      }
    }
    cur = nst;
    __syncthreads();  // sh.part is written again by the next block
  }
}

}  // namespace

// Launch shape of the W2-stationary verify product, or false when the shape
// does not fit it: bf16, r = 256, one workgroup per compute unit holding at
// most 5 tiles (640 columns) of W2.
bool verify_stationary_shape(int V, int r, bool bf16, int *grid, int *nt) {
  if (!bf16 || r != kMaxRank || V < kTileN) return false;
  const int n_tiles = (V + kTileN - 1) / kTileN;
  const int G = n_tiles < kComputeUnits ? n_tiles : kComputeUnits;
  const int per = (n_tiles + G - 1) / G;
  if (per > 5) return false;
  *grid = G;
  *nt = per <= 4 ? 4 : 5;
  return true;
}

hipError_t launch_verify_stationary(const VerifyLaunch &L, int G, int nt, hipStream_t stream) {
  VStatParams vp{};
  vp.R = L.R; vp.gamma = L.gamma; vp.V = L.V; vp.n_tiles = (L.V + kTileN - 1) / kTileN;
  vp.rows_capacity = L.rows_capacity; vp.invT = L.invT;
  vp.U = reinterpret_cast<const bf16_t *>(L.U);
  vp.W2 = reinterpret_cast<const bf16_t *>(L.W2);
  vp.P = reinterpret_cast<const bf16_t *>(L.P);
  vp.A = reinterpret_cast<const bf16_t *>(L.A_rows);
  vp.row_offset = L.row_offset; vp.p_chunks = L.p_chunks; vp.q_stats = L.q_stats;
  vp.row_map = L.row_map; vp.row_stats = L.row_stats; vp.pair_partials = L.pair_partials;
  vp.err = L.err;
  DSPARK_LAUNCH("verify_row_stats", stream, verify_row_stats_kernel,
                (L.R * L.gamma + kBlock - 1) / kBlock, kBlock, vp);
  const bool mask = L.V % kTileN != 0;
  if (nt == 4) {
    if (mask) DSPARK_LAUNCH("bias_tile_verify", stream, (verify_stationary_kernel<4, true>), G, kBlock, vp);
    else DSPARK_LAUNCH("bias_tile_verify", stream, (verify_stationary_kernel<4, false>), G, kBlock, vp);
  } else {
    if (mask) DSPARK_LAUNCH("bias_tile_verify", stream, (verify_stationary_kernel<5, true>), G, kBlock, vp);
    else DSPARK_LAUNCH("bias_tile_verify", stream, (verify_stationary_kernel<5, false>), G, kBlock, vp);
  }
  return hipGetLastError();
}

}  // namespace dspark
