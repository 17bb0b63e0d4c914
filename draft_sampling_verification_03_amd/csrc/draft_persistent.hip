// Persistent Markov-head draft: all gamma steps of one dspark_draft call in a
// single cooperative launch, with the W2 factor held on chip for the whole call.
//
// The Markov head (Blog, "Markov sequential head"; KB section 2) multiplies
// the same r x V factor W2 at every one of the gamma serial steps; the head is
// meant to cost a small, sequential amount on top of the parallel block
// (Bangkok 5.3).  Streaming W2 from memory at every step would triple the
// bytes of a step at R = 128 (W2 is 77.8 MB, the step's U_k rows 38.9 MB).
// Here each workgroup (one per compute unit) owns a fixed range of at most NT
// whole 128-column vocabulary tiles and keeps their W2 columns for the whole
// call: wave w holds the 32-column block w of every tile, the first NT - 1
// tiles' operands in its registers (64 per tile), the last one in LDS.  Per
// step only U_k and the transition rows move.  Past 128 requests the steps
// below run per chunk of 128 requests, and the draws of a chunk come after
// the next chunk's products (see the step loop).
//
// One step k:
//   1. the transition rows A_k = W1[x_{k-1}] of every request (x_0 = anchor)
//      go to LDS, gathered straight from W1 once the step's draws are
//      published;
//   2. for each 32-request row block, each wave multiplies its W2 blocks with
//      the rows on the matrix cores (bf16 32x32x16, fp32 accumulation from
//      zero, K ascending, W2 as the first operand: the same instruction
//      sequence as the per-step product kernel, so every z = acc + U is
//      bit-identical to what the sampler recomputes), adds U_k and reduces
//      each row's 32 columns to (max, sum of exp) in the epilogue, which runs
//      while the next tile slot's products issue;
//   3. the four waves' block partials of a tile combine in a fixed order into
//      the tile partial (m_t, s_t), stored as one 8-byte word in the half of
//      the partial buffer that belongs to the step's parity;
//   4. the workgroups that own requests (rho = g, g + G, ...) poll their row's
//      partial words until every one is written, reset them, draw x_k with the
//      two-level inverse CDF of sampler.h and publish (k << 32) | x_k in the
//      request's word;
//   5. every workgroup waits for all R words of step k before step k + 1.
// The data itself is the signal: no flag word stands between a write and its
// reader, and no store has to be acknowledged before another is issued,
// except the resets, which complete before the draw that follows them is
// published (the partial words are written again two steps later, only
// after that draw).  Every access to shared words is device-coherent, every
// wait is bounded, and a wait that runs out sets DSPARK_DEVERR_SYNC and ends
// the kernel.  The cooperative launch guarantees that all workgroups are
// resident at once.
#include "bias_tile.h"
#include "kernels.h"
#include "sampler.h"
#include "trace.h"

namespace dspark {

constexpr int kPRows = 128;                 // requests whose rows fit in LDS
constexpr int kPKS = kMaxRank / 16;         // K steps (r = 256)
constexpr int kPPitch = kMaxRank + 8;       // LDS pitch of a transition row (bf16 elements)

struct PersistParams {
  int R, gamma, V, n_tiles;
  float invT;
  const bf16_t *U;      // [R][gamma][V]
  const bf16_t *W1;     // [V][256]
  const bf16_t *W2;     // column-major 256 x V
  const int32_t *x0;    // [R]
  uint64_t *tiles;      // [2][R][n_tiles]: partial words of steps of each parity
  uint64_t *pub;        // [R]: (k << 32) | x_k, the last published draw
  SampleParams sp;      // x, q_stats, q_x, head, forcing, err (A_cur, a_tokens unused)
  int32_t *err;
};

template <int NT>
struct PersistLds {
  bf16_t rows[kPRows * kPPitch];                    // A_k, one row per request
  int tok[kPRows];                                   // x_{k-1} of every request
  u32x4 w2l[kPKS * 4 * kWave];                       // W2 of the last tile slot, per lane
  float2 part[kPRows][NT][4];                        // (max of v, sum) per row, tile, wave
  bf16_t own[2][kPPitch];                            // chunked: A_k of this workgroup's request
                                                     // in a chunk, by chunk parity
  SampleLds sl;
  int abort;
};

// The draws x_step of requests [r0, r1) into sh.tok[row - r0], once
// published (thread t polls requests r0 + t, r0 + t + kBlock, ...).  Returns
// false (and flags the error) if a poll ran out.
template <int NT>
__device__ __forceinline__ bool wait_tokens(const PersistParams &p, PersistLds<NT> &sh, int step,
                                            int r0, int r1) {
  bool ok = true;
  for (int row = r0 + threadIdx.x; row < r1; row += kBlock) {
    uint64_t v = ld_coherent(p.pub + row);
    for (int spins = 0; (int64_t)(v >> 32) < step; ++spins) {
      if (spins > kSpinLimit) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      v = ld_coherent(p.pub + row);
    }
    sh.tok[row - r0] = (int)min((uint32_t)v, (uint32_t)(p.V - 1));  // in range when published
  }
  if (!ok) {
    sh.abort = 1;
    flag_error(p.err, kErrSync);
  }
  __syncthreads();
  return sh.abort == 0;
}

// The anchors x_0 (validated) of requests [r0, r1) into sh.tok[row - r0]
// (step 1's transition rows are W1[x_0]); thread t takes requests r0 + t,
// r0 + t + kBlock, ...
template <int NT>
__device__ __forceinline__ void anchor_tokens(const PersistParams &p, PersistLds<NT> &sh, int r0,
                                              int r1) {
  bool bad = false;
  for (int row = r0 + threadIdx.x; row < r1; row += kBlock) {
    int tok = p.x0[row];
    if (tok < 0 || tok >= p.V) {
      bad = true;
      tok = tok < 0 ? 0 : p.V - 1;
    }
    sh.tok[row - r0] = tok;
  }
  if (bad) flag_error(p.err, kErrToken);
  __syncthreads();
}

// NT: vocabulary tiles per workgroup (at most); kMask: V is not a multiple of
// the tile width, so the last tile has columns past V.
template <int NT, bool kMask, bool kChunked>
__global__ __launch_bounds__(kBlock, 1) void draft_persistent_kernel(PersistParams p) {
  __shared__ __align__(16) PersistLds<NT> sh;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int G = gridDim.x, g = blockIdx.x;
  const int R = p.R, gamma = p.gamma, V = p.V, nT = p.n_tiles;
  const int t0 = (int)((int64_t)g * nT / G), t1 = (int)((int64_t)(g + 1) * nT / G);
  const int ntl = t1 - t0;  // <= NT (checked by the host)
  const int nrb = (R + kRowsPerWave - 1) / kRowsPerWave;
  const float invT = p.invT, cl = invT * kLog2e;
  const int m = lane & 31, half = lane >> 5;
  if (tid == 0) sh.abort = 0;

  // ---- W2 of this wave's blocks: block `wave` of tiles t0 .. t0 + NT - 1
  //      (a slot past the range, or a column past V, reads a clamped column;
  //      its results are dropped); slots 0 .. NT - 2 in registers, the last
  //      slot in LDS, where each lane keeps its own 16-byte pieces
  constexpr int kPRegTiles = NT - 1;
  u16x8 w2r[kPRegTiles][kPKS];
  {
    u16x8 w2f[kPKS];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int col = min((t0 + i) * kTileN + wave * kBlockCols + block_col_of_m(m), V - 1);
      const bf16_t *src = p.W2 + (int64_t)col * kMaxRank + half * 8;
#pragma unroll
      for (int ks = 0; ks < kPKS; ++ks) {
        const u16x8 v = *reinterpret_cast<const u16x8 *>(src + ks * 16);
        if (i < kPRegTiles) w2r[i < kPRegTiles ? i : 0][ks] = v;
        else w2f[ks] = v;
      }
    }
    // keep the operand in the accumulation registers (the products read it
    // there directly; left to itself the allocator moved parts of it to
    // scratch or copied it into vector registers before every product).  The
    // pins come after every load is in flight: a pin consumes its value, so a
    // pin after each load made the loads one round trip each.
#pragma unroll
    for (int i = 0; i < kPRegTiles; ++i)
#pragma unroll
      for (int ks = 0; ks < kPKS; ++ks) asm volatile("" : "+a"(w2r[i][ks]));
#pragma unroll
    for (int ks = 0; ks < kPKS; ++ks)
      sh.w2l[(ks * 4 + wave) * kWave + lane] = __builtin_bit_cast(u32x4, w2f[ks]);
  }

  // ---- U of item (row block rb, tile slot i) at step k: this lane's 16
  //      columns of its row, two 16-byte pieces, each clamped on its own (a
  //      piece is wholly inside or outside [0, V) because V % 8 == 0, but the
  //      two pieces of a lane straddle V when V % 16 == 8)
  struct UPiece { u32x4 a, b; };
  auto load_u = [&](int k, int rb, int i, int m, int half) __attribute__((always_inline)) {
    const int rho = min(rb * kRowsPerWave + m, R - 1);
    const int c0 = (t0 + i) * kTileN + wave * kBlockCols + half * 16;
    const bf16_t *row = p.U + ((int64_t)rho * gamma + (k - 1)) * V;
    UPiece u;
    if constexpr (kMask) {
      u.a = *reinterpret_cast<const u32x4 *>(row + min(c0, V - 8));
      u.b = *reinterpret_cast<const u32x4 *>(row + min(c0 + 8, V - 8));
    } else {  // V % 128 == 0: a lane's 16 columns are all inside or all outside
      const int cc = min(c0, V - 16);
      u.a = *reinterpret_cast<const u32x4 *>(row + cc);
      u.b = *reinterpret_cast<const u32x4 *>(row + cc + 8);
    }
    return u;
  };
  // the U ring holds one row block of items ahead (item i is tile slot i)
  UPiece ur[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) ur[i] = load_u(1, 0, i, m, half);

  // this workgroup's requests are rho = g, g + G, ...; the first one at or
  // after row r0
  auto first_own = [&](int r0) __attribute__((always_inline)) {
    return kChunked ? r0 + ((g - r0) % G + G) % G : g;
  };
  // ---- 4. draws of this workgroup's requests among rows [r0, r1) at step k;
  //      false when a wait ran out
  auto draws = [&](int k, int ch, int r0, int r1) __attribute__((always_inline)) {
    uint64_t *tiles = p.tiles + (int64_t)(k & 1) * R * nT;
    for (int rho = first_own(r0); rho < r1; rho += G) {
      const PersistIo io{tiles, p.pub, &sh.abort};
      bf16_t *arow = kChunked ? sh.own[ch & 1] : sh.rows + rho * kPPitch;
      // (a thread index made opaque in every draw: 1.7% faster at R = 128,
      // and the chunked kernel held no address in scratch across the loop)
      if (!sample_row<bf16_t, true, kPKS, true>(p.sp, k, nullptr, rho, arow, false, sh.sl, io))
        return false;
      __syncthreads();  // LDS of the draw is reused by the next request
    }
    return true;
  };
  // requests in chunks of kPRows (one chunk unless kChunked): the draws of a
  // chunk run after the next chunk's products, so every workgroup's partials
  // of the chunk are long written when its samplers poll them, and the draws
  // of step k - 1 are out before step k reaches the chunk
  const int n_chunks = kChunked ? (R + kPRows - 1) / kPRows : 1;

  for (int k = 1; k <= gamma; ++k) {
    for (int ch = 0; ch < n_chunks; ++ch) {
      const int r0 = kChunked ? ch * kPRows : 0, r1 = kChunked ? min(R, r0 + kPRows) : R;
      const int rb0 = kChunked ? r0 / kRowsPerWave : 0;
      const int rb1 = kChunked ? (r1 + kRowsPerWave - 1) / kRowsPerWave : nrb;
      // the thread's index, opaque to the compiler once per step (and chunk):
      // addresses derived from it are formed again every step instead of
      // being held across the whole loop (where they went to scratch, and
      // every reload waited for all loads in flight, the U prefetch included)
      int tid_k = tid;
      asm volatile("" : "+v"(tid_k));
      const int lane_k = tid_k & (kWave - 1), m_k = lane_k & 31, half_k = lane_k >> 5;
      // ---- 1. transition rows of the chunk at step k into LDS: W1[x_{k-1}],
      //      x_0 the anchors, then the draws the samplers published (rows
      //      past R are zero)
      if (k == 1) anchor_tokens<NT>(p, sh, r0, r1);
      else if (!wait_tokens<NT>(p, sh, k - 1, r0, r1)) return;
      {
        // thread t: 16-byte piece t % 32 of rows t / 32 + 8 j: every load in
        // flight before the first LDS store, and no branch between them (a
        // row past R reads row R - 1 and stores zeros)
        constexpr int kPieces = kMaxRank * 2 / 16;  // 16-byte pieces per row
        constexpr int kIt = kPRows * kPieces / kBlock;
        const int off = (tid_k % kPieces) * 8, row0 = tid_k / kPieces;
        u32x4 v[kIt];
#pragma unroll
        for (int j = 0; j < kIt; ++j) {
          const int row = min(row0 + j * (kBlock / kPieces), r1 - r0 - 1);
          v[j] = *reinterpret_cast<const u32x4 *>(p.W1 + (int64_t)sh.tok[row] * kMaxRank + off);
        }
#pragma unroll
        for (int j = 0; j < kIt; ++j) {
          const int row = row0 + j * (kBlock / kPieces);
          const u32x4 z = {0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4 *>(sh.rows + row * kPPitch + off) = row < r1 - r0 ? v[j] : z;
        }
      }
      __syncthreads();
      if constexpr (kChunked) {
        // this workgroup's request of the chunk (at most one: G >= kPRows)
        // keeps its row until its draw, after the next chunk's rows replace
        // these
        const int mine = first_own(r0);
        constexpr int kPieces = kMaxRank * 2 / 16;
        if (mine < r1 && tid_k < kPieces)
          *reinterpret_cast<u32x4 *>(sh.own[ch & 1] + tid_k * 8) =
              *reinterpret_cast<const u32x4 *>(sh.rows + (mine - r0) * kPPitch + tid_k * 8);
      }

      // ---- 2. products and epilogues, row block by row block.  Item i of a
      //      row block is tile slot i: the register-held slots first (the first
      //      products wait only for the rows' LDS reads), the LDS-held slot last
      for (int rb = rb0; rb < rb1; ++rb) {
        const int rbl = rb - rb0;  // row block within the chunk (LDS rows and partials)
        u16x8 bfr[kPKS];
        {
          const bf16_t *rowp = sh.rows + (rbl * kRowsPerWave + m_k) * kPPitch + half_k * 8;
  #pragma unroll
          for (int ks = 0; ks < kPKS; ++ks) bfr[ks] = *reinterpret_cast<const u16x8 *>(rowp + ks * 16);
        }
        // products of item i < NT - 1 (W2 from registers)
        auto mma = [&](int i) __attribute__((always_inline)) {
          floatx16 acc;
  #pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  #pragma unroll
          for (int ks = 0; ks < kPKS; ++ks) acc = mfma16<true>(w2r[i < NT - 1 ? i : 0][ks], bfr[ks], acc);
          return acc;
        };
        // the next U of an item: the same tile slot one row block later, or
        // the first row block of the next step (the last step reloads its own)
        const bool last_rb = rb + 1 == nrb;
        const int k_next = last_rb ? min(k + 1, gamma) : k;
        const int rb_next = last_rb ? 0 : rb + 1;
        auto epilogue = [&](int i, const floatx16 &acc) __attribute__((always_inline)) {
          const int sl = i;
          float v[16];
          unpack16(ur[i].a, (bf16_t *)nullptr, v);
          unpack16(ur[i].b, (bf16_t *)nullptr, v + 8);
          const int c0 = (t0 + sl) * kTileN + wave * kBlockCols + half_k * 16;
  #pragma unroll
          for (int c = 0; c < 16; ++c) {
            v[c] = acc[c] + v[c];  // z * T: the product kernels' exact expression
            if (kMask && c0 + c >= V) v[c] = -INFINITY;
          }
          ur[i] = load_u(k_next, rb_next, sl, m_k, half_k);
          float bm = v[0];
  #pragma unroll
          for (int c = 1; c < 16; ++c) bm = fmaxf(bm, v[c]);
          float s = 0.0f;
          if (!kMask || bm != -INFINITY) {
            // (v - max) first: exact near the maximum, where the mass is; one
            // fused multiply-add with -max * log2(e) / T rounded would shift
            // every term by up to half an ulp of that product (~1e-6 relative
            // at |max| ~ 40), enough to lift a q(x) near 1 above 1 + 1e-6
  #pragma unroll
            for (int c = 0; c < 16; ++c) s += exp2_fast((v[c] - bm) * cl);
          }
          // the other 16 columns of the row are in lane l ^ 32
          // (both lanes of a row form the same sum: their operands are swapped
          // and addition is commutative, so both store the same value)
          const float om = half_swap(bm), os = half_swap(s);
          const float M = fmaxf(bm, om);
          const float S2 = s * exp2_fast((bm - M) * cl) + os * exp2_fast((om - M) * cl);
          sh.part[rbl * kRowsPerWave + m_k][sl][wave] = make_float2(M, M != -INFINITY ? S2 : 0.0f);
        };
        // item 0 from registers: its products wait only for the rows' reads;
        // the LDS-held slot's operands are read one item ahead of its products
        floatx16 acc0 = mma(0), acc1;
        u16x8 w2f[kPKS];
  #pragma unroll
        for (int i = 0; i < NT; ++i) {
          if (i + 2 == NT) {
  #pragma unroll
            for (int ks = 0; ks < kPKS; ++ks)
              w2f[ks] = __builtin_bit_cast(u16x8, sh.w2l[(ks * 4 + wave) * kWave + lane_k]);
          }
          if (i + 1 < NT) {
            floatx16 nx;
            if (i + 1 < NT - 1) {
              nx = mma(i + 1);
            } else {
  #pragma unroll
              for (int e = 0; e < 16; ++e) nx[e] = 0.0f;
  #pragma unroll
              for (int ks = 0; ks < kPKS; ++ks) nx = mfma16<true>(w2f[ks], bfr[ks], nx);
            }
            if (i & 1) acc0 = nx;
            else acc1 = nx;
          }
          epilogue(i, (i & 1) ? acc1 : acc0);
          // the epilogue of item i issues while the products of item i + 1 run
  #pragma unroll
          for (int j = 0; j < 16; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix instruction
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // then six vector ALU
          }
          // nothing moves across items: hoisting the next items' loads would
          // run out of registers
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();

      // ---- 3. tile partials (fixed wave order) into the step's half
      uint64_t *tiles = p.tiles + (int64_t)(k & 1) * R * nT;
      for (int q = tid_k; q < (r1 - r0) * ntl; q += kBlock) {
        const int rl = q / ntl, i = q - rl * ntl;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.part[rl][i][w].x);
        float S = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float2 pw = sh.part[rl][i][w];
            if (pw.x != -INFINITY) S += pw.y * exp2_fast((pw.x - M) * cl);
          }
        }
        // max z = (max of acc + u) / T exactly (rounding is monotone)
        uint64_t word = __builtin_bit_cast(uint64_t, make_float2(M * invT, S));
        if (word == kTileEmpty) word = kTileEmpty - 1;  // another NaN: still read as non-finite
        st_coherent(tiles + (int64_t)(r0 + rl) * nT + t0 + i, word);
      }

      // ---- 4. draws: this chunk's (one chunk), else the previous chunk's
      if (!kChunked) {
        if (!draws(k, ch, r0, r1)) return;
      } else if (ch > 0) {
        if (!draws(k, ch - 1, r0 - kPRows, r0)) return;
      }
    }
    if (kChunked && !draws(k, n_chunks - 1, (n_chunks - 1) * kPRows, R)) return;
    // ---- 5. the next step waits for the draws of this one (step 1 above)
  }
}

// Before each launch: every partial word empty, every draw unpublished.
__global__ void persist_clear_kernel(uint64_t *tiles, int n_words, uint64_t *pub, int R) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += gridDim.x * blockDim.x)
    tiles[i] = kTileEmpty;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < R; i += gridDim.x * blockDim.x) pub[i] = 0;
}

// Launch shape of the persistent draft, or false when the shape does not fit
// it (then the per-step kernels run).  One workgroup per compute unit; each
// holds at most 5 tiles (640 columns) of W2.  Past kPRows requests the rows
// go in chunks of kPRows (at most kMaxChunks), which needs a grid of at least
// kPRows workgroups: each then draws at most one request of a chunk.
constexpr int kMaxChunks = 4;
bool persistent_draft_shape(int R, int V, int r, bool bf16, int *grid, int *nt) {
  if (!bf16 || r != kMaxRank || R > kMaxChunks * kPRows || V < kTileN) return false;
  const int n_tiles = (V + kTileN - 1) / kTileN;
  const int G = n_tiles < kComputeUnits ? n_tiles : kComputeUnits;
  const int per = (n_tiles + G - 1) / G;
  if (per > 5 || (R > kPRows && G < kPRows)) return false;
  *grid = G;
  *nt = per <= 4 ? 4 : 5;
  return true;
}

template <int NT, bool kMask, bool kChunked>
static hipError_t launch_persistent_t(PersistParams &pp, int G, hipStream_t stream) {
  void *args[] = {&pp};
  hipEvent_t start = nullptr, stop = nullptr;
  if (trace_on()) trace_events("draft_persistent", &start, &stop);
  if (start) (void)hipEventRecord(start, stream);
  hipError_t e = hipLaunchCooperativeKernel(
      reinterpret_cast<const void *>(&draft_persistent_kernel<NT, kMask, kChunked>), dim3(G), dim3(kBlock),
      args, 0, stream);
  if (stop) (void)hipEventRecord(stop, stream);
  return e;
}

hipError_t launch_draft_persistent(const DraftLaunch &L, int G, int nt, const SampleParams &sp,
                                   hipStream_t stream) {
  const int n_tiles = (L.V + kTileN - 1) / kTileN;
  PersistParams pp{};
  pp.R = L.R; pp.gamma = L.gamma; pp.V = L.V; pp.n_tiles = n_tiles; pp.invT = L.invT;
  pp.U = reinterpret_cast<const bf16_t *>(L.U);
  pp.W1 = reinterpret_cast<const bf16_t *>(L.W1);
  pp.W2 = reinterpret_cast<const bf16_t *>(L.W2);
  pp.x0 = L.x0;
  pp.tiles = reinterpret_cast<uint64_t *>(L.tile_stats);  // [2][R][n_tiles]
  pp.pub = L.pub;
  pp.sp = sp;
  pp.err = L.err;
  const int n_words = 2 * L.R * n_tiles;
  DSPARK_LAUNCH("persist_clear", stream, persist_clear_kernel,
                std::min((n_words + 255) / 256, 4 * kComputeUnits), 256, pp.tiles, n_words, L.pub,
                L.R);
  const bool mask = L.V % kTileN != 0;
  if (L.R > kPRows) {
    if (nt == 4) return mask ? launch_persistent_t<4, true, true>(pp, G, stream)
                             : launch_persistent_t<4, false, true>(pp, G, stream);
    return mask ? launch_persistent_t<5, true, true>(pp, G, stream)
                : launch_persistent_t<5, false, true>(pp, G, stream);
  }
  if (nt == 4) return mask ? launch_persistent_t<4, true, false>(pp, G, stream)
                           : launch_persistent_t<4, false, false>(pp, G, stream);
  return mask ? launch_persistent_t<5, true, false>(pp, G, stream)
              : launch_persistent_t<5, false, false>(pp, G, stream);
}

}  // namespace dspark
