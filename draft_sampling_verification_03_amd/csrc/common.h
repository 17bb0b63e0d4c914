// Device-side building blocks of the DSpark hot path on gfx950 (CDNA4).
//
// - bf16 / fp32 element access with 16-byte vector loads
// - exp on the transcendental unit
// - wave (64 lanes) and workgroup reductions and scans in a fixed order, so
//   every result is reproducible bit for bit (no floating-point atomics)
// - Philox4x64-10 uniforms (Salmon et al., SC'11)
// - the matrix-core main loop that forms the Markov bias W1[x] W2 for a tile of
//   rows and 128 vocabulary columns.  Every kernel that needs z = U + bias
//   calls this one loop, with the same instruction and the same K order, so a
//   recomputed z is bit-identical to the z the draft sampled from.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

constexpr int kWave = 64;
constexpr int kBlock = 256;          // threads of every workgroup
constexpr int kTileN = 128;          // vocabulary columns per tile
constexpr int kXcds = 8;             // accelerator complex dies, each with its own L2
constexpr int kMaxTiles = 2048;      // V <= 262144
constexpr int kMaxRank = 256;
constexpr int kMaxGamma = 64;       // draft positions per request

// sticky device error bits (mirrors dspark.h)
constexpr int kErrToken = 1, kErrConfidence = 2, kErrLength = 4, kErrNonFinite = 8, kErrSync = 16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// binary32 -> bfloat16, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ void store_elem(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(bf16_t *p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }

// element type traits: T = float (DSPARK_F32) or bf16_t (DSPARK_BF16)
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerVec = 4;  // elements per 16-byte load
  __device__ static __forceinline__ float at(const float *p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void vec(const float *p, int64_t i, float *out) {
    floatx4 v = *reinterpret_cast<const floatx4 *>(p + i);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ float at(const bf16_t *p, int64_t i) {
    return bf16_to_f32(p[i].bits);
  }
  __device__ static __forceinline__ void vec(const bf16_t *p, int64_t i, float *out) {
    u16x8 v = *reinterpret_cast<const u16x8 *>(p + i);
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = bf16_to_f32(v[j]);
  }
};

// 16 bytes of a stream that is read once (logit rows): a non-temporal load, so
// it does not displace data that is re-read (the W2 factor) from the caches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ld_stream4(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// e^x on the transcendental unit: 2^(x log2 e).  Every kernel uses this one
// function, so equal arguments give equal results everywhere.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
// 2^x and log2(x) on the transcendental unit
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Order LDS accesses of the lanes of one wave (LDS executes a wave's accesses
// in issue order; this keeps the compiler from reordering them).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Device-coherent 8-byte accesses (agent-scope relaxed atomics): data that one
// workgroup writes and workgroups on other XCDs read within the same kernel
// travel this way, so no L2 writeback or invalidation is needed around them.
__device__ __forceinline__ void st_coherent(void *p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coherent(const void *p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void flag_error(int32_t *err, int bits) {
  if (err) atomicOr(err, bits);
}

// ------------------------------------------------------------------ reductions
// Max and min over the wave: DPP steps within each row of 16 lanes (xor 1,
// xor 2, then the mirrors within 8 and 16 lanes pair every lane with one of
// the other half), after which each row is uniform; the four rows are read
// back as scalars.  Exact in any order, and no LDS round trip per step.
template <typename Op> __device__ __forceinline__ int dpp_rows_reduce(int v, Op op) {
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));  // row_mirror
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return op(op(a, b), op(c, d));
}
__device__ __forceinline__ float wave_max(float v) {
  return __int_as_float(dpp_rows_reduce(__float_as_int(v), [](int x, int y) {
    return __float_as_int(fmaxf(__int_as_float(x), __int_as_float(y)));
  }));
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
  return dpp_rows_reduce(v, [](int x, int y) { return min(x, y); });
}
__device__ __forceinline__ int wave_max_int(int v) {
  return dpp_rows_reduce(v, [](int x, int y) { return max(x, y); });
}
// reductions over groups of G consecutive lanes (G a power of two <= 64)
template <int G> __device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
template <int G> __device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// inclusive scan over the wave, lane order: Hillis-Steele steps within each
// row of 16 lanes by DPP row shifts (a lane without a source adds 0), then
// the totals of rows 0 and 2 are added to rows 1 and 3 and the total of rows
// 0-1 to rows 2 and 3 (DPP row broadcasts).  Fixed order: deterministic.
template <int kCtrl, int kRowMask> __device__ __forceinline__ float dpp_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, true));
}
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  v += dpp_or_zero<0x111, 0xF>(v);  // row_shr:1
  v += dpp_or_zero<0x112, 0xF>(v);  // row_shr:2
  v += dpp_or_zero<0x114, 0xF>(v);  // row_shr:4
  v += dpp_or_zero<0x118, 0xF>(v);  // row_shr:8
  v += dpp_or_zero<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_or_zero<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
// the value of the previous lane (0 in lane 0): DPP wave_shr:1
__device__ __forceinline__ float wave_prev_lane(float v) { return dpp_or_zero<0x138, 0xF>(v); }

// Workgroup-wide reductions (kBlock threads); `scratch` holds >= 4 floats.
__device__ __forceinline__ float block_max(float v, float *scratch) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_sum(float v, float *scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  float r = ((scratch[0] + scratch[1]) + scratch[2]) + scratch[3];
  __syncthreads();
  return r;
}
__device__ __forceinline__ int block_min_int(int v, int *scratch) {
  v = wave_min_int(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  int r = min(min(scratch[0], scratch[1]), min(scratch[2], scratch[3]));
  __syncthreads();
  return r;
}
__device__ __forceinline__ int block_max_int(int v, int *scratch) {
  v = wave_max_int(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  int r = max(max(scratch[0], scratch[1]), max(scratch[2], scratch[3]));
  __syncthreads();
  return r;
}
// Exclusive scan over the workgroup in thread order; returns the thread's
// exclusive prefix and writes the total.  `scratch` holds >= 4 floats.
__device__ __forceinline__ float block_exclusive_scan(float v, float *scratch, float *total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  float inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane == kWave - 1) scratch[w] = inc;
  __syncthreads();
  float before = 0.0f;
  for (int i = 0; i < w; ++i) before += scratch[i];
  *total = ((scratch[0] + scratch[1]) + scratch[2]) + scratch[3];
  __syncthreads();
  return before + (inc - v);
}

// ------------------------------------------------------------------ Philox
// Philox4x64-10: per round (X0, X1, X2, X3) -> (hi(M1 X2) ^ X1 ^ K0, lo(M1 X2),
// hi(M0 X0) ^ X3 ^ K1, lo(M0 X0)); the key advances by the Weyl constants.
struct Philox4x64 {
  uint64_t x[4];
};
__device__ __forceinline__ Philox4x64 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                                    uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
  const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  Philox4x64 r;
  r.x[0] = c0; r.x[1] = c1; r.x[2] = c2; r.x[3] = c3;
  return r;
}
constexpr uint64_t kStreamDraft = 0, kStreamAccept = 1, kStreamFinal = 2;
// uniform on [0, 1): the top 24 bits of the first word, exact in binary32
__device__ __forceinline__ float uniform01(uint64_t seed, uint64_t round, uint64_t pos,
                                           uint64_t req, uint64_t stream) {
  Philox4x64 o = philox4x64_10(pos, req, stream, round, seed, 0);
  return (float)(uint32_t)(o.x[0] >> 40) * (1.0f / 16777216.0f);
}

// ------------------------------------------------------------ matrix cores
// LDS row pitch (elements) of an r-wide operand row: r + 16 bytes of padding,
// which spreads consecutive rows over different banks for 16-byte reads.
template <typename T> __host__ __device__ constexpr int lds_pitch(int r) {
  return r + 16 / (int)sizeof(T);
}

// Matrix-core bias product of a block of 32 A rows with 32 W2 columns, K
// advancing in increasing order (bf16: one 32x32x16 MFMA per 16; fp32: one
// 32x32x2 MFMA per 2) from a zero accumulator.  Output element (M index i,
// N index j) of a 32x32 block is in lane j + 32 ((i / 4) % 2), register
// 4 (i / 8) + i % 4.  Two operand orders are used:
//   W2 first (kW2First): the columns are the M index, entered in the order
//     block_col_of_m, the rows the N index; lane l then holds columns
//     16 (l / 32) .. +15 of row l % 32 in registers 0..15, ready for a
//     reduction over the row (the draft step);
//   rows first: the rows are the M index, the columns the N index in natural
//     order; lane l holds 16 rows of column l % 32 (the verify pass, which
//     transposes through LDS).
// Each product kernel and the recompute of its tiles issue the same sequence
// with the same operand order, so the same element always comes out of the
// same instructions.
__host__ __device__ constexpr int block_col_of_m(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}
// its inverse: the matrix row that column c of a block feeds
__host__ __device__ constexpr int block_m_of_col(int c) {
  return 8 * ((c >> 2) & 3) + 4 * (c >> 4) + (c & 3);
}
// Rows first: row i (0..31) of a 32x32 accumulator block, lane half and register.
__device__ __forceinline__ int acc_half_of_row(int i) { return (i >> 2) & 1; }
__device__ __forceinline__ int acc_reg_of_row(int i) { return 4 * (i >> 3) + (i & 3); }

template <typename T> struct BFrag;
template <> struct BFrag<bf16_t> {
  static constexpr int kSteps = kMaxRank / 16;  // K = 16 per step
  u16x8 v[kSteps];
};
template <> struct BFrag<float> {
  static constexpr int kSteps = 128 / 2;        // fp32: r <= 128, K = 2 per step
  float v[kSteps];
};

// The r coefficients of W2 column col (this lane's column) as an operand;
// a column >= V reads as zero.  Every load is issued unconditionally
// from a clamped in-bounds address (no branches between them) and masked
// afterwards.
__device__ __forceinline__ void load_bfrag(const bf16_t *W2, int V, int r, int col,
                                           BFrag<bf16_t> &b) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool ok = col < V;
  const bf16_t *ptr = W2 + (int64_t)(ok ? col : 0) * r + (lane >> 5) * 8;
  const u16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < BFrag<bf16_t>::kSteps; ++ks) {
    const int kk = ks * 16 < r ? ks * 16 : r - 16;
    const u16x8 t = *reinterpret_cast<const u16x8 *>(ptr + kk);
    b.v[ks] = (ok && ks * 16 < r) ? t : zero;
  }
}
__device__ __forceinline__ void load_bfrag(const float *W2, int V, int r, int col,
                                           BFrag<float> &b) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool ok = col < V;
  const float *ptr = W2 + (int64_t)(ok ? col : 0) * r + (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < BFrag<float>::kSteps; ++ks) {
    const int kk = ks * 2 < r ? ks * 2 : r - 2;
    const float t = ptr[kk];
    b.v[ks] = (ok && ks * 2 < r) ? t : 0.0f;
  }
}

// KS > 0 fixes the number of K steps at compile time (r = 16 KS for bf16, 2 KS
// for fp32: no branch between the matrix-core instructions, so the LDS reads
// of later steps are issued early); KS = 0 takes r at run time.  Both forms
// issue the same instructions in the same order for the same r.
template <bool kW2First, int WMB, int KS = 0>
__device__ __forceinline__ void mma_rows(const bf16_t *ldsA, int a_pitch, int a_row0, int r,
                                         const BFrag<bf16_t> &b, floatx16 (&acc)[WMB]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int kq = (lane >> 5) * 8;
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mb][e] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < (KS > 0 ? KS : BFrag<bf16_t>::kSteps); ++ks) {
    if (KS > 0 || ks * 16 < r) {
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb) {
        const u16x8 a = *reinterpret_cast<const u16x8 *>(
            ldsA + (a_row0 + 32 * mb + (lane & 31)) * a_pitch + ks * 16 + kq);
        if constexpr (kW2First)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, b.v[ks]), __builtin_bit_cast(bf16x8, a), acc[mb], 0, 0, 0);
        else
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b.v[ks]), acc[mb], 0, 0, 0);
      }
    }
  }
}
template <bool kW2First, int WMB, int KS = 0>
__device__ __forceinline__ void mma_rows(const float *ldsA, int a_pitch, int a_row0, int r,
                                         const BFrag<float> &b, floatx16 (&acc)[WMB]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int kq = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mb][e] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < (KS > 0 ? KS : BFrag<float>::kSteps); ++ks) {
    if (KS > 0 || ks * 2 < r) {
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb) {
        const float a = ldsA[(a_row0 + 32 * mb + (lane & 31)) * a_pitch + ks * 2 + kq];
        if constexpr (kW2First)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(b.v[ks], a, acc[mb], 0, 0, 0);
        else
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b.v[ks], acc[mb], 0, 0, 0);
      }
    }
  }
}

// 16 bytes of row data as floats (8 bf16 or 4 fp32)
__device__ __forceinline__ void unpack16(const uint4 &v, bf16_t *, float *out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void unpack16(const u32x4 &v, bf16_t *, float *out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(v[i] << 16);
    out[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void unpack16(const u32x4 &v, float *, float *out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
}
__device__ __forceinline__ void unpack16(const uint4 &v, float *, float *out) {
  out[0] = __uint_as_float(v.x);
  out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z);
  out[3] = __uint_as_float(v.w);
}

// Copy n elements (n <= kBlock * MAXIT) from global memory to LDS, thread-strided
// and unrolled so that every load is in flight before the first store.
template <int MAXIT, typename E>
__device__ __forceinline__ void stage_to_lds(const E *__restrict__ src, int n, E *dst) {
  E v[MAXIT];
#pragma unroll
  for (int j = 0; j < MAXIT; ++j) {
    const int i = threadIdx.x + j * kBlock;
    if (i < n) v[j] = src[i];
  }
#pragma unroll
  for (int j = 0; j < MAXIT; ++j) {
    const int i = threadIdx.x + j * kBlock;
    if (i < n) dst[i] = v[j];
  }
}

}  // namespace dspark
