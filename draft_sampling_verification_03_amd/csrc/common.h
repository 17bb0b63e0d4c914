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
constexpr int kMaxTiles = 2048;      // V <= 262144
constexpr int kMaxRank = 256;

// sticky device error bits (mirrors dspark.h)
constexpr int kErrToken = 1, kErrConfidence = 2, kErrLength = 4, kErrNonFinite = 8;

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

// e^x on the transcendental unit: 2^(x log2 e).  Every kernel uses this one
// function, so equal arguments give equal results everywhere.
__device__ __forceinline__ float fexp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ void flag_error(int32_t *err, int bits) {
  if (err) atomicOr(err, bits);
}

// ------------------------------------------------------------------ reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
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

// inclusive scan over the wave, lane order
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    float t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

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

// Bias main loop for one wave: acc[mb][nb] (32 x 32 blocks) += A * B^T over
// K = r, where
//   A rows come from LDS:   row (a_row0 + 32 mb + lane % 32), pitch a_pitch
//                           (a_pitch = 0 makes every row read the same data)
//   B rows from global:     W2 column v = b_col0 + 32 nb + lane % 32 (r contiguous
//                           coefficients); columns >= V read as zero
// K advances in steps of 16 (bf16: one 32x32x16 MFMA) in increasing order, and
// each accumulator starts at zero.  Output element (row i, column j) of a block
// is in lane (j + 32 * ((i / 4) % 2)), register 4 * (i / 8) + i % 4.
template <int WMB, int WNB>
__device__ __forceinline__ void bias_mainloop(const bf16_t *ldsA, int a_pitch, int a_row0,
                                              const bf16_t *W2, int V, int r, int b_col0,
                                              floatx16 (&acc)[WMB][WNB]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int kq = (lane >> 5) * 8;
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.0f;
  const bf16_t *bptr[WNB];
  bool bvalid[WNB];
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb) {
    const int v = b_col0 + 32 * nb + (lane & 31);
    bvalid[nb] = v < V;
    bptr[nb] = W2 + (int64_t)(bvalid[nb] ? v : 0) * r + kq;
  }
  const u16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
  u16x8 bnext[WNB];
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb)
    bnext[nb] = bvalid[nb] ? *reinterpret_cast<const u16x8 *>(bptr[nb]) : zero;
  for (int k0 = 0; k0 < r; k0 += 16) {
    u16x8 bcur[WNB];
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) bcur[nb] = bnext[nb];
    if (k0 + 16 < r) {
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
        bnext[nb] = bvalid[nb] ? *reinterpret_cast<const u16x8 *>(bptr[nb] + k0 + 16) : zero;
    }
    u16x8 a[WMB];
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
      a[mb] = *reinterpret_cast<const u16x8 *>(ldsA + (a_row0 + 32 * mb + (lane & 31)) * a_pitch +
                                               k0 + kq);
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a[mb]), __builtin_bit_cast(bf16x8, bcur[nb]), acc[mb][nb],
            0, 0, 0);
  }
}

// fp32 variant: one 32x32x2 fp32 MFMA per K step of 2, K order increasing.
template <int WMB, int WNB>
__device__ __forceinline__ void bias_mainloop(const float *ldsA, int a_pitch, int a_row0,
                                              const float *W2, int V, int r, int b_col0,
                                              floatx16 (&acc)[WMB][WNB]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int kq = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.0f;
  const float *bptr[WNB];
  bool bvalid[WNB];
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb) {
    const int v = b_col0 + 32 * nb + (lane & 31);
    bvalid[nb] = v < V;
    bptr[nb] = W2 + (int64_t)(bvalid[nb] ? v : 0) * r + kq;
  }
  for (int k0 = 0; k0 < r; k0 += 2) {
    float b[WNB], a[WMB];
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) b[nb] = bvalid[nb] ? bptr[nb][k0] : 0.0f;
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
      a[mb] = ldsA[(a_row0 + 32 * mb + (lane & 31)) * a_pitch + k0 + kq];
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
  }
}

// Row i (0..31) of a 32x32 accumulator block: which lane half and register.
__device__ __forceinline__ int acc_half_of_row(int i) { return (i >> 2) & 1; }
__device__ __forceinline__ int acc_reg_of_row(int i) { return 4 * (i >> 3) + (i & 3); }

// Copy one r-wide row (W1[x]) from global memory to LDS with 16-byte pieces.
template <typename T>
__device__ __forceinline__ void copy_row_to_lds(T *dst, const T *src, int r, int piece,
                                                int n_pieces_per_row) {
  constexpr int kPer = Elem<T>::kPerVec;
  (void)n_pieces_per_row;
  *reinterpret_cast<uint4 *>(dst + piece * kPer) =
      *reinterpret_cast<const uint4 *>(src + piece * kPer);
  (void)r;
}

}  // namespace dspark
