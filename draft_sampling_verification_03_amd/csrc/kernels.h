// Launch descriptors shared by the host-side ABI layer (abi.cpp) and the
// kernel translation units.  Plain structs of device pointers and sizes; the
// ABI layer has validated every field before a launch function is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

constexpr int kComputeUnits = 256;  // MI355X

// bytes 0..3 of every workspace hold the sticky error word
constexpr size_t kWsHeader = 256;

// recurrent head: the transition row of step k is the GRU state s_k
struct RnnHead {
  const void *G_E;    // [V][3r] token input projection
  const float *G_h;   // [R][gamma][3r] hidden-state input projection (input biases folded in)
  const void *W_hh;   // [r][3r] column-major recurrent weights
  const float *b_hh;  // [3r]
  const float *s0;    // [R][r] or NULL
  float *s;           // [R][gamma][r] states (fp32)
  void *A;            // [gamma][R][r] states in the weights' element type
};

struct DraftLaunch {
  int R, gamma, V, r, d;
  bool bf16;
  float invT;
  const void *U, *W1, *W2;
  const int32_t *x0;
  const void *h;
  const float *w_conf;
  float b_conf;
  const float *conf_temp;  // [gamma] or NULL
  uint64_t seed, round;
  int32_t *x;
  float *q_stats, *q_x, *c;
  const int32_t *x_force;  // [R][gamma] labels (teacher forcing) or NULL
  float *logq_x;           // [R][gamma] or NULL
  const RnnHead *rnn;      // recurrent head instead of the W1 table, or NULL
  // workspace pieces
  int32_t *err;
  float2 *tile_stats;  // [2][R][n_tiles]: the per-step kernels use the first half, the
                       // persistent draft both, by the parity of the step
  float *sh;           // [R][gamma]
  void *A0, *A1;       // [R][r] each: transition rows of the current and next step
  uint64_t *pub;       // [R]: draws published by the persistent draft
};

struct ScheduleLaunch {
  int R, gamma, mode;
  float threshold;  // THRESHOLD mode
  const float *c, *c_prev2;
  const double *SPS;
  int32_t *ell, *row_offset;
  float *a;
  int32_t *n_admitted;
  double *theta;
  int32_t *err;
};

struct VerifyLaunch {
  int R, gamma, V, r, rows_capacity;
  bool bf16;
  float invT;
  const int32_t *ell, *row_offset;
  const void *P, *U, *W1, *W2;
  const int32_t *x0, *x;
  const float *q_stats, *q_x;
  uint64_t seed, round;
  int32_t *n_acc, *y;
  float *c_star;
  // workspace pieces
  int32_t *err;
  float2 *p_chunks;      // [rows_capacity][4]
  float2 *bonus_tiles;   // [R][n_tiles]
  float2 *pair_partials; // [R * gamma][n_tiles]
  int4 *row_map;         // [R * gamma]
  float4 *row_stats;     // [R * gamma]: (m_q, log2 S_q, m_p, log2 S_p) of the compact rows
  void *A_rows;          // [R * gamma][r] transition rows of the compact rows
  const void *A_given;   // [gamma][R][r] given transition rows (recurrent head), or NULL
};

struct OverlapLaunch {
  int n_rows, V;
  bool bf16;
  float invT;
  const void *P, *Q;
  const float *p_stats, *q_stats;
  float *c_star;
  int32_t *err;
  float2 *p_chunks, *q_chunks;  // [n_rows][4] each
  float *partial;               // [n_rows][4]
};

struct TrainLaunch {
  int R, gamma;
  DraftLaunch draft;    // teacher-forced: x_force = labels, logq_x set
  VerifyLaunch verify;  // every position admitted; its c_star feeds the losses
  int32_t *ell, *row_offset;  // [R], [R + 1]: filled on the device
  const float *c;
  double a_ce, a_tv, a_conf;
  float *per_pos;  // [3][R][gamma] or NULL
  double *totals;  // [4]
  double *req_sums;  // [R][3]: each request's weighted (CE, L1, BCE) means
};

hipError_t launch_draft(const DraftLaunch &L, hipStream_t stream);
hipError_t launch_schedule(const ScheduleLaunch &L, hipStream_t stream);
hipError_t launch_verify(const VerifyLaunch &L, hipStream_t stream);
hipError_t launch_overlap(const OverlapLaunch &L, hipStream_t stream);
hipError_t launch_train(const TrainLaunch &L, hipStream_t stream);
hipError_t launch_clear_error(int32_t *err, hipStream_t stream);

// workspace layouts (bytes), each piece 256-byte aligned
inline size_t ws_align(size_t b) { return (b + 255) & ~(size_t)255; }
inline int n_tiles_of(int V) { return (V + 127) / 128; }

// a transition row W1[x] holds r <= 256 bf16 or r <= 128 fp32 values: <= 512 bytes
constexpr size_t kMaxRowBytes = 512;

inline size_t draft_ws_bytes(int R, int gamma, int V) {
  return kWsHeader + ws_align((size_t)2 * R * n_tiles_of(V) * 8) + ws_align((size_t)R * gamma * 4) +
         2 * ws_align((size_t)R * kMaxRowBytes) + ws_align((size_t)R * 8);
}
inline size_t schedule_ws_bytes(int R, int gamma) {
  (void)R; (void)gamma;
  return kWsHeader;
}
inline size_t verify_ws_bytes(int R, int gamma, int V, int rows_capacity) {
  return kWsHeader + ws_align((size_t)rows_capacity * 4 * 8) +
         ws_align((size_t)R * n_tiles_of(V) * 8) + ws_align((size_t)R * gamma * n_tiles_of(V) * 8) +
         2 * ws_align((size_t)R * gamma * 16) + ws_align((size_t)R * gamma * kMaxRowBytes);
}
inline size_t train_ws_bytes(int R, int gamma, int V) {
  const size_t n = (size_t)R * gamma;
  return draft_ws_bytes(R, gamma, V) + verify_ws_bytes(R, gamma, V, R * (gamma + 1)) +
         4 * ws_align(n * 4) + ws_align(n * 8) + 3 * ws_align(((size_t)R + 1) * 4) +
         ws_align((size_t)R * (gamma + 1) * 4) + ws_align((size_t)R * 3 * 8);
}
inline size_t overlap_ws_bytes(int n_rows, int V) {
  (void)V;
  return kWsHeader + 2 * ws_align((size_t)n_rows * 4 * 8) + ws_align((size_t)n_rows * 4 * 4);
}

}  // namespace dspark
