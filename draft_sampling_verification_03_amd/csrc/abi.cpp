// Host side of the C ABI declared in include/dspark.h: argument validation
// (which touches no GPU, so it runs and is tested on any host), workspace
// carving, and kernel launches on the caller's stream.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/dspark.h"
#include "kernels.h"

using namespace dspark;

// Scratch of dspark_draft_noalloc: one copy per GPU, held until the process
// ends.  Host code never passes this name to a kernel (on the host it is only a
// stand-in for the symbol); it uses the device address that hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) unsigned char scratch[DSPARK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device (nullptr: not yet)

// The device address of `scratch` on the current device, looked up on the
// first call on that device.
hipError_t scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool bad_temp(float t) { return !(t > 0.0f) || !isfinite(t); }

dspark_status check_common(int R, int gamma, int V, int r, dspark_dtype dt, float temp) {
  if (dt != DSPARK_F32 && dt != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  if (R < 1 || gamma < 1 || gamma > 64) return DSPARK_ERR_SHAPE;
  if (V < 8 || V > 262144 || V % 8 != 0) return DSPARK_ERR_SHAPE;
  if (r < 16 || r % 16 != 0 || r > (dt == DSPARK_F32 ? 128 : 256)) return DSPARK_ERR_SHAPE;
  if (bad_temp(temp)) return DSPARK_ERR_VALUE;
  return DSPARK_OK;
}

dspark_status from_hip(hipError_t e) { return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP; }

char *carve(void *ws, size_t *off, size_t bytes) {
  char *p = (char *)ws + *off;
  *off += ws_align(bytes);
  return p;
}

// the draft's workspace pieces after the header, in the order draft_ws_bytes sums them
void carve_draft(void *base, size_t *off, int R, int gamma, int V, DraftLaunch &L) {
  L.tile_stats = (float2 *)carve(base, off, (size_t)2 * R * n_tiles_of(V) * 8);
  L.sh = (float *)carve(base, off, (size_t)R * gamma * 4);
  L.A0 = carve(base, off, (size_t)R * kMaxRowBytes);
  L.A1 = carve(base, off, (size_t)R * kMaxRowBytes);
  L.pub = (uint64_t *)carve(base, off, (size_t)R * 8);
}

}  // namespace

extern "C" {

const char *dspark_status_string(dspark_status s) {
  switch (s) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_NULL: return "a required pointer is NULL";
    case DSPARK_ERR_SHAPE: return "a size is outside the supported limits";
    case DSPARK_ERR_DTYPE: return "unknown element type";
    case DSPARK_ERR_VALUE: return "invalid scalar argument (temperature must be finite and > 0)";
    case DSPARK_ERR_WORKSPACE: return "workspace smaller than the *_workspace() size";
    case DSPARK_ERR_SPS_TABLE: return "SPS table missing or shorter than R*(1+gamma)+1";
    case DSPARK_ERR_MODE: return "unknown scheduler mode or missing confidences";
    case DSPARK_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case DSPARK_ERR_HIP: return "HIP launch or runtime error";
    case DSPARK_ERR_SCRATCH: return "shape needs more than the library's static scratch";
  }
  return "unknown status";
}

size_t dspark_draft_workspace(int R, int gamma, int V, int r, dspark_dtype dt) {
  (void)r; (void)dt;
  if (R < 1 || gamma < 1 || V < 1) return 0;
  return draft_ws_bytes(R, gamma, V);
}

dspark_status dspark_draft(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                           const void *U, const void *W1, const void *W2, const int32_t *x0,
                           const void *h, int d, const float *w_conf, float b_conf,
                           const float *conf_temp, uint64_t seed, uint64_t round, int32_t *x,
                           float *q_stats, float *q_x,
                           float *c, void *ws, size_t ws_bytes, hipStream_t stream) {
  dspark_status s = check_common(R, gamma, V, r, dt, temp);
  if (s != DSPARK_OK) return s;
  if (!U || !W1 || !W2 || !x0 || !x || !q_stats || !q_x || !ws) return DSPARK_ERR_NULL;
  if (h != nullptr) {
    if (!w_conf || !c) return DSPARK_ERR_NULL;
    if (d < 8 || d > 65536 || d % 8 != 0) return DSPARK_ERR_SHAPE;
    if (!isfinite(b_conf)) return DSPARK_ERR_VALUE;
    if (!aligned16(h) || !aligned16(w_conf)) return DSPARK_ERR_ALIGN;
  }
  if (!aligned16(U) || !aligned16(W1) || !aligned16(W2) || !aligned16(ws)) return DSPARK_ERR_ALIGN;
  if (ws_bytes < draft_ws_bytes(R, gamma, V)) return DSPARK_ERR_WORKSPACE;
  size_t off = 0;
  DraftLaunch L{};
  L.err = (int32_t *)carve(ws, &off, kWsHeader);
  carve_draft(ws, &off, R, gamma, V, L);
  L.R = R; L.gamma = gamma; L.V = V; L.r = r; L.d = d; L.bf16 = dt == DSPARK_BF16;
  L.invT = 1.0f / temp; L.U = U; L.W1 = W1; L.W2 = W2; L.x0 = x0; L.h = h; L.w_conf = w_conf;
  L.b_conf = b_conf; L.conf_temp = h != nullptr ? conf_temp : nullptr;
  L.seed = seed; L.round = round; L.x = x; L.q_stats = q_stats; L.q_x = q_x;
  L.c = c;
  return from_hip(launch_draft(L, stream));
}

size_t dspark_draft_noalloc_scratch(int R, int gamma, int V) {
  if (R < 1 || gamma < 1 || V < 1) return 0;
  return draft_ws_bytes(R, gamma, V) - kWsHeader;
}

dspark_status dspark_draft_noalloc(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                                   const void *U, const void *W1, const void *W2,
                                   const int32_t *x0, const void *h, int d, const float *w_conf,
                                   float b_conf, const float *conf_temp, uint64_t seed,
                                   uint64_t round, int32_t *x, float *q_stats, float *q_x,
                                   float *c, int32_t *dev_error, hipStream_t stream) {
  dspark_status s = check_common(R, gamma, V, r, dt, temp);
  if (s != DSPARK_OK) return s;
  if (!U || !W1 || !W2 || !x0 || !x || !q_stats || !q_x || !dev_error) return DSPARK_ERR_NULL;
  if (h != nullptr) {
    if (!w_conf || !c) return DSPARK_ERR_NULL;
    if (d < 8 || d > 65536 || d % 8 != 0) return DSPARK_ERR_SHAPE;
    if (!isfinite(b_conf)) return DSPARK_ERR_VALUE;
    if (!aligned16(h) || !aligned16(w_conf)) return DSPARK_ERR_ALIGN;
  }
  if (!aligned16(U) || !aligned16(W1) || !aligned16(W2) || ((uintptr_t)dev_error & 3u) != 0)
    return DSPARK_ERR_ALIGN;
  const size_t need = draft_ws_bytes(R, gamma, V) - kWsHeader;
  if (need > (size_t)DSPARK_NOALLOC_SCRATCH_BYTES) return DSPARK_ERR_SCRATCH;
  void *base = nullptr;
  if (scratch_of_current_device(&base) != hipSuccess) return DSPARK_ERR_HIP;
  // the same pieces as dspark_draft's workspace, without its header: the
  // sticky error word is the caller's dev_error, cleared by a kernel here
  size_t off = 0;
  DraftLaunch L{};
  L.err = dev_error;
  carve_draft(base, &off, R, gamma, V, L);
  L.R = R; L.gamma = gamma; L.V = V; L.r = r; L.d = d; L.bf16 = dt == DSPARK_BF16;
  L.invT = 1.0f / temp; L.U = U; L.W1 = W1; L.W2 = W2; L.x0 = x0; L.h = h; L.w_conf = w_conf;
  L.b_conf = b_conf; L.conf_temp = h != nullptr ? conf_temp : nullptr;
  L.seed = seed; L.round = round; L.x = x; L.q_stats = q_stats; L.q_x = q_x;
  L.c = c;
  if (launch_clear_error(dev_error, stream) != hipSuccess) return DSPARK_ERR_HIP;
  return from_hip(launch_draft(L, stream));
}

dspark_status dspark_draft_rnn(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                               const void *U, const void *W_o, const void *G_E, const float *G_h,
                               const void *W_hh, const float *b_hh, const int32_t *x0,
                               const float *s0, uint64_t seed, uint64_t round, int32_t *x,
                               float *q_stats, float *q_x, float *s, void *A, void *ws,
                               size_t ws_bytes, hipStream_t stream) {
  dspark_status st = check_common(R, gamma, V, r, dt, temp);
  if (st != DSPARK_OK) return st;
  if (!U || !W_o || !G_E || !G_h || !W_hh || !b_hh || !x0 || !x || !q_stats || !q_x || !s || !A ||
      !ws)
    return DSPARK_ERR_NULL;
  if (!aligned16(U) || !aligned16(W_o) || !aligned16(W_hh) || !aligned16(A) || !aligned16(ws))
    return DSPARK_ERR_ALIGN;
  if (ws_bytes < draft_ws_bytes(R, gamma, V)) return DSPARK_ERR_WORKSPACE;
  size_t off = 0;
  DraftLaunch L{};
  L.err = (int32_t *)carve(ws, &off, kWsHeader);
  carve_draft(ws, &off, R, gamma, V, L);
  L.R = R; L.gamma = gamma; L.V = V; L.r = r; L.bf16 = dt == DSPARK_BF16; L.invT = 1.0f / temp;
  L.U = U; L.W1 = nullptr; L.W2 = W_o; L.x0 = x0; L.seed = seed; L.round = round; L.x = x;
  L.q_stats = q_stats; L.q_x = q_x;
  RnnHead H{G_E, G_h, W_hh, b_hh, s0, s, A};
  L.rnn = &H;
  return from_hip(launch_draft(L, stream));
}

size_t dspark_schedule_workspace(int R, int gamma) {
  if (R < 1 || gamma < 1) return 0;
  return schedule_ws_bytes(R, gamma);
}

dspark_status dspark_schedule(int R, int gamma, dspark_sched_mode mode, float threshold,
                              const float *c, const float *c_prev2, const double *SPS, int B_max,
                              int32_t *ell,
                              int32_t *row_offset, float *a, int32_t *n_admitted, double *theta,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
  if (R < 1 || gamma < 1 || gamma > 64 || (int64_t)R * gamma > 8192) return DSPARK_ERR_SHAPE;
  if ((int)mode < 0 || (int)mode > 4) return DSPARK_ERR_MODE;
  if (!ell || !row_offset || !n_admitted || !theta || !ws) return DSPARK_ERR_NULL;
  if (mode != DSPARK_SCHED_OFF && !c) return DSPARK_ERR_MODE;
  if (mode == DSPARK_SCHED_ASYNC_TOPK && !c_prev2) return DSPARK_ERR_MODE;
  if (mode == DSPARK_SCHED_THRESHOLD && !isfinite(threshold)) return DSPARK_ERR_VALUE;
  const bool sps_optional = mode == DSPARK_SCHED_OFF || mode == DSPARK_SCHED_THRESHOLD;
  const bool need_sps = !sps_optional || (c != nullptr && SPS != nullptr);
  if (!sps_optional && !SPS) return DSPARK_ERR_SPS_TABLE;
  if (need_sps && (int64_t)B_max < (int64_t)R * (1 + gamma)) return DSPARK_ERR_SPS_TABLE;
  if (!aligned16(ws)) return DSPARK_ERR_ALIGN;
  if (ws_bytes < schedule_ws_bytes(R, gamma)) return DSPARK_ERR_WORKSPACE;
  ScheduleLaunch L{};
  L.R = R; L.gamma = gamma; L.mode = (int)mode; L.threshold = threshold; L.c = c;
  L.c_prev2 = mode == DSPARK_SCHED_ASYNC_TOPK ? c_prev2 : nullptr;
  L.SPS = need_sps ? SPS : nullptr; L.ell = ell; L.row_offset = row_offset;
  L.a = c ? a : nullptr; L.n_admitted = n_admitted; L.theta = theta; L.err = (int32_t *)ws;
  return from_hip(launch_schedule(L, stream));
}

size_t dspark_verify_workspace(int R, int gamma, int V, int rows_capacity) {
  if (R < 1 || gamma < 1 || V < 1 || rows_capacity < 1) return 0;
  return verify_ws_bytes(R, gamma, V, rows_capacity);
}

static dspark_status verify_impl(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                                 const int32_t *ell, const int32_t *row_offset, int rows_capacity,
                                 const void *P, const void *U, const void *W1, const void *W2,
                                 const int32_t *x0, const int32_t *x, const float *q_stats,
                                 const float *q_x, uint64_t seed, uint64_t round, int32_t *n_acc,
                                 int32_t *y, float *c_star, void *ws, size_t ws_bytes,
                                 hipStream_t stream, const void *A_given) {
  dspark_status s = check_common(R, gamma, V, r, dt, temp);
  if (s != DSPARK_OK) return s;
  if ((int64_t)rows_capacity < R || (int64_t)rows_capacity > (int64_t)R * (1 + gamma))
    return DSPARK_ERR_SHAPE;
  if (!ell || !row_offset || !P || !U || !W1 || !W2 || !x0 || !x || !q_stats || !q_x || !n_acc ||
      !y || !c_star || !ws)
    return DSPARK_ERR_NULL;
  if (!aligned16(P) || !aligned16(U) || !aligned16(W1) || !aligned16(W2) || !aligned16(ws))
    return DSPARK_ERR_ALIGN;
  if (ws_bytes < verify_ws_bytes(R, gamma, V, rows_capacity)) return DSPARK_ERR_WORKSPACE;
  size_t off = 0;
  VerifyLaunch L{};
  L.err = (int32_t *)carve(ws, &off, kWsHeader);
  L.p_chunks = (float2 *)carve(ws, &off, (size_t)rows_capacity * 4 * 8);
  L.bonus_tiles = (float2 *)carve(ws, &off, (size_t)R * n_tiles_of(V) * 8);
  L.pair_partials = (float2 *)carve(ws, &off, (size_t)R * gamma * n_tiles_of(V) * 8);
  L.row_map = (int4 *)carve(ws, &off, (size_t)R * gamma * 16);
  L.row_stats = (float4 *)carve(ws, &off, (size_t)R * gamma * 16);
  L.A_rows = carve(ws, &off, (size_t)R * gamma * kMaxRowBytes);
  L.R = R; L.gamma = gamma; L.V = V; L.r = r; L.rows_capacity = rows_capacity;
  L.bf16 = dt == DSPARK_BF16; L.invT = 1.0f / temp; L.ell = ell; L.row_offset = row_offset;
  L.P = P; L.U = U; L.W1 = W1; L.W2 = W2; L.x0 = x0; L.x = x; L.q_stats = q_stats; L.q_x = q_x;
  L.seed = seed; L.round = round; L.n_acc = n_acc; L.y = y; L.c_star = c_star;
  L.A_given = A_given;
  return from_hip(launch_verify(L, stream));
}

dspark_status dspark_verify(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                            const int32_t *ell, const int32_t *row_offset, int rows_capacity,
                            const void *P, const void *U, const void *W1, const void *W2,
                            const int32_t *x0, const int32_t *x, const float *q_stats,
                            const float *q_x, uint64_t seed, uint64_t round, int32_t *n_acc,
                            int32_t *y, float *c_star, void *ws, size_t ws_bytes,
                            hipStream_t stream) {
  return verify_impl(R, gamma, V, r, dt, temp, ell, row_offset, rows_capacity, P, U, W1, W2, x0,
                     x, q_stats, q_x, seed, round, n_acc, y, c_star, ws, ws_bytes, stream,
                     nullptr);
}

dspark_status dspark_verify_rnn(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                                const int32_t *ell, const int32_t *row_offset, int rows_capacity,
                                const void *P, const void *U, const void *A, const void *W_o,
                                const int32_t *x0, const int32_t *x, const float *q_stats,
                                const float *q_x, uint64_t seed, uint64_t round, int32_t *n_acc,
                                int32_t *y, float *c_star, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (!A) return DSPARK_ERR_NULL;
  if (!aligned16(A)) return DSPARK_ERR_ALIGN;
  // the table argument only has to pass the pointer checks: with given rows
  // no kernel reads it
  return verify_impl(R, gamma, V, r, dt, temp, ell, row_offset, rows_capacity, P, U, A, W_o, x0,
                     x, q_stats, q_x, seed, round, n_acc, y, c_star, ws, ws_bytes, stream, A);
}

size_t dspark_train_losses_workspace(int R, int gamma, int V) {
  if (R < 1 || gamma < 1 || V < 1) return 0;
  return train_ws_bytes(R, gamma, V);
}

dspark_status dspark_train_losses(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                                  const void *U, const void *W1, const void *W2, const void *P,
                                  const int32_t *x0, const int32_t *y, const float *c, float a_ce,
                                  float a_tv, float a_conf, float *per_pos, double *totals,
                                  void *ws, size_t ws_bytes, hipStream_t stream) {
  dspark_status s = check_common(R, gamma, V, r, dt, temp);
  if (s != DSPARK_OK) return s;
  if (!U || !W1 || !W2 || !P || !x0 || !y || !c || !totals || !ws) return DSPARK_ERR_NULL;
  if (!isfinite(a_ce) || !isfinite(a_tv) || !isfinite(a_conf)) return DSPARK_ERR_VALUE;
  if (!aligned16(P) || !aligned16(U) || !aligned16(W1) || !aligned16(W2) || !aligned16(ws))
    return DSPARK_ERR_ALIGN;
  if ((int64_t)R * (gamma + 1) > (1 << 24)) return DSPARK_ERR_SHAPE;
  if (ws_bytes < train_ws_bytes(R, gamma, V)) return DSPARK_ERR_WORKSPACE;
  const size_t n = (size_t)R * gamma;
  const int rows = R * (gamma + 1);
  size_t off = 0;
  int32_t *err = (int32_t *)carve(ws, &off, kWsHeader);
  TrainLaunch T{};
  DraftLaunch &D = T.draft;
  D.err = err;
  carve_draft(ws, &off, R, gamma, V, D);
  D.x = (int32_t *)carve(ws, &off, n * 4);
  D.q_stats = (float *)carve(ws, &off, n * 8);
  D.q_x = (float *)carve(ws, &off, n * 4);
  D.logq_x = (float *)carve(ws, &off, n * 4);
  D.R = R; D.gamma = gamma; D.V = V; D.r = r; D.bf16 = dt == DSPARK_BF16; D.invT = 1.0f / temp;
  D.U = U; D.W1 = W1; D.W2 = W2; D.x0 = x0; D.x_force = y;
  VerifyLaunch &L = T.verify;
  L.err = err;
  L.p_chunks = (float2 *)carve(ws, &off, (size_t)rows * 4 * 8);
  L.bonus_tiles = (float2 *)carve(ws, &off, (size_t)R * n_tiles_of(V) * 8);
  L.pair_partials = (float2 *)carve(ws, &off, n * n_tiles_of(V) * 8);
  L.row_map = (int4 *)carve(ws, &off, n * 16);
  L.row_stats = (float4 *)carve(ws, &off, n * 16);
  L.A_rows = carve(ws, &off, n * kMaxRowBytes);
  T.ell = (int32_t *)carve(ws, &off, ((size_t)R + 1) * 4);
  T.row_offset = (int32_t *)carve(ws, &off, ((size_t)R + 1) * 4);
  L.n_acc = (int32_t *)carve(ws, &off, ((size_t)R + 1) * 4);
  L.y = (int32_t *)carve(ws, &off, (size_t)rows * 4);
  L.c_star = (float *)carve(ws, &off, n * 4);
  L.R = R; L.gamma = gamma; L.V = V; L.r = r; L.rows_capacity = rows; L.bf16 = D.bf16;
  L.invT = D.invT; L.ell = T.ell; L.row_offset = T.row_offset; L.P = P; L.U = U; L.W1 = W1;
  L.W2 = W2; L.x0 = x0; L.x = y; L.q_stats = D.q_stats; L.q_x = D.q_x;
  T.R = R; T.gamma = gamma; T.c = c; T.a_ce = a_ce; T.a_tv = a_tv; T.a_conf = a_conf;
  T.per_pos = per_pos; T.totals = totals;
  T.req_sums = (double *)carve(ws, &off, (size_t)R * 3 * 8);
  return from_hip(launch_train(T, stream));
}

size_t dspark_tv_overlap_workspace(int n_rows, int V) {
  if (n_rows < 1 || V < 1) return 0;
  return overlap_ws_bytes(n_rows, V);
}

dspark_status dspark_tv_overlap(int n_rows, int V, dspark_dtype dt, float temp, const void *P,
                                const void *Q, const float *p_stats, const float *q_stats,
                                float *c_star, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (dt != DSPARK_F32 && dt != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  if (n_rows < 1 || V < 8 || V > 262144 || V % 8 != 0) return DSPARK_ERR_SHAPE;
  if (bad_temp(temp)) return DSPARK_ERR_VALUE;
  if (!P || !Q || !c_star || !ws) return DSPARK_ERR_NULL;
  if ((p_stats == nullptr) != (q_stats == nullptr)) return DSPARK_ERR_NULL;
  if (!aligned16(P) || !aligned16(Q) || !aligned16(ws)) return DSPARK_ERR_ALIGN;
  if (ws_bytes < overlap_ws_bytes(n_rows, V)) return DSPARK_ERR_WORKSPACE;
  size_t off = 0;
  OverlapLaunch L{};
  L.err = (int32_t *)carve(ws, &off, kWsHeader);
  L.p_chunks = (float2 *)carve(ws, &off, (size_t)n_rows * 4 * 8);
  L.q_chunks = (float2 *)carve(ws, &off, (size_t)n_rows * 4 * 8);
  L.partial = (float *)carve(ws, &off, (size_t)n_rows * 4 * 4);
  L.n_rows = n_rows; L.V = V; L.bf16 = dt == DSPARK_BF16; L.invT = 1.0f / temp; L.P = P; L.Q = Q;
  L.p_stats = p_stats; L.q_stats = q_stats; L.c_star = c_star;
  return from_hip(launch_overlap(L, stream));
}

dspark_status dspark_device_error(const void *ws, int32_t *code, hipStream_t stream) {
  if (!ws || !code) return DSPARK_ERR_NULL;
  if (hipStreamSynchronize(stream) != hipSuccess) return DSPARK_ERR_HIP;
  if (hipMemcpy(code, ws, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

dspark_status dspark_clear_device_error(void *ws, hipStream_t stream) {
  if (!ws) return DSPARK_ERR_NULL;
  if (!aligned16(ws)) return DSPARK_ERR_ALIGN;
  return from_hip(launch_clear_error((int32_t *)ws, stream));
}

}  // extern "C"
