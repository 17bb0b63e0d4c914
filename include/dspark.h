/*
 * dspark.h -- C ABI of the DSpark per-round speculative-decoding hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The method: DSpark, "Confidence-Scheduled Speculative Decoding with
 * Semi-Autoregressive Generation" (arXiv 2607.05147), as described by
 *   [Blog]    numb3r33 blog, "DSpark: confidence-scheduled speculative decoding"
 *   [Bangkok] vllmbangkok blog, "DSpark"
 *   [KB]      edgeai1 speculative-decoding knowledge base, "DSpark 精读"
 *   [Reaper]  mkdocs.reaper.mx, "3 · DSpark"
 *
 * Four operations, each one call:
 *   dspark_draft       Markov-head drafting of a gamma-token block per request
 *   dspark_schedule    confidence scheduler: how many drafts each request verifies
 *   dspark_verify      exact speculative-sampling verification of the ragged batch
 *   dspark_tv_overlap  the soft confidence label c* = sum_v min(p, q) on logit pairs
 *
 * Notation.  q is the draft law and p the target law (Blog, "One-token
 * exactness").  R requests, indexed rho = 0..R-1; block length gamma; draft
 * positions k = 1..gamma; vocabulary size V; rank r of the low-rank transition
 * B = W1 W2 (Blog, "Markov sequential head"); temperature T ("temp").
 *
 * Conventions for every entry point.
 *  - Array pointers are DEVICE pointers (memory of the GPU that is current on
 *    the calling thread), 16-byte aligned, densely packed, row-major unless
 *    stated.  Inputs are never modified.  The caller owns every buffer; the
 *    library allocates nothing and keeps no state except inside the caller's
 *    workspace.
 *  - Each call validates its arguments on the host first; on failure it returns
 *    the status and enqueues nothing.  Otherwise it enqueues kernels on
 *    `stream` and returns DSPARK_OK without waiting (asynchronous).  A launch
 *    failure returns DSPARK_ERR_HIP.  No C++ exception crosses the ABI.
 *  - Element type dt applies to every logit and weight array of a call:
 *    DSPARK_F32 = IEEE binary32, DSPARK_BF16 = bfloat16.  Accumulation is fp32.
 *  - Shape limits: 1 <= R; 1 <= gamma <= 64; 8 <= V <= 262144 with V % 8 == 0;
 *    r a multiple of 16 with 16 <= r <= 256 (r <= 128 for DSPARK_F32).
 *  - Random numbers: counter-based Philox4x64-10 (Salmon et al., SC'11) with
 *    key (seed, 0) and counter (position, rho, stream, round); the uniform is
 *    the top 24 bits of the first output word times 2^-24.  Streams: 0 = draft
 *    sample, 1 = accept test, 2 = final (residual or bonus) sample.  A round is
 *    reproducible bit for bit from (seed, round).
 *  - Device-side data errors (a token outside [0, V), a confidence outside
 *    [0, 1] or NaN, an inconsistent ell/row_offset, a non-finite logit
 *    statistic) cannot be seen by the host.  Kernels then stay in bounds, write
 *    sentinel outputs and OR a DSPARK_DEVERR_* bit into a sticky word held in
 *    the first 256 bytes of the call's workspace.  dspark_device_error reads it;
 *    dspark_clear_device_error clears it.  Clear a workspace once after
 *    allocating it.
 *  - Calls that share a workspace must be ordered on one stream.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* Scheduler modes (KB section 4; Bangkok 4.2.2; Blog "Async scheduler in
 * practice").  OFF verifies every draft (ell = gamma, the offline setting of
 * Bangkok 5.1).  EARLY_STOP admits along the sorted path while the throughput
 * strictly increases (the non-anticipating ideal).  FULL_SEARCH takes the
 * smallest admission count that maximizes throughput over the whole path (for
 * a stepped SPS table).  ASYNC_TOPK takes the capacity K from the confidences
 * of round t-2 (FULL_SEARCH on c_prev2) and admits the top K by current
 * survival. */
typedef enum {
  DSPARK_SCHED_OFF = 0,
  DSPARK_SCHED_EARLY_STOP = 1,
  DSPARK_SCHED_FULL_SEARCH = 2,
  DSPARK_SCHED_ASYNC_TOPK = 3,
  DSPARK_SCHED_THRESHOLD = 4
} dspark_sched_mode;

typedef enum {
  DSPARK_OK = 0,
  DSPARK_ERR_NULL = 1,      /* a required pointer is NULL                     */
  DSPARK_ERR_SHAPE = 2,     /* a size outside the limits above                */
  DSPARK_ERR_DTYPE = 3,     /* unknown element type                           */
  DSPARK_ERR_VALUE = 4,     /* temp not finite and > 0, or a bad scalar       */
  DSPARK_ERR_WORKSPACE = 5, /* ws_bytes below the *_workspace() size          */
  DSPARK_ERR_SPS_TABLE = 6, /* SPS table missing or shorter than R(1+gamma)+1 */
  DSPARK_ERR_MODE = 7,      /* unknown scheduler mode or missing c / c_prev2  */
  DSPARK_ERR_ALIGN = 8,     /* a pointer not 16-byte aligned                  */
  DSPARK_ERR_HIP = 9,       /* a HIP launch or runtime call failed            */
  DSPARK_ERR_SCRATCH = 10   /* the shape needs more than the static scratch   */
} dspark_status;

/* Bits of the sticky device error word. */
#define DSPARK_DEVERR_TOKEN 1      /* a token (anchor or draft) outside [0, V)      */
#define DSPARK_DEVERR_CONFIDENCE 2 /* a confidence outside [0, 1] or NaN           */
#define DSPARK_DEVERR_LENGTH 4     /* ell outside [0, gamma] or row_offset mismatch */
#define DSPARK_DEVERR_NONFINITE 8  /* a row max or normalizer not finite           */
#define DSPARK_DEVERR_SYNC 16      /* a device-wide wait of the persistent draft
                                      ran out (its outputs are then incomplete)    */

/* ------------------------------------------------------------------ draft --
 * Semi-autoregressive Markov-head drafting (Blog "Markov sequential head";
 * Bangkok 4.1; KB section 2).  For every request rho, with x_0 = x0[rho], for
 * k = 1..gamma (left to right; step k needs x_{k-1}):
 *   z_k(v) = (U[rho][k-1][v] + sum_i W1[x_{k-1}][i] * W2(i, v)) * (1/temp)
 *   q_k    = softmax(z_k),  m = max_v z_k(v),  S = sum_v exp(z_k(v) - m)
 *   x_k    = smallest v with u*S < sum_{w<=v} exp(z_k(w) - m),
 *            u = uniform(position k, rho, stream 0, round)
 * The bias row W1[x_{k-1}] W2 is a [R, r] x [r, V] product on bf16 matrix
 * cores with fp32 accumulation.  Optional confidence head (Bangkok 4.2.1; KB
 * section 4): c_k = sigmoid(z_k / T_k),
 *   z_k = sum_j w_conf[j] h[rho][k-1][j] + sum_i w_conf[d+i] W1[x_{k-1}][i] + b_conf,
 * with T_k the position's temperature of sequential temperature scaling (Blog
 * "Sequential temperature scaling"; Bangkok 4.2.1), 1 when conf_temp is NULL.
 *
 * Inputs
 *   U      [R][gamma][V]  draft base logits U_k of the parallel backbone (dt)
 *   W1     [V][r]         row x is the transition embedding W1[x, :] (dt)
 *   W2     r x V factor stored COLUMN-major: element (i, v) at W2[v*r + i],
 *          so the r coefficients of vocabulary entry v are contiguous (dt)
 *   x0     [R]            anchor tokens (the target's last token), int32
 *   h      [R][gamma][d]  backbone hidden states for the confidence head (dt), or NULL
 *   d      width of h (d % 8 == 0, 8 <= d <= 65536); ignored when h == NULL
 *   w_conf [d + r] fp32 head weights; b_conf fp32 bias; ignored when h == NULL
 *   conf_temp [gamma] fp32 per-position temperatures T_k > 0, or NULL (all 1);
 *          ignored when h == NULL.  A T_k that is not a finite positive number
 *          sets DSPARK_DEVERR_CONFIDENCE and is taken as 1.
 *   seed, round           Philox key and round counter
 * Outputs
 *   x       [R][gamma]    drafted tokens x_1..x_gamma, int32
 *   q_stats [R][gamma][2] (m, S) of z_k, so q_k(v) = exp(z_k(v) - m) / S, fp32
 *   q_x     [R][gamma]    q_k(x_k), fp32
 *   c       [R][gamma]    confidences c_k, written iff h != NULL (may be NULL otherwise)
 * Execution: with bf16, r = 256, R <= 512 and at most 5 vocabulary tiles of
 * 128 per compute unit (past R = 128 also at least 128 tiles: V >= 16384),
 * all gamma steps run in one cooperative launch of one workgroup per compute
 * unit that keeps W2 on chip for the call (past R = 128 the requests go in
 * chunks of 128, the draws of one chunk beside the next chunk's products); its
 * workgroups exchange tile partials and draws through the workspace with
 * device-coherent accesses and bounded waits (a wait that runs out sets
 * DSPARK_DEVERR_SYNC and the outputs are incomplete).  If the device refuses
 * the cooperative launch, or DSPARK_PERSISTENT_DRAFT=0 is set in the
 * environment, gamma launches of the per-step kernels run instead.  Both
 * follow the same law; they sum the tile partials in different orders, so a
 * draw whose uniform falls within rounding of a CDF boundary may differ.
 * Workspace: dspark_draft_workspace(R, gamma, V, r, dt) bytes. */
size_t dspark_draft_workspace(int R, int gamma, int V, int r, dspark_dtype dt);
dspark_status dspark_draft(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                           const void *U, const void *W1, const void *W2, const int32_t *x0,
                           const void *h, int d, const float *w_conf, float b_conf,
                           const float *conf_temp, uint64_t seed, uint64_t round,
                           int32_t *x, float *q_stats, float *q_x, float *c,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------- draft without allocation --
 * dspark_draft for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels and results as dspark_draft; the
 * draft's scratch (two halves of tile partials, 2 * R * ceil(V/128) * 8
 * bytes, the head's dot products, two transition-row buffers, R published
 * draws) lives in a static device array of
 * DSPARK_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * workspace); its first call on a GPU looks up that GPU's copy of the array.
 *   dev_error  [1] int32 device word: cleared by the call, then receives the
 *              DSPARK_DEVERR_* bits of this call (as the workspace word of
 *              dspark_draft does).
 * Limit: dspark_draft_noalloc_scratch(R, gamma, V) <= DSPARK_NOALLOC_SCRATCH_BYTES,
 * e.g. R <= 512 at V = 151936; larger shapes return DSPARK_ERR_SCRATCH and
 * enqueue nothing.  All calls on one GPU share the array: calls whose kernels
 * may overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller. */
#define DSPARK_NOALLOC_SCRATCH_BYTES (16u << 20)
size_t dspark_draft_noalloc_scratch(int R, int gamma, int V);
dspark_status dspark_draft_noalloc(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                                   const void *U, const void *W1, const void *W2,
                                   const int32_t *x0, const void *h, int d, const float *w_conf,
                                   float b_conf, const float *conf_temp, uint64_t seed,
                                   uint64_t round, int32_t *x, float *q_stats, float *q_x,
                                   float *c, int32_t *dev_error, hipStream_t stream);

/* --------------------------------------------------------------- schedule --
 * Hardware-aware prefix scheduler (KB section 4; Blog "Scheduler objective",
 * "Greedy prefix allocation"; Reaper 3.3).  One workgroup:
 *   a[rho][j] = fl32(a[rho][j-1] * c[rho][j]), a[rho][0] = 1, binary32 left to right
 *   candidates (rho, j), sorted by a descending, then j ascending, then rho ascending
 *   A_n = sum of floor(a * 2^32) over the first n candidates (int64)
 *   tau_n = R + A_n * 2^-32,  B_n = R + n,  theta_n = tau_n * SPS[B_n]   (fp64)
 *   n* by mode; ell[rho] = admitted candidates of rho (a prefix by the order);
 *   row_offset = exclusive scan of (1 + ell).
 * THRESHOLD mode (the static confidence cutoff the pages test before the
 * scheduler, Bangkok 5.3; KB section 7): no sort; request rho keeps its
 * leading positions with c[rho][j] >= threshold, up to the first one below it;
 * n* = sum ell and theta = tau * SPS[R + n*] over the kept positions.
 * Inputs
 *   c       [R][gamma] conditional confidences in [0, 1], fp32 (may be NULL in OFF mode)
 *   c_prev2 [R][gamma] confidences of round t-2, ASYNC_TOPK only (else ignored)
 *   SPS     [B_max + 1] target steps per second indexed by verify batch size B,
 *           fp64; B_max >= R * (1 + gamma).  May be NULL in OFF and THRESHOLD
 *           modes (theta is then NaN).
 *   threshold  THRESHOLD mode's cutoff (finite; ignored in other modes)
 *   R * gamma <= 8192, gamma <= 64.
 * Outputs
 *   ell [R], row_offset [R + 1] int32; a [R][gamma] fp32 (may be NULL);
 *   n_admitted [1] int32; theta [1] fp64 (theta_{n*}; NaN when c is NULL).
 * Workspace: dspark_schedule_workspace(R, gamma) bytes. */
size_t dspark_schedule_workspace(int R, int gamma);
dspark_status dspark_schedule(int R, int gamma, dspark_sched_mode mode, float threshold,
                              const float *c, const float *c_prev2,
                              const double *SPS, int B_max,
                              int32_t *ell, int32_t *row_offset, float *a,
                              int32_t *n_admitted, double *theta,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------- verify --
 * Exact speculative-sampling verification of the flattened ragged batch (Blog
 * "One-token exactness", "Why only the longest accepted prefix survives",
 * "Variable-length verification without wasting kernels"; KB sections 7-8).
 * For request rho with ell = ell[rho] and base = row_offset[rho]:
 *   p_k = softmax(P[base + k - 1] * (1/temp)), k = 1..ell+1
 *   q_k = the draft law of dspark_draft at position k (z_k recomputed from
 *         x_{k-1} with the draft's arithmetic; normalized by q_stats)
 *   accept x_k iff uniform(k, rho, stream 1, round) * q_x[rho][k-1] < p_k(x_k)
 *   n = (first rejected k) - 1, or ell when all are accepted
 *   final token: if n < ell, drawn from (p_{n+1} - q_{n+1})_+ (from p_{n+1}
 *   if that mass is not positive); otherwise the bonus token from p_{ell+1};
 *   both by inverse CDF with uniform(position, rho, stream 2, round)
 *   c*_k = sum_v min(p_k(v), q_k(v)) = 1 - TV(p_k, q_k), k = 1..ell
 * Inputs
 *   ell [R], row_offset [R+1]: as written by dspark_schedule (ell in [0, gamma],
 *        row_offset[rho+1] = row_offset[rho] + 1 + ell[rho], row_offset[0] = 0)
 *   rows_capacity: host bound on row_offset[R], R <= rows_capacity <= R(1+gamma)
 *   P   [rows_capacity][V] target logits; row row_offset[rho] + k - 1 holds
 *       position k = 1..ell+1 of request rho (dt)
 *   U, W1, W2, x0: as given to dspark_draft; x [R][gamma] the drafted tokens
 *   q_stats, q_x: as written by dspark_draft (verification uses the SAME q)
 * Outputs
 *   n_acc  [R]           accepted drafts n, int32
 *   y      [R][gamma+1]  x_1..x_n, then the final token, then -1, int32
 *   c_star [R][gamma]    c*_k for k <= ell, NaN beyond, fp32
 * Execution: with bf16, r = 256, R * gamma > 256 and at most 5 vocabulary
 * tiles of 128 per compute unit, the c* and residual tile partials come from
 * one workgroup per compute unit that keeps its tiles of W2 on chip while
 * every verified row streams past; otherwise (or with DSPARK_STATIONARY_VERIFY=0 in the
 * environment) from a kernel that keeps rows on chip and streams W2.  Both
 * compute the same products; they add the partials in different orders, so
 * c* may differ in the last bits and a residual draw whose uniform falls
 * within rounding of a CDF boundary may differ.
 * Workspace: dspark_verify_workspace(R, gamma, V, rows_capacity) bytes. */
size_t dspark_verify_workspace(int R, int gamma, int V, int rows_capacity);
dspark_status dspark_verify(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                            const int32_t *ell, const int32_t *row_offset, int rows_capacity,
                            const void *P, const void *U, const void *W1, const void *W2,
                            const int32_t *x0, const int32_t *x,
                            const float *q_stats, const float *q_x,
                            uint64_t seed, uint64_t round,
                            int32_t *n_acc, int32_t *y, float *c_star,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------- recurrent head --
 * The draft with the recurrent sequential head instead of the Markov table
 * (Blog "RNN sequential head"; KB section 3): a running state replaces the
 * previous-token lookup, z_k = (U_k + s_k W_o) / temp, with the gated update
 * read as a GRU over the previous token's embedding and the position's
 * backbone hidden state:
 *   g   = G_E[x_{k-1}] + G_h[rho][k-1]          input pre-activations [3r]
 *   a   = W_hh s_{k-1} + b_hh                    recurrent pre-activations [3r]
 *   s_k = (1 - zg) tanh(g_n + rg a_n) + zg s_{k-1},
 *         rg = sigmoid(g_r + a_r), zg = sigmoid(g_z + a_z)   (gate blocks r, z, n)
 * with s_0 = s0[rho] (zeros if s0 is NULL) and x_0 = x0[rho].  s_k is kept in
 * fp32; the product uses A_k = s_k rounded to dt (round to nearest even).
 * Sampling, q_stats and q_x are those of dspark_draft (same streams and
 * uniforms).  No confidence head here.
 * Inputs
 *   U [R][gamma][V] (dt); W_o column-major like W2 of dspark_draft (dt)
 *   G_E [V][3r] (dt): the token embedding table times the input weights of the
 *       update, computed once from the static weights
 *   G_h [R][gamma][3r] fp32: the backbone hidden states times the hidden-state
 *       input weights, plus the input biases (a product of the backbone's
 *       outputs, made with the backbone)
 *   W_hh [r][3r] column-major (dt, 16-byte aligned): element (g, i) at W_hh[i * 3r + g]
 *   b_hh [3r] fp32; x0 [R] int32; s0 [R][r] fp32 or NULL
 * Outputs
 *   x, q_stats, q_x as dspark_draft
 *   s [R][gamma][r] fp32 states; A [gamma][R][r] (dt) the transition rows the
 *   product used (row ((k-1) R + rho)): dspark_verify_rnn takes them
 * Workspace: dspark_draft_workspace(R, gamma, V, r, dt) bytes. */
dspark_status dspark_draft_rnn(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                               const void *U, const void *W_o, const void *G_E, const float *G_h,
                               const void *W_hh, const float *b_hh, const int32_t *x0,
                               const float *s0, uint64_t seed, uint64_t round, int32_t *x,
                               float *q_stats, float *q_x, float *s, void *A,
                               void *ws, size_t ws_bytes, hipStream_t stream);

/* dspark_verify for drafts of the recurrent head: the draft law of position k
 * is recomputed from the given transition row A[(k-1) R + rho] (as written by
 * dspark_draft_rnn) instead of W1[x_{k-1}]; W_o takes the place of W2.  All
 * other arguments, outputs and the workspace are those of dspark_verify. */
dspark_status dspark_verify_rnn(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                                const int32_t *ell, const int32_t *row_offset, int rows_capacity,
                                const void *P, const void *U, const void *A, const void *W_o,
                                const int32_t *x0, const int32_t *x,
                                const float *q_stats, const float *q_x,
                                uint64_t seed, uint64_t round,
                                int32_t *n_acc, int32_t *y, float *c_star,
                                void *ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------- train_losses --
 * Forward-only training reductions of the drafter on the ground-truth prefix
 * (Blog "Training objective"; KB section 5).  With the label prefix
 * x_0 = x0[rho], x_k = y[rho][k-1] (teacher forcing):
 *   q_k    = the draft law of dspark_draft at position k, conditioned on x_{k-1}
 *   p_k    = softmax(P[rho (gamma+1) + k - 1] * (1/temp))
 *   CE_k   = -log q_k(y_k)
 *   L1_k   = sum_v |p_k(v) - q_k(v)| = 2 (1 - c*_k), twice the total variation
 *   BCE_k  = -(c*_k log c_k + (1 - c*_k) log(1 - c_k)), c*_k = sum_v min(p_k, q_k)
 *   w_k    = exp(-(k - 1) / gamma)
 *   L_x    = (1/R) sum_rho (sum_k w_k x_k) / (sum_k w_k) for x = CE, L1, BCE
 *   L      = a_ce L_ce + a_tv L_tv + a_conf L_conf (the page's defaults 0.1, 0.9, 1.0)
 * q and c* come from the draft and verification kernels themselves (a
 * teacher-forced draft pass, then a verification pass with every position
 * admitted), so the losses see exactly the distributions the hot path draws from.
 * Inputs
 *   U [R][gamma][V], W1, W2, x0: as for dspark_draft (device, dt)
 *   P [R][gamma+1][V] target logits, position k of request rho at row
 *     rho (gamma+1) + k - 1 (the last row of each request is not read) (dt)
 *   y [R][gamma] labels in [0, V), int32; an out-of-range label sets the
 *     DSPARK_DEVERR_TOKEN bit of the device error word and is read as 0
 *   c [R][gamma] confidences, fp32 (log of 0 or 1 gives an infinite BCE)
 *   a_ce, a_tv, a_conf: finite loss weights
 * Outputs (device)
 *   per_pos [3][R][gamma] (CE, L1, BCE) per position, fp32, or NULL
 *   totals  [4] (L_ce, L_tv, L_conf, L), fp64, summed in a fixed order
 * Workspace: dspark_train_losses_workspace(R, gamma, V) bytes; the device
 * error word is its first word (dspark_device_error). */
size_t dspark_train_losses_workspace(int R, int gamma, int V);
dspark_status dspark_train_losses(int R, int gamma, int V, int r, dspark_dtype dt, float temp,
                                  const void *U, const void *W1, const void *W2, const void *P,
                                  const int32_t *x0, const int32_t *y, const float *c,
                                  float a_ce, float a_tv, float a_conf,
                                  float *per_pos, double *totals,
                                  void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------- tv_overlap --
 * Soft confidence label on explicit logit pairs (Blog "Total variation label";
 * KB section 4): c*[i] = sum_v min(p_i(v), q_i(v)) with p_i = softmax(P[i]/temp)
 * and q_i = softmax(Q[i]/temp).
 * Inputs
 *   P, Q [n_rows][V] logits (dt)
 *   p_stats, q_stats [n_rows][2] fp32 (m, S) with p(v) = exp(P[i][v]/temp - m) / S,
 *   both given (one pass over P and Q) or both NULL (computed: two passes)
 * Output: c_star [n_rows] fp32.
 * Workspace: dspark_tv_overlap_workspace(n_rows, V) bytes. */
size_t dspark_tv_overlap_workspace(int n_rows, int V);
dspark_status dspark_tv_overlap(int n_rows, int V, dspark_dtype dt, float temp,
                                const void *P, const void *Q,
                                const float *p_stats, const float *q_stats,
                                float *c_star, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------- utilities -- */
const char *dspark_status_string(dspark_status s);
/* Waits for `stream`, then copies the sticky device error word of workspace ws
 * to *code (0 = no error).  Returns DSPARK_ERR_HIP if the stream faulted. */
dspark_status dspark_device_error(const void *ws, int32_t *code, hipStream_t stream);
/* Enqueues a kernel on `stream` that zeroes the sticky error word of ws. */
dspark_status dspark_clear_device_error(void *ws, hipStream_t stream);

/* Opt-in kernel timing (diagnostics; off by default).  While enabled, every
 * kernel the library launches is bracketed by two HIP events on its stream.
 * dspark_trace_enable(1) discards earlier records; dspark_trace_collect waits
 * for the recorded events and returns the number of distinct kernel names (or
 * -1 on a HIP error); dspark_trace_entry(i, ...) returns the i-th name (a
 * string owned by the library, valid until the next collect or enable), its
 * summed elapsed milliseconds and its launch count.  Not for concurrent use
 * from several host threads while enabled. */
dspark_status dspark_trace_enable(int on);
int dspark_trace_collect(void);
dspark_status dspark_trace_entry(int i, const char **name, double *total_ms, int *launches);

#ifdef __cplusplus
}
#endif
#endif /* DSPARK_H */
