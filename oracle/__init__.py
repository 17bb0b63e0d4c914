"""CPU oracle for the DSpark per-round hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It wraps ``liboracle.so`` (plain single-threaded C++, fp64) with
numpy marshalling.  It shares no code with the HIP library.

Element types: ``F32`` arrays are float32; ``BF16`` arrays are uint16 holding
bfloat16 bit patterns.  Layouts are listed in ``oracle.h``.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1
STREAM_DRAFT, STREAM_ACCEPT, STREAM_FINAL = 0, 1, 2
SCHED_OFF, SCHED_EARLY_STOP, SCHED_FULL_SEARCH, SCHED_ASYNC_TOPK, SCHED_THRESHOLD = 0, 1, 2, 3, 4

_lib = None


def lib():
    """Load (building first if absent) the oracle library."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


_vp = C.c_void_p
_dp = C.POINTER(C.c_double)
_i32p = C.POINTER(C.c_int32)
_f32p = C.POINTER(C.c_float)
_u64p = C.POINTER(C.c_uint64)


def _declare(L):
    L.orc_philox4x64_10.argtypes = [_u64p, _u64p, _u64p]
    L.orc_uniform.argtypes = [C.c_uint64] * 5
    L.orc_uniform.restype = C.c_double
    L.orc_row_stats.argtypes = [C.c_int, C.c_int, C.c_double, _vp, _dp, _dp]
    L.orc_inverse_cdf.argtypes = [C.c_int, _dp, C.c_double, _dp]
    L.orc_draft_position.argtypes = [C.c_int, C.c_int, C.c_int, C.c_double, _vp, _vp, _vp, C.c_int,
                                     C.c_double, _dp, _dp, _dp, _dp, _dp]
    L.orc_conf_head.argtypes = [C.c_int, C.c_int, C.c_int, _vp, _f32p, C.c_float, C.c_double, _vp,
                                C.c_int]
    L.orc_conf_head.restype = C.c_double
    L.orc_draft_request.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_double, _vp, _vp, _vp,
                                    C.c_int, _i32p, _vp, C.c_int, _f32p, C.c_float, _f32p,
                                    C.c_uint64, C.c_uint64, C.c_int, _i32p, _dp, _dp, _dp, _dp]
    L.orc_overlap.argtypes = [C.c_int, C.c_int, C.c_double, _vp, _vp, _dp]
    L.orc_overlap.restype = C.c_double
    L.orc_select_n.argtypes = [_dp, C.c_int, C.c_int]
    L.orc_schedule.argtypes = [C.c_int, C.c_int, C.c_int, C.c_double, _f32p, _f32p, _dp, C.c_int,
                               _i32p, _i32p, _f32p, _i32p, _dp, _i32p, _dp]
    L.orc_train_losses.argtypes = [C.c_int] * 5 + [C.c_double, _vp, _vp, _vp, _i32p, _i32p, _vp,
                                                   _f32p, C.c_double, C.c_double, C.c_double, _dp, _dp]
    L.orc_schedule_bruteforce.argtypes = [C.c_int, C.c_int, _f32p, _dp, C.c_int, _i32p]
    L.orc_schedule_bruteforce.restype = C.c_double
    L.orc_verify_request.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_double, C.c_int, _vp,
                                     _vp, _vp, _vp, C.c_int, _i32p, C.c_uint64, C.c_uint64, C.c_int,
                                     C.c_int, _i32p, _i32p, _dp, _dp, _dp, _dp, _dp, _i32p]
    L.orc_verify_request_rows.argtypes = L.orc_verify_request.argtypes
    L.orc_rnn_states.argtypes = [C.c_int] * 4 + [_vp, _f32p, _vp, _f32p, C.c_int, _i32p, _f32p,
                                                 _dp]


def _ptr(a, ctype=None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(C.POINTER(ctype)) if ctype is not None else C.c_void_p(a.ctypes.data)


def dtype_code(a):
    """F32 for float32 arrays, BF16 for uint16 (bfloat16 bit pattern) arrays."""
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle arrays must be float32 or uint16 (bf16 bits), got {a.dtype}")


# --------------------------------------------------------------------------- RNG
def philox4x64_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    lib().orc_philox4x64_10(_ptr(c, C.c_uint64), _ptr(k, C.c_uint64), _ptr(out, C.c_uint64))
    return out


def uniform(seed, rnd, pos, req, stream):
    return lib().orc_uniform(seed, rnd, pos, req, stream)


# --------------------------------------------------------------------- softmax
def widen(a):
    a = np.ascontiguousarray(a)
    out = np.empty(a.size, dtype=np.float64)
    lib().orc_widen(dtype_code(a), _ptr(a), a.size, _ptr(out, C.c_double))
    return out.reshape(a.shape)


def row_stats(row, temp=1.0):
    row = np.ascontiguousarray(row)
    m, S = C.c_double(), C.c_double()
    rc = lib().orc_row_stats(row.size, dtype_code(row), temp, _ptr(row), C.byref(m), C.byref(S))
    assert rc == 0
    return m.value, S.value


def inverse_cdf(w, u, want_cdf=False):
    w = np.ascontiguousarray(w, dtype=np.float64)
    cdf = np.empty_like(w) if want_cdf else None
    v = lib().orc_inverse_cdf(w.size, _ptr(w, C.c_double), u, _ptr(cdf, C.c_double))
    return (v, cdf) if want_cdf else v


def overlap(P_row, Q_row, temp=1.0, with_tv=False):
    P_row, Q_row = np.ascontiguousarray(P_row), np.ascontiguousarray(Q_row)
    assert P_row.dtype == Q_row.dtype and P_row.size == Q_row.size
    tv = C.c_double()
    c = lib().orc_overlap(P_row.size, dtype_code(P_row), temp, _ptr(P_row), _ptr(Q_row),
                          C.byref(tv))
    return (c, tv.value) if with_tv else c


# ----------------------------------------------------------------------- draft
def draft_position(U_row, W1, W2, prev, u, temp=1.0, want_law=False):
    """One Markov-head position.  W1 is [V][r] (any table of transition rows,
    indexed by prev); W2 is column-major, i.e. the array W2[v, i] holds element
    (i, v) of the r x V factor."""
    U_row = np.ascontiguousarray(U_row)
    V, r = U_row.shape[-1], W1.shape[1]
    assert W2.shape == (V, r) and 0 <= prev < W1.shape[0]
    dt = dtype_code(U_row)
    q = np.empty(V) if want_law else None
    cdf = np.empty(V) if want_law else None
    m, S, qx = C.c_double(), C.c_double(), C.c_double()
    x = lib().orc_draft_position(V, r, dt, temp, _ptr(U_row), _ptr(W1), _ptr(W2), int(prev), u,
                                 _ptr(q, C.c_double), _ptr(cdf, C.c_double), C.byref(m),
                                 C.byref(S), C.byref(qx))
    out = dict(x=x, m=m.value, S=S.value, qx=qx.value)
    if want_law:
        out.update(q=q, cdf=cdf)
    return out


def conf_head(h_row, w_conf, b_conf, W1, prev, T=1.0):
    """c = sigmoid(z / T) for the head's logit z; T is the position's temperature."""
    V, r = W1.shape
    h_row = np.ascontiguousarray(h_row)
    w = np.ascontiguousarray(w_conf, dtype=np.float32)
    return lib().orc_conf_head(h_row.size, r, dtype_code(h_row), _ptr(h_row), _ptr(w, C.c_float),
                               float(b_conf), float(T), _ptr(W1), int(prev))


def draft_request(U_req, W1, W2, x0, seed, rnd, rho, temp=1.0, x_cond=None, h_req=None,
                  w_conf=None, b_conf=0.0, conf_temp=None):
    """Whole block of one request; U_req is [gamma][V]."""
    gamma, V = U_req.shape
    r = W1.shape[1]
    U_req = np.ascontiguousarray(U_req)
    x = np.zeros(gamma, dtype=np.int32)
    qx, m, S = np.zeros(gamma), np.zeros(gamma), np.zeros(gamma)
    c = np.full(gamma, np.nan) if h_req is not None else None
    xc = None if x_cond is None else np.ascontiguousarray(x_cond, dtype=np.int32)
    d = 0 if h_req is None else h_req.shape[1]
    h = None if h_req is None else np.ascontiguousarray(h_req)
    w = None if w_conf is None else np.ascontiguousarray(w_conf, dtype=np.float32)
    ct = None if conf_temp is None else np.ascontiguousarray(conf_temp, dtype=np.float32)
    rc = lib().orc_draft_request(gamma, V, r, dtype_code(U_req), temp, _ptr(U_req), _ptr(W1),
                                 _ptr(W2), int(x0), _ptr(xc, C.c_int32), _ptr(h), d,
                                 _ptr(w, C.c_float), float(b_conf), _ptr(ct, C.c_float), seed, rnd,
                                 rho,
                                 _ptr(x, C.c_int32), _ptr(qx, C.c_double), _ptr(m, C.c_double),
                                 _ptr(S, C.c_double), _ptr(c, C.c_double))
    assert rc == 0, "oracle draft rejected its arguments"
    return dict(x=x, qx=qx, m=m, S=S, c=c)


# ------------------------------------------------------------------- schedule
def select_n(theta, mode):
    theta = np.ascontiguousarray(theta, dtype=np.float64)
    return lib().orc_select_n(_ptr(theta, C.c_double), theta.size - 1, mode)


def schedule(c, SPS, mode, c_prev2=None, R=None, gamma=None, threshold=0.0):
    """c is [R][gamma] float32 (or None for OFF); SPS is the float64 table indexed by B
    (optional in OFF and THRESHOLD modes); threshold is the THRESHOLD mode's cutoff."""
    if c is not None:
        c = np.ascontiguousarray(c, dtype=np.float32)
        R, gamma = c.shape
    cp = None if c_prev2 is None else np.ascontiguousarray(c_prev2, dtype=np.float32)
    sps = None if SPS is None else np.ascontiguousarray(SPS, dtype=np.float64)
    ell = np.zeros(R, dtype=np.int32)
    row_offset = np.zeros(R + 1, dtype=np.int32)
    a = np.zeros((R, gamma), dtype=np.float32)
    n_adm, n_plain = C.c_int32(), C.c_int32()
    theta, theta_plain = C.c_double(), C.c_double()
    rc = lib().orc_schedule(R, gamma, mode, float(threshold), _ptr(c, C.c_float), _ptr(cp, C.c_float),
                            _ptr(sps, C.c_double), 0 if sps is None else sps.size - 1,
                            _ptr(ell, C.c_int32), _ptr(row_offset, C.c_int32), _ptr(a, C.c_float),
                            C.byref(n_adm), C.byref(theta), C.byref(n_plain), C.byref(theta_plain))
    if rc != 0:
        raise ValueError("oracle schedule rejected its arguments")
    return dict(ell=ell, row_offset=row_offset, a=a if c is not None else None,
                n_admitted=n_adm.value, theta=theta.value, n_plain=n_plain.value,
                theta_plain=theta_plain.value)


def schedule_bruteforce(c, SPS):
    c = np.ascontiguousarray(c, dtype=np.float32)
    R, gamma = c.shape
    sps = np.ascontiguousarray(SPS, dtype=np.float64)
    ell = np.zeros(R, dtype=np.int32)
    best = lib().orc_schedule_bruteforce(R, gamma, _ptr(c, C.c_float), _ptr(sps, C.c_double),
                                         sps.size - 1, _ptr(ell, C.c_int32))
    return best, ell


def acceptance_counts(ell_rounds, n_acc_rounds, gamma):
    """Per request and draft position k = 1..gamma, over past rounds: the rounds
    in which position k was verified (k <= ell and all k - 1 before it were
    accepted, so verification reached it) and those in which it was accepted
    (k <= n_acc).  These are the numerator and denominator of the conditional
    acceptance P(A_k | A_1..A_{k-1}) (Blog, "Conditional acceptance curves").
    Plain loops: one round, request and position at a time."""
    R = len(ell_rounds[0]) if len(ell_rounds) else 0
    verified = [[0] * gamma for _ in range(R)]
    accepted = [[0] * gamma for _ in range(R)]
    for ell, n_acc in zip(ell_rounds, n_acc_rounds):
        for rho in range(R):
            for k in range(1, gamma + 1):
                reached = k <= int(ell[rho]) and int(n_acc[rho]) >= k - 1
                if reached:
                    verified[rho][k - 1] += 1
                    if int(n_acc[rho]) >= k:
                        accepted[rho][k - 1] += 1
    return verified, accepted


def acceptance_estimates(ell_rounds, n_acc_rounds, R, gamma, alpha=4.0, beta=1.0):
    """[R][gamma] float32 confidences from a loop's own history: the conditional
    acceptance of each (request, position) with a Beta(alpha, beta) prior,
    (accepted + alpha) / (verified + alpha + beta), in float64 rounded once.
    With no past round every entry is alpha / (alpha + beta)."""
    c = np.full((R, gamma), alpha / (alpha + beta), dtype=np.float64)
    if len(ell_rounds):
        verified, accepted = acceptance_counts(ell_rounds, n_acc_rounds, gamma)
        for rho in range(R):
            for k in range(gamma):
                c[rho, k] = (accepted[rho][k] + alpha) / (verified[rho][k] + alpha + beta)
    return c.astype(np.float32)


def conditional_acceptance_curve(ell_rounds, n_acc_rounds, gamma):
    """P(A_k | A_1..A_{k-1}) for k = 1..gamma over all requests and rounds (nan
    where position k was never verified)."""
    verified, accepted = acceptance_counts(ell_rounds, n_acc_rounds, gamma)
    out = []
    for k in range(gamma):
        v = sum(row[k] for row in verified)
        a = sum(row[k] for row in accepted)
        out.append(a / v if v else float("nan"))
    return np.array(out)


# --------------------------------------------------------------------- verify
def verify_request(P_req, U_req, W1, W2, x0, x, ell, seed, rnd, rho, temp=1.0, force_n=-1,
                   want_cdf=False, A_rows=None):
    """P_req is [ell+1][V] (the request's flattened target rows), U_req [gamma][V].
    With A_rows [gamma][r] the draft's transition row of position k is
    A_rows[k-1] (W1 is then ignored)."""
    gamma, V = U_req.shape
    r = (W1 if A_rows is None else A_rows).shape[1]
    fn = lib().orc_verify_request
    if A_rows is not None:
        A_rows = np.ascontiguousarray(A_rows)
        assert A_rows.shape == (gamma, r) and A_rows.dtype == U_req.dtype
        W1, fn = A_rows, lib().orc_verify_request_rows
    P_req, U_req = np.ascontiguousarray(P_req), np.ascontiguousarray(U_req)
    assert P_req.shape[0] >= ell + 1
    x = np.ascontiguousarray(x, dtype=np.int32)
    n_acc = C.c_int32()
    y = np.zeros(gamma + 1, dtype=np.int32)
    c_star, ratio, u_acc = np.zeros(gamma), np.zeros(gamma), np.zeros(gamma)
    fcdf = np.zeros(V) if want_cdf else None
    fu = C.c_double()
    fb = C.c_int32()
    rc = fn(gamma, V, r, dtype_code(U_req), temp, int(ell), _ptr(P_req),
                                  _ptr(U_req), _ptr(W1), _ptr(W2), int(x0), _ptr(x, C.c_int32),
                                  seed, rnd, rho, int(force_n), C.byref(n_acc), _ptr(y, C.c_int32),
                                  _ptr(c_star, C.c_double), _ptr(ratio, C.c_double),
                                  _ptr(u_acc, C.c_double), _ptr(fcdf, C.c_double), C.byref(fu),
                                  C.byref(fb))
    assert rc == 0, "oracle verify rejected its arguments"
    return dict(n_acc=n_acc.value, y=y, c_star=c_star, ratio=ratio, u_acc=u_acc,
                final_cdf=fcdf, final_u=fu.value, residual_fallback=fb.value)


# ------------------------------------------------------------ training losses
def train_losses(U, W1, W2, x0, y, P, c, temp=1.0, alpha=(0.1, 0.9, 1.0)):
    """Forward-only training reductions, teacher-forced.  U [R][gamma][V], y
    [R][gamma] ground-truth tokens, P [R][gamma + 1][V] (verify layout), c
    [R][gamma].  Returns per-position (CE, L1, BCE) [3][R][gamma] and the totals
    (L_ce, L_tv, L_conf, L)."""
    R, gamma, V = U.shape
    r = W1.shape[1]
    U, P = np.ascontiguousarray(U), np.ascontiguousarray(P)
    x0 = np.ascontiguousarray(x0, dtype=np.int32)
    y = np.ascontiguousarray(y, dtype=np.int32)
    c = np.ascontiguousarray(c, dtype=np.float32)
    per = np.zeros((3, R, gamma))
    tot = np.zeros(4)
    rc = lib().orc_train_losses(R, gamma, V, r, dtype_code(U), float(temp), _ptr(U), _ptr(W1),
                                _ptr(W2), _ptr(x0, C.c_int32), _ptr(y, C.c_int32), _ptr(P),
                                _ptr(c, C.c_float), float(alpha[0]), float(alpha[1]),
                                float(alpha[2]), _ptr(per, C.c_double), _ptr(tot, C.c_double))
    assert rc == 0, "oracle train_losses rejected its arguments"
    return per, tot



# ---------------------------------------------------------- recurrent head
def rnn_states(G_E, G_h_req, W_hh, b_hh, x0, x, s0=None):
    """GRU states s_1..s_gamma of one request (fp64 [gamma][r]).  G_E [V][3r]
    (float32 or bf16 bits), G_h_req [gamma][3r] fp32, W_hh [r][3r] column-major
    (same dtype as G_E), b_hh [3r] fp32, s0 [r] fp32 or None; tokens x0, then
    x[0..gamma-2]."""
    gamma, g3 = G_h_req.shape
    r = g3 // 3
    V = G_E.shape[0]
    G_E, W_hh = np.ascontiguousarray(G_E), np.ascontiguousarray(W_hh)
    assert G_E.shape == (V, g3) and W_hh.shape == (r, g3) and W_hh.dtype == G_E.dtype
    G_h_req = np.ascontiguousarray(G_h_req, dtype=np.float32)
    b_hh = np.ascontiguousarray(b_hh, dtype=np.float32)
    x = np.ascontiguousarray(np.resize(np.asarray(x, dtype=np.int32), max(gamma - 1, 1)))
    s0 = None if s0 is None else np.ascontiguousarray(s0, dtype=np.float32)
    out = np.zeros((gamma, r))
    rc = lib().orc_rnn_states(gamma, V, r, dtype_code(G_E), _ptr(G_E), _ptr(G_h_req, C.c_float),
                              _ptr(W_hh), _ptr(b_hh, C.c_float), int(x0), _ptr(x, C.c_int32),
                              _ptr(s0, C.c_float), _ptr(out, C.c_double))
    assert rc == 0, "oracle rnn_states rejected its arguments"
    return out
