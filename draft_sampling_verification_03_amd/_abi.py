"""ctypes binding of libdspark.so: the C ABI of include/dspark.h, name for name.

Pointer arguments accept an int (a device address), None (NULL) or any
object with ``data_ptr()`` (a torch tensor); streams accept an int handle,
None (the null stream) or an object with ``cuda_stream``.
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdspark.so")

DSPARK_F32, DSPARK_BF16 = 0, 1
(DSPARK_SCHED_OFF, DSPARK_SCHED_EARLY_STOP, DSPARK_SCHED_FULL_SEARCH, DSPARK_SCHED_ASYNC_TOPK,
 DSPARK_SCHED_THRESHOLD) = range(5)
STATUS_NAMES = ["DSPARK_OK", "DSPARK_ERR_NULL", "DSPARK_ERR_SHAPE", "DSPARK_ERR_DTYPE",
                "DSPARK_ERR_VALUE", "DSPARK_ERR_WORKSPACE", "DSPARK_ERR_SPS_TABLE",
                "DSPARK_ERR_MODE", "DSPARK_ERR_ALIGN", "DSPARK_ERR_HIP", "DSPARK_ERR_SCRATCH"]
NOALLOC_SCRATCH_BYTES = 16 << 20  # DSPARK_NOALLOC_SCRATCH_BYTES


class DSparkError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{where}: {name} ({dspark_status_string(status)})")


_lib = None
_vp, _sz, _i, _f, _u64 = C.c_void_p, C.c_size_t, C.c_int, C.c_float, C.c_uint64


def library():
    """Load libdspark.so.  Raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m draft_sampling_verification_03_amd.build` "
                              "(there is no CPU fallback)")
        L = C.CDLL(LIB_PATH)
        L.dspark_status_string.argtypes = [_i]
        L.dspark_status_string.restype = C.c_char_p
        L.dspark_draft_workspace.argtypes = [_i, _i, _i, _i, _i]
        L.dspark_draft_workspace.restype = _sz
        L.dspark_draft.argtypes = ([_i] * 5 + [_f] + [_vp] * 5 + [_i, _vp, _f, _vp, _u64, _u64]
                                   + [_vp] * 5 + [_sz, _vp])
        L.dspark_draft_noalloc_scratch.argtypes = [_i, _i, _i]
        L.dspark_draft_noalloc_scratch.restype = _sz
        L.dspark_draft_noalloc.argtypes = ([_i] * 5 + [_f] + [_vp] * 5 + [_i, _vp, _f, _vp, _u64,
                                           _u64] + [_vp] * 6)
        L.dspark_schedule_workspace.argtypes = [_i, _i]
        L.dspark_schedule_workspace.restype = _sz
        L.dspark_schedule.argtypes = [_i, _i, _i, _f, _vp, _vp, _vp, _i] + [_vp] * 6 + [_sz, _vp]
        L.dspark_verify_workspace.argtypes = [_i, _i, _i, _i]
        L.dspark_verify_workspace.restype = _sz
        L.dspark_verify.argtypes = ([_i] * 5 + [_f, _vp, _vp, _i] + [_vp] * 8 + [_u64, _u64]
                                    + [_vp] * 4 + [_sz, _vp])
        L.dspark_tv_overlap_workspace.argtypes = [_i, _i]
        L.dspark_tv_overlap_workspace.restype = _sz
        L.dspark_tv_overlap.argtypes = [_i, _i, _i, _f] + [_vp] * 6 + [_sz, _vp]
        L.dspark_draft_rnn.argtypes = ([_i] * 5 + [_f] + [_vp] * 8 + [_u64, _u64] + [_vp] * 6
                                       + [_sz, _vp])
        L.dspark_verify_rnn.argtypes = L.dspark_verify.argtypes
        L.dspark_train_losses_workspace.argtypes = [_i, _i, _i]
        L.dspark_train_losses_workspace.restype = _sz
        L.dspark_train_losses.argtypes = ([_i] * 5 + [_f] + [_vp] * 7 + [_f, _f, _f]
                                          + [_vp] * 3 + [_sz, _vp])
        L.dspark_device_error.argtypes = [_vp, _vp, _vp]
        L.dspark_clear_device_error.argtypes = [_vp, _vp]
        L.dspark_trace_enable.argtypes = [_i]
        L.dspark_trace_collect.argtypes = []
        L.dspark_trace_entry.argtypes = [_i, C.POINTER(C.c_char_p), C.POINTER(C.c_double),
                                         C.POINTER(C.c_int)]
        for name in ("dspark_draft", "dspark_draft_noalloc", "dspark_schedule", "dspark_verify",
                     "dspark_tv_overlap", "dspark_train_losses", "dspark_draft_rnn", "dspark_verify_rnn",
                     "dspark_device_error", "dspark_clear_device_error", "dspark_trace_enable",
                     "dspark_trace_collect", "dspark_trace_entry"):
            getattr(L, name).restype = _i
        _lib = L
    return _lib


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _s(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dspark_status_string(status):
    return library().dspark_status_string(int(status)).decode()


def dspark_draft_workspace(R, gamma, V, r, dt):
    return library().dspark_draft_workspace(R, gamma, V, r, dt)


def dspark_draft(R, gamma, V, r, dt, temp, U, W1, W2, x0, h, d, w_conf, b_conf, conf_temp, seed,
                 round_, x, q_stats, q_x, c, ws, ws_bytes, stream):
    return library().dspark_draft(R, gamma, V, r, dt, temp, _p(U), _p(W1), _p(W2), _p(x0), _p(h),
                                  d, _p(w_conf), b_conf, _p(conf_temp), seed, round_, _p(x),
                                  _p(q_stats), _p(q_x), _p(c), _p(ws), ws_bytes, _s(stream))


def dspark_draft_noalloc_scratch(R, gamma, V):
    return library().dspark_draft_noalloc_scratch(R, gamma, V)


def dspark_draft_noalloc(R, gamma, V, r, dt, temp, U, W1, W2, x0, h, d, w_conf, b_conf, conf_temp,
                         seed, round_, x, q_stats, q_x, c, dev_error, stream):
    return library().dspark_draft_noalloc(R, gamma, V, r, dt, temp, _p(U), _p(W1), _p(W2), _p(x0),
                                          _p(h), d, _p(w_conf), b_conf, _p(conf_temp), seed,
                                          round_, _p(x), _p(q_stats), _p(q_x), _p(c),
                                          _p(dev_error), _s(stream))


def dspark_schedule_workspace(R, gamma):
    return library().dspark_schedule_workspace(R, gamma)


def dspark_schedule(R, gamma, mode, threshold, c, c_prev2, SPS, B_max, ell, row_offset, a,
                    n_admitted, theta, ws, ws_bytes, stream):
    return library().dspark_schedule(R, gamma, mode, threshold, _p(c), _p(c_prev2), _p(SPS), B_max,
                                     _p(ell),
                                     _p(row_offset), _p(a), _p(n_admitted), _p(theta), _p(ws),
                                     ws_bytes, _s(stream))


def dspark_verify_workspace(R, gamma, V, rows_capacity):
    return library().dspark_verify_workspace(R, gamma, V, rows_capacity)


def dspark_verify(R, gamma, V, r, dt, temp, ell, row_offset, rows_capacity, P, U, W1, W2, x0, x,
                  q_stats, q_x, seed, round_, n_acc, y, c_star, ws, ws_bytes, stream):
    return library().dspark_verify(R, gamma, V, r, dt, temp, _p(ell), _p(row_offset),
                                   rows_capacity, _p(P), _p(U), _p(W1), _p(W2), _p(x0), _p(x),
                                   _p(q_stats), _p(q_x), seed, round_, _p(n_acc), _p(y),
                                   _p(c_star), _p(ws), ws_bytes, _s(stream))


def dspark_tv_overlap_workspace(n_rows, V):
    return library().dspark_tv_overlap_workspace(n_rows, V)


def dspark_tv_overlap(n_rows, V, dt, temp, P, Q, p_stats, q_stats, c_star, ws, ws_bytes, stream):
    return library().dspark_tv_overlap(n_rows, V, dt, temp, _p(P), _p(Q), _p(p_stats),
                                       _p(q_stats), _p(c_star), _p(ws), ws_bytes, _s(stream))


def dspark_draft_rnn(R, gamma, V, r, dt, temp, U, W_o, G_E, G_h, W_hh, b_hh, x0, s0, seed, round_,
                     x, q_stats, q_x, s, A, ws, ws_bytes, stream):
    return library().dspark_draft_rnn(R, gamma, V, r, dt, temp, _p(U), _p(W_o), _p(G_E), _p(G_h),
                                      _p(W_hh), _p(b_hh), _p(x0), _p(s0), seed, round_, _p(x),
                                      _p(q_stats), _p(q_x), _p(s), _p(A), _p(ws), ws_bytes,
                                      _s(stream))


def dspark_verify_rnn(R, gamma, V, r, dt, temp, ell, row_offset, rows_capacity, P, U, A, W_o, x0,
                      x, q_stats, q_x, seed, round_, n_acc, y, c_star, ws, ws_bytes, stream):
    return library().dspark_verify_rnn(R, gamma, V, r, dt, temp, _p(ell), _p(row_offset),
                                       rows_capacity, _p(P), _p(U), _p(A), _p(W_o), _p(x0),
                                       _p(x), _p(q_stats), _p(q_x), seed, round_, _p(n_acc),
                                       _p(y), _p(c_star), _p(ws), ws_bytes, _s(stream))


def dspark_train_losses_workspace(R, gamma, V):
    return library().dspark_train_losses_workspace(R, gamma, V)


def dspark_train_losses(R, gamma, V, r, dt, temp, U, W1, W2, P, x0, y, c, a_ce, a_tv, a_conf,
                        per_pos, totals, ws, ws_bytes, stream):
    return library().dspark_train_losses(R, gamma, V, r, dt, temp, _p(U), _p(W1), _p(W2), _p(P),
                                         _p(x0), _p(y), _p(c), a_ce, a_tv, a_conf, _p(per_pos),
                                         _p(totals), _p(ws), ws_bytes, _s(stream))


def dspark_device_error(ws, stream):
    """Returns (status, code)."""
    code = C.c_int32(0)
    st = library().dspark_device_error(_p(ws), C.addressof(code), _s(stream))
    return st, code.value


def dspark_clear_device_error(ws, stream):
    return library().dspark_clear_device_error(_p(ws), _s(stream))


def dspark_trace_enable(on):
    return library().dspark_trace_enable(1 if on else 0)


def dspark_trace_collect():
    return library().dspark_trace_collect()


def dspark_trace_entry(i):
    """Returns (status, name, total_ms, launches)."""
    name, ms, n = C.c_char_p(), C.c_double(), C.c_int()
    st = library().dspark_trace_entry(i, C.byref(name), C.byref(ms), C.byref(n))
    return st, (name.value.decode() if name.value else None), ms.value, n.value


def trace_summary():
    """{kernel name: (total_ms, launches)} of the records since dspark_trace_enable(1)."""
    n = dspark_trace_collect()
    if n < 0:
        raise DSparkError(9, "dspark_trace_collect")
    out = {}
    for i in range(n):
        st, name, ms, cnt = dspark_trace_entry(i)
        if st == 0:
            out[name] = (ms, cnt)
    return out
