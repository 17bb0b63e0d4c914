"""torch-facing wrappers over the C ABI: allocate outputs and workspaces with
torch (device memory and streams only) and call the dspark_* entry points.
No arithmetic of the method happens here."""
import torch

from . import _abi as A


def _dt(t):
    if t.dtype == torch.bfloat16:
        return A.DSPARK_BF16
    if t.dtype == torch.float32:
        return A.DSPARK_F32
    raise TypeError(f"logits and weights must be bfloat16 or float32, got {t.dtype}")


def _check(status, where):
    if status != 0:
        raise A.DSparkError(status, where)


def _stream(stream):
    return torch.cuda.current_stream() if stream is None else stream


class Workspace:
    """Device scratch for one entry point, zeroed once at allocation (the sticky
    error word lives in its first 256 bytes); grows on demand."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf

    def error_code(self, stream=None):
        st, code = A.dspark_device_error(self.buf, _stream(stream))
        _check(st, "dspark_device_error")
        return code

    def clear_error(self, stream=None):
        _check(A.dspark_clear_device_error(self.buf, _stream(stream)), "dspark_clear_device_error")


def draft(U, W1, W2, x0, *, temp=1.0, seed=0, round=0, h=None, w_conf=None, b_conf=0.0,
          conf_temp=None, ws=None, stream=None, out=None):
    """U [R][gamma][V], W1 [V][r], W2 column-major ([V][r] storage), x0 [R] int32;
    conf_temp [gamma] fp32 per-position temperatures of the confidence head."""
    R, gamma, V = U.shape
    r = W1.shape[1]
    dt = _dt(U)
    dev = U.device
    if out is None:
        out = dict(x=torch.empty((R, gamma), dtype=torch.int32, device=dev),
                   q_stats=torch.empty((R, gamma, 2), dtype=torch.float32, device=dev),
                   q_x=torch.empty((R, gamma), dtype=torch.float32, device=dev),
                   c=torch.empty((R, gamma), dtype=torch.float32, device=dev) if h is not None else None)
    ws = ws or Workspace(dev)
    nbytes = A.dspark_draft_workspace(R, gamma, V, r, dt)
    buf = ws.get(nbytes)
    d = 0 if h is None else h.shape[-1]
    st = A.dspark_draft(R, gamma, V, r, dt, float(temp), U, W1, W2, x0, h, d, w_conf, float(b_conf),
                        conf_temp, int(seed), int(round), out["x"], out["q_stats"], out["q_x"],
                        out["c"], buf,
                        buf.numel(), _stream(stream))
    _check(st, "dspark_draft")
    return out


def schedule(c, SPS, mode, *, c_prev2=None, R=None, gamma=None, ws=None, stream=None, out=None,
             want_a=True, threshold=0.0):
    """c [R][gamma] fp32 (None in OFF mode with R, gamma given); SPS fp64 table;
    threshold: the THRESHOLD mode's cutoff."""
    if c is not None:
        R, gamma = c.shape
        dev = c.device
    else:
        dev = SPS.device if SPS is not None else torch.device("cuda")
    if out is None:
        out = dict(ell=torch.empty(R, dtype=torch.int32, device=dev),
                   row_offset=torch.empty(R + 1, dtype=torch.int32, device=dev),
                   a=torch.empty((R, gamma), dtype=torch.float32, device=dev)
                   if (c is not None and want_a) else None,
                   n_admitted=torch.empty(1, dtype=torch.int32, device=dev),
                   theta=torch.empty(1, dtype=torch.float64, device=dev))
    ws = ws or Workspace(dev)
    buf = ws.get(A.dspark_schedule_workspace(R, gamma))
    B_max = 0 if SPS is None else SPS.numel() - 1
    st = A.dspark_schedule(R, gamma, int(mode), float(threshold), c, c_prev2, SPS, B_max, out["ell"],
                           out["row_offset"], out["a"], out["n_admitted"], out["theta"], buf,
                           buf.numel(), _stream(stream))
    _check(st, "dspark_schedule")
    return out


def verify(ell, row_offset, P, U, W1, W2, x0, x, q_stats, q_x, *, rows_capacity=None, temp=1.0,
           seed=0, round=0, ws=None, stream=None, out=None):
    """P [rows_capacity][V] flattened target rows; other inputs as for draft."""
    R, gamma, V = U.shape
    r = W1.shape[1]
    dt = _dt(U)
    dev = U.device
    rows_capacity = P.shape[0] if rows_capacity is None else rows_capacity
    if out is None:
        out = dict(n_acc=torch.empty(R, dtype=torch.int32, device=dev),
                   y=torch.empty((R, gamma + 1), dtype=torch.int32, device=dev),
                   c_star=torch.empty((R, gamma), dtype=torch.float32, device=dev))
    ws = ws or Workspace(dev)
    buf = ws.get(A.dspark_verify_workspace(R, gamma, V, rows_capacity))
    st = A.dspark_verify(R, gamma, V, r, dt, float(temp), ell, row_offset, rows_capacity, P, U, W1,
                         W2, x0, x, q_stats, q_x, int(seed), int(round), out["n_acc"], out["y"],
                         out["c_star"], buf, buf.numel(), _stream(stream))
    _check(st, "dspark_verify")
    return out


def tv_overlap(P, Q, *, p_stats=None, q_stats=None, temp=1.0, ws=None, stream=None, out=None):
    n_rows, V = P.shape
    dt = _dt(P)
    if out is None:
        out = torch.empty(n_rows, dtype=torch.float32, device=P.device)
    ws = ws or Workspace(P.device)
    buf = ws.get(A.dspark_tv_overlap_workspace(n_rows, V))
    st = A.dspark_tv_overlap(n_rows, V, dt, float(temp), P, Q, p_stats, q_stats, out, buf,
                             buf.numel(), _stream(stream))
    _check(st, "dspark_tv_overlap")
    return out


def train_losses(U, W1, W2, P, x0, y, c, *, temp=1.0, alpha=(0.1, 0.9, 1.0), per_pos=True,
                 ws=None, stream=None, out=None):
    """Forward-only training losses on the label prefix.  U [R][gamma][V], P
    [R][gamma + 1][V] (position k of request rho at row rho (gamma + 1) + k - 1),
    y [R][gamma] int32 labels, c [R][gamma] fp32 confidences.  Returns
    {"per_pos": [3][R][gamma] (CE, L1, BCE) or None, "totals": [4] fp64
    (L_ce, L_tv, L_conf, L)}."""
    R, gamma, V = U.shape
    r = W1.shape[1]
    dt = _dt(U)
    dev = U.device
    if out is None:
        out = dict(per_pos=torch.empty((3, R, gamma), dtype=torch.float32, device=dev)
                   if per_pos else None,
                   totals=torch.empty(4, dtype=torch.float64, device=dev))
    ws = ws or Workspace(dev)
    buf = ws.get(A.dspark_train_losses_workspace(R, gamma, V))
    st = A.dspark_train_losses(R, gamma, V, r, dt, float(temp), U, W1, W2, P, x0, y, c,
                               float(alpha[0]), float(alpha[1]), float(alpha[2]), out["per_pos"],
                               out["totals"], buf, buf.numel(), _stream(stream))
    _check(st, "dspark_train_losses")
    return out


def draft_rnn(U, W_o, G_E, G_h, W_hh, b_hh, x0, *, s0=None, temp=1.0, seed=0, round=0, ws=None,
              stream=None, out=None):
    """Draft with the recurrent head.  U [R][gamma][V], W_o [V][r] storage
    (column-major r x V), G_E [V][3r], G_h [R][gamma][3r] fp32, W_hh [r][3r]
    storage, b_hh [3r] fp32, x0 [R] int32, s0 [R][r] fp32 or None.  Returns x,
    q_stats, q_x, s [R][gamma][r] fp32 and A [gamma][R][r] (U's dtype)."""
    R, gamma, V = U.shape
    r = W_o.shape[1]
    dt = _dt(U)
    dev = U.device
    if out is None:
        out = dict(x=torch.empty((R, gamma), dtype=torch.int32, device=dev),
                   q_stats=torch.empty((R, gamma, 2), dtype=torch.float32, device=dev),
                   q_x=torch.empty((R, gamma), dtype=torch.float32, device=dev),
                   s=torch.empty((R, gamma, r), dtype=torch.float32, device=dev),
                   A=torch.empty((gamma, R, r), dtype=U.dtype, device=dev))
    ws = ws or Workspace(dev)
    buf = ws.get(A.dspark_draft_workspace(R, gamma, V, r, dt))
    st = A.dspark_draft_rnn(R, gamma, V, r, dt, float(temp), U, W_o, G_E, G_h, W_hh, b_hh, x0, s0,
                            int(seed), int(round), out["x"], out["q_stats"], out["q_x"], out["s"],
                            out["A"], buf, buf.numel(), _stream(stream))
    _check(st, "dspark_draft_rnn")
    return out


def verify_rnn(ell, row_offset, P, U, A_rows, W_o, x0, x, q_stats, q_x, *, rows_capacity=None,
               temp=1.0, seed=0, round=0, ws=None, stream=None, out=None):
    """verify() for recurrent-head drafts: A_rows [gamma][R][r] from draft_rnn."""
    R, gamma, V = U.shape
    r = W_o.shape[1]
    dt = _dt(U)
    dev = U.device
    rows_capacity = P.shape[0] if rows_capacity is None else rows_capacity
    if out is None:
        out = dict(n_acc=torch.empty(R, dtype=torch.int32, device=dev),
                   y=torch.empty((R, gamma + 1), dtype=torch.int32, device=dev),
                   c_star=torch.empty((R, gamma), dtype=torch.float32, device=dev))
    ws = ws or Workspace(dev)
    buf = ws.get(A.dspark_verify_workspace(R, gamma, V, rows_capacity))
    st = A.dspark_verify_rnn(R, gamma, V, r, dt, float(temp), ell, row_offset, rows_capacity, P, U,
                             A_rows, W_o, x0, x, q_stats, q_x, int(seed), int(round),
                             out["n_acc"], out["y"], out["c_star"], buf, buf.numel(),
                             _stream(stream))
    _check(st, "dspark_verify_rnn")
    return out
