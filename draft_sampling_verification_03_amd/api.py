"""torch-facing wrappers over the C ABI: allocate outputs and workspaces with
torch (device memory and streams only) and call the dspark_* entry points.
No arithmetic of the method happens here.

Every tensor argument is checked before anything is launched: element type,
shape, contiguity, and that it lives on the same GPU as the call's first
logit array (a host address or a strided view handed to a kernel would be
misread or fault).  A wrong element type raises TypeError, anything else
ValueError.  Outputs and workspaces are allocated on the launch stream, so
their zero-fills and first uses are ordered before the kernels.
"""
import contextlib

import torch

from . import _abi as A

_ANY = None  # a dimension of any size


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


def _on_stream(stream):
    """Context that makes `stream` current for torch's allocations and fills."""
    if stream is None or not isinstance(stream, torch.cuda.Stream):
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


class _Args:
    """Collects the tensors of one call and checks them in a fixed order:
    dtype, shape, contiguity (each as it is added), then one device for all."""

    def __init__(self, where):
        self.where = where
        self.tensors = []

    def req(self, t, name, dtype, shape, optional=False):
        if t is None:
            if optional:
                return None
            raise ValueError(f"{self.where}: {name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.where}: {name} must be a torch.Tensor, got {type(t).__name__}")
        if t.dtype != dtype:
            raise TypeError(f"{self.where}: {name} must be {dtype}, got {t.dtype}")
        if len(shape) != t.dim() or any(s is not None and s != d for s, d in zip(shape, t.shape)):
            want = "[" + ", ".join("*" if s is None else str(s) for s in shape) + "]"
            raise ValueError(f"{self.where}: {name} must have shape {want}, got {list(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{self.where}: {name} must be contiguous")
        self.tensors.append((name, t))
        return t

    def device(self):
        """The common CUDA device of every tensor checked so far."""
        name0, t0 = self.tensors[0]
        if not t0.is_cuda:
            raise ValueError(f"{self.where}: {name0} is not a GPU tensor (device {t0.device})")
        for name, t in self.tensors[1:]:
            if t.device != t0.device:
                raise ValueError(f"{self.where}: {name} is on {t.device}, {name0} on {t0.device}")
        return t0.device


class Workspace:
    """Device scratch for one entry point, zeroed once at allocation (the sticky
    error word lives in its first 256 bytes); grows on demand.  The buffer is
    allocated and zeroed on the stream of the call that needs it; a call on
    another stream marks it as used there."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None
        self._streams = set()

    def get(self, nbytes, stream=None, device=None):
        dev = device if device is not None else self.device
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(dev):
            with _on_stream(stream):
                self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
            self._streams = {id(stream)}
        elif isinstance(stream, torch.cuda.Stream) and id(stream) not in self._streams:
            self.buf.record_stream(stream)
            self._streams.add(id(stream))
        return self.buf

    def error_code(self, stream=None):
        st, code = A.dspark_device_error(self.buf, _stream(stream))
        _check(st, "dspark_device_error")
        return code

    def clear_error(self, stream=None):
        _check(A.dspark_clear_device_error(self.buf, _stream(stream)), "dspark_clear_device_error")


def _empty(shape, dtype, dev):
    return torch.empty(shape, dtype=dtype, device=dev)


def _outputs(args, out, spec, dev):
    """Allocate the outputs of `spec` ({name: (shape, dtype)}) or check the
    caller's (None entries of spec are outputs the call does not produce)."""
    if out is None:
        return {k: (None if v is None else _empty(v[0], v[1], dev)) for k, v in spec.items()}
    for k, v in spec.items():
        if v is not None:
            args.req(out.get(k), f"out[{k!r}]", v[1], v[0])
    return out


I32, F32, F64 = torch.int32, torch.float32, torch.float64


def draft(U, W1, W2, x0, *, temp=1.0, seed=0, round=0, h=None, w_conf=None, b_conf=0.0,
          conf_temp=None, ws=None, stream=None, out=None):
    """U [R][gamma][V], W1 [V][r], W2 column-major ([V][r] storage), x0 [R] int32;
    h [R][gamma][d] (U's dtype) with w_conf [d + r] fp32 for the confidence head;
    conf_temp [gamma] fp32 per-position temperatures of the confidence head."""
    a = _Args("draft")
    if not isinstance(U, torch.Tensor) or U.dim() != 3:
        raise ValueError("draft: U must be a [R][gamma][V] tensor")
    R, gamma, V = U.shape
    dt_t = U.dtype
    dt = _dt(U)
    a.req(U, "U", dt_t, (R, gamma, V))
    if not isinstance(W1, torch.Tensor) or W1.dim() != 2:
        raise ValueError("draft: W1 must be a [V][r] tensor")
    r = W1.shape[1]
    a.req(W1, "W1", dt_t, (V, r))
    a.req(W2, "W2", dt_t, (V, r))
    a.req(x0, "x0", I32, (R,))
    d = 0
    if h is not None:
        if not isinstance(h, torch.Tensor) or h.dim() != 3:
            raise ValueError("draft: h must be a [R][gamma][d] tensor")
        d = h.shape[-1]
        a.req(h, "h", dt_t, (R, gamma, d))
        a.req(w_conf, "w_conf", F32, (d + r,))
        a.req(conf_temp, "conf_temp", F32, (gamma,), optional=True)
    dev = a.device()
    with _on_stream(stream):
        out = _outputs(a, out, dict(x=((R, gamma), I32), q_stats=((R, gamma, 2), F32),
                                    q_x=((R, gamma), F32),
                                    c=((R, gamma), F32) if h is not None else None), dev)
        if h is None:
            out.setdefault("c", None)
        a.device()
        ws = ws or Workspace(dev)
        buf = ws.get(A.dspark_draft_workspace(R, gamma, V, r, dt), stream, dev)
    st = A.dspark_draft(R, gamma, V, r, dt, float(temp), U, W1, W2, x0, h, d, w_conf, float(b_conf),
                        conf_temp if h is not None else None, int(seed), int(round), out["x"],
                        out["q_stats"], out["q_x"], out["c"] if h is not None else None, buf,
                        buf.numel(), _stream(stream))
    _check(st, "dspark_draft")
    return out


def schedule(c, SPS, mode, *, c_prev2=None, R=None, gamma=None, ws=None, stream=None, out=None,
             want_a=True, threshold=0.0):
    """c [R][gamma] fp32 (None in OFF mode with R, gamma given); SPS fp64 table
    [B_max + 1]; c_prev2 [R][gamma] fp32 (ASYNC_TOPK); threshold: the THRESHOLD
    mode's cutoff."""
    a = _Args("schedule")
    if c is not None:
        if not isinstance(c, torch.Tensor) or c.dim() != 2:
            raise ValueError("schedule: c must be a [R][gamma] tensor")
        R, gamma = c.shape
        a.req(c, "c", F32, (R, gamma))
    elif R is None or gamma is None:
        raise ValueError("schedule: R and gamma are required when c is None")
    if SPS is not None:
        a.req(SPS, "SPS", F64, (_ANY,))
    if int(mode) == A.DSPARK_SCHED_ASYNC_TOPK:
        a.req(c_prev2, "c_prev2", F32, (R, gamma))
    if a.tensors:
        dev = a.device()
    else:
        dev = torch.device("cuda", torch.cuda.current_device())
    with _on_stream(stream):
        out = _outputs(a, out, dict(ell=((R,), I32), row_offset=((R + 1,), I32),
                                    a=((R, gamma), F32) if (c is not None and want_a) else None,
                                    n_admitted=((1,), I32), theta=((1,), F64)), dev)
        out.setdefault("a", None)
        if a.tensors:
            a.device()
        ws = ws or Workspace(dev)
        buf = ws.get(A.dspark_schedule_workspace(R, gamma), stream, dev)
    B_max = 0 if SPS is None else SPS.numel() - 1
    st = A.dspark_schedule(R, gamma, int(mode), float(threshold), c,
                           c_prev2 if int(mode) == A.DSPARK_SCHED_ASYNC_TOPK else None, SPS, B_max,
                           out["ell"], out["row_offset"], out["a"] if c is not None else None,
                           out["n_admitted"], out["theta"], buf, buf.numel(), _stream(stream))
    _check(st, "dspark_schedule")
    return out


def _verify_common(where, ell, row_offset, P, U, x0, x, q_stats, q_x, rows_capacity):
    a = _Args(where)
    if not isinstance(U, torch.Tensor) or U.dim() != 3:
        raise ValueError(f"{where}: U must be a [R][gamma][V] tensor")
    R, gamma, V = U.shape
    a.req(U, "U", U.dtype, (R, gamma, V))
    _dt(U)
    a.req(ell, "ell", I32, (R,))
    a.req(row_offset, "row_offset", I32, (R + 1,))
    if not isinstance(P, torch.Tensor) or P.dim() != 2:
        raise ValueError(f"{where}: P must be a [rows][V] tensor")
    a.req(P, "P", U.dtype, (_ANY, V))
    rows_capacity = P.shape[0] if rows_capacity is None else int(rows_capacity)
    if rows_capacity > P.shape[0]:
        raise ValueError(f"{where}: rows_capacity {rows_capacity} exceeds P's {P.shape[0]} rows")
    a.req(x0, "x0", I32, (R,))
    a.req(x, "x", I32, (R, gamma))
    a.req(q_stats, "q_stats", F32, (R, gamma, 2))
    a.req(q_x, "q_x", F32, (R, gamma))
    return a, R, gamma, V, rows_capacity


def verify(ell, row_offset, P, U, W1, W2, x0, x, q_stats, q_x, *, rows_capacity=None, temp=1.0,
           seed=0, round=0, ws=None, stream=None, out=None):
    """P [rows_capacity][V] flattened target rows; other inputs as for draft."""
    a, R, gamma, V, rows_capacity = _verify_common("verify", ell, row_offset, P, U, x0, x, q_stats,
                                                   q_x, rows_capacity)
    if not isinstance(W1, torch.Tensor) or W1.dim() != 2:
        raise ValueError("verify: W1 must be a [V][r] tensor")
    r = W1.shape[1]
    a.req(W1, "W1", U.dtype, (V, r))
    a.req(W2, "W2", U.dtype, (V, r))
    dt = _dt(U)
    dev = a.device()
    with _on_stream(stream):
        out = _outputs(a, out, dict(n_acc=((R,), I32), y=((R, gamma + 1), I32),
                                    c_star=((R, gamma), F32)), dev)
        a.device()
        ws = ws or Workspace(dev)
        buf = ws.get(A.dspark_verify_workspace(R, gamma, V, rows_capacity), stream, dev)
    st = A.dspark_verify(R, gamma, V, r, dt, float(temp), ell, row_offset, rows_capacity, P, U, W1,
                         W2, x0, x, q_stats, q_x, int(seed), int(round), out["n_acc"], out["y"],
                         out["c_star"], buf, buf.numel(), _stream(stream))
    _check(st, "dspark_verify")
    return out


def tv_overlap(P, Q, *, p_stats=None, q_stats=None, temp=1.0, ws=None, stream=None, out=None):
    """P, Q [n_rows][V] logits (one dtype); p_stats, q_stats [n_rows][2] fp32, both or neither."""
    a = _Args("tv_overlap")
    if not isinstance(P, torch.Tensor) or P.dim() != 2:
        raise ValueError("tv_overlap: P must be a [n_rows][V] tensor")
    n_rows, V = P.shape
    a.req(P, "P", P.dtype, (n_rows, V))
    dt = _dt(P)
    a.req(Q, "Q", P.dtype, (n_rows, V))
    if (p_stats is None) != (q_stats is None):
        raise ValueError("tv_overlap: give both p_stats and q_stats, or neither")
    a.req(p_stats, "p_stats", F32, (n_rows, 2), optional=True)
    a.req(q_stats, "q_stats", F32, (n_rows, 2), optional=True)
    dev = a.device()
    with _on_stream(stream):
        if out is None:
            out = _empty(n_rows, F32, dev)
        else:
            a.req(out, "out", F32, (n_rows,))
            a.device()
        ws = ws or Workspace(dev)
        buf = ws.get(A.dspark_tv_overlap_workspace(n_rows, V), stream, dev)
    st = A.dspark_tv_overlap(n_rows, V, dt, float(temp), P, Q, p_stats, q_stats, out, buf,
                             buf.numel(), _stream(stream))
    _check(st, "dspark_tv_overlap")
    return out


def train_losses(U, W1, W2, P, x0, y, c, *, temp=1.0, alpha=(0.1, 0.9, 1.0), per_pos=True,
                 ws=None, stream=None, out=None):
    """Forward-only training losses on the label prefix.  U [R][gamma][V], P
    [R][gamma + 1][V] or [R (gamma + 1)][V] (position k of request rho at row
    rho (gamma + 1) + k - 1), y [R][gamma] int32 labels, c [R][gamma] fp32
    confidences.  Returns {"per_pos": [3][R][gamma] (CE, L1, BCE) or None,
    "totals": [4] fp64 (L_ce, L_tv, L_conf, L)}."""
    a = _Args("train_losses")
    if not isinstance(U, torch.Tensor) or U.dim() != 3:
        raise ValueError("train_losses: U must be a [R][gamma][V] tensor")
    R, gamma, V = U.shape
    a.req(U, "U", U.dtype, (R, gamma, V))
    dt = _dt(U)
    if not isinstance(W1, torch.Tensor) or W1.dim() != 2:
        raise ValueError("train_losses: W1 must be a [V][r] tensor")
    r = W1.shape[1]
    a.req(W1, "W1", U.dtype, (V, r))
    a.req(W2, "W2", U.dtype, (V, r))
    if isinstance(P, torch.Tensor) and P.dim() == 3:
        a.req(P, "P", U.dtype, (R, gamma + 1, V))
    else:
        a.req(P, "P", U.dtype, (R * (gamma + 1), V))
    a.req(x0, "x0", I32, (R,))
    a.req(y, "y", I32, (R, gamma))
    a.req(c, "c", F32, (R, gamma))
    dev = a.device()
    with _on_stream(stream):
        out = _outputs(a, out, dict(per_pos=((3, R, gamma), F32) if per_pos else None,
                                    totals=((4,), F64)), dev)
        out.setdefault("per_pos", None)
        a.device()
        ws = ws or Workspace(dev)
        buf = ws.get(A.dspark_train_losses_workspace(R, gamma, V), stream, dev)
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
    a = _Args("draft_rnn")
    if not isinstance(U, torch.Tensor) or U.dim() != 3:
        raise ValueError("draft_rnn: U must be a [R][gamma][V] tensor")
    R, gamma, V = U.shape
    a.req(U, "U", U.dtype, (R, gamma, V))
    dt = _dt(U)
    if not isinstance(W_o, torch.Tensor) or W_o.dim() != 2:
        raise ValueError("draft_rnn: W_o must be a [V][r] tensor")
    r = W_o.shape[1]
    a.req(W_o, "W_o", U.dtype, (V, r))
    a.req(G_E, "G_E", U.dtype, (V, 3 * r))
    a.req(G_h, "G_h", F32, (R, gamma, 3 * r))
    a.req(W_hh, "W_hh", U.dtype, (r, 3 * r))
    a.req(b_hh, "b_hh", F32, (3 * r,))
    a.req(x0, "x0", I32, (R,))
    a.req(s0, "s0", F32, (R, r), optional=True)
    dev = a.device()
    with _on_stream(stream):
        out = _outputs(a, out, dict(x=((R, gamma), I32), q_stats=((R, gamma, 2), F32),
                                    q_x=((R, gamma), F32), s=((R, gamma, r), F32),
                                    A=((gamma, R, r), U.dtype)), dev)
        a.device()
        ws = ws or Workspace(dev)
        buf = ws.get(A.dspark_draft_workspace(R, gamma, V, r, dt), stream, dev)
    st = A.dspark_draft_rnn(R, gamma, V, r, dt, float(temp), U, W_o, G_E, G_h, W_hh, b_hh, x0, s0,
                            int(seed), int(round), out["x"], out["q_stats"], out["q_x"], out["s"],
                            out["A"], buf, buf.numel(), _stream(stream))
    _check(st, "dspark_draft_rnn")
    return out


def verify_rnn(ell, row_offset, P, U, A_rows, W_o, x0, x, q_stats, q_x, *, rows_capacity=None,
               temp=1.0, seed=0, round=0, ws=None, stream=None, out=None):
    """verify() for recurrent-head drafts: A_rows [gamma][R][r] from draft_rnn."""
    a, R, gamma, V, rows_capacity = _verify_common("verify_rnn", ell, row_offset, P, U, x0, x,
                                                   q_stats, q_x, rows_capacity)
    if not isinstance(W_o, torch.Tensor) or W_o.dim() != 2:
        raise ValueError("verify_rnn: W_o must be a [V][r] tensor")
    r = W_o.shape[1]
    a.req(W_o, "W_o", U.dtype, (V, r))
    a.req(A_rows, "A_rows", U.dtype, (gamma, R, r))
    dt = _dt(U)
    dev = a.device()
    with _on_stream(stream):
        out = _outputs(a, out, dict(n_acc=((R,), I32), y=((R, gamma + 1), I32),
                                    c_star=((R, gamma), F32)), dev)
        a.device()
        ws = ws or Workspace(dev)
        buf = ws.get(A.dspark_verify_workspace(R, gamma, V, rows_capacity), stream, dev)
    st = A.dspark_verify_rnn(R, gamma, V, r, dt, float(temp), ell, row_offset, rows_capacity, P, U,
                             A_rows, W_o, x0, x, q_stats, q_x, int(seed), int(round),
                             out["n_acc"], out["y"], out["c_star"], buf, buf.numel(),
                             _stream(stream))
    _check(st, "dspark_verify_rnn")
    return out
