"""Many rounds of speculative decoding with the hot path: the multi-round loop
around dspark_draft -> dspark_schedule -> (target forward) -> dspark_verify.

The pages' decoding loop (Blog, "Lossless speculative decoding" and "Dynamic
block scheduling"; Bangkok 4.2) feeds each round's emitted tokens back as the
next round's anchors, and the asynchronous top-K scheduler reads the
confidences of round t - 2.  This module is that loop, nothing more: every
step of the method runs in the library's kernels; the target forward is the
caller's (a callable that returns the target logits of the scheduled rows).
Tokens and lengths come back to the host once per round, because the next
round's target rows depend on them.

Confidence history.  Without a trained confidence head, the loop can supply
its own: per request and draft position, the empirical conditional acceptance
P(A_k | A_1..A_{k-1}) = (# rounds position k was accepted) / (# rounds it was
verified after positions 1..k-1 were accepted) (Blog, "Conditional acceptance
curves"), with a Beta(alpha, beta) prior so that an untried position starts at
alpha / (alpha + beta).  Round t schedules with the estimate from rounds
before t, and the asynchronous top-K mode reads the estimate as it stood at
round t - 2 (Blog, "Async scheduler in practice").  The estimate is formed
from integer counts in float64 and rounded once to float32.
"""
import numpy as np
import torch

from . import _abi as A
from . import api


class AcceptanceHistory:
    """Per-request, per-position counts of verified and accepted draft positions."""

    def __init__(self, R, gamma, alpha=4.0, beta=1.0):
        self.alpha, self.beta = float(alpha), float(beta)
        self.tried = np.zeros((R, gamma), dtype=np.int64)
        self.passed = np.zeros((R, gamma), dtype=np.int64)

    def confidences(self):
        """[R][gamma] float32 conditional-acceptance estimates."""
        return ((self.passed + self.alpha) / (self.tried + self.alpha + self.beta)).astype(np.float32)

    def record(self, ell, n_acc):
        """Position k (1-based) is verified when k <= ell and the k - 1 before it
        were accepted, and accepted when k <= n_acc."""
        k = np.arange(1, self.tried.shape[1] + 1)[None, :]
        ell, n_acc = np.asarray(ell)[:, None], np.asarray(n_acc)[:, None]
        self.tried += (k <= ell) & (k - 1 <= n_acc)
        self.passed += k <= n_acc

    def curve(self):
        """P(A_k | A_1..A_{k-1}) over all requests (nan where never verified)."""
        t = self.tried.sum(axis=0)
        with np.errstate(invalid="ignore", divide="ignore"):
            return np.where(t > 0, self.passed.sum(axis=0) / np.maximum(t, 1), np.nan)


def decode(rounds, x0, W1, W2, U_of_round, target_rows, *, SPS=None, mode=0, threshold=0.0,
           conf_of_round=None, history=None, temp=1.0, seed=0, first_round=0, stream=None):
    """Run `rounds` rounds for R requests.

    x0            [R] int32 anchors of the first round (host or device)
    W1, W2        draft head factors, device tensors as for api.draft
    U_of_round    t -> U [R][gamma][V] device tensor of round t
    target_rows   prev (host int64 array of previous tokens) -> [len(prev)][V]
                  device tensor: the target logits after each given token
    conf_of_round t -> c [R][gamma] float32 device tensor (None: scheduler off)
    history       (alpha, beta): the loop's own conditional-acceptance estimates
                  are the confidences instead (conf_of_round is then ignored)
    mode          scheduler mode (ASYNC_TOPK reads the confidences of round t - 2;
                  THRESHOLD keeps each request's leading drafts with c >= threshold)

    Returns a dict of per-round host arrays (x, ell, n_acc, y, theta,
    n_admitted; with confidences also c and a, the predicted tokens
    tau_pred = sum_r (1 + sum_{k <= ell_r} a_rk) and the realized tau_real =
    sum_r (n_acc_r + 1)), the emitted token stream of every request (anchors
    excluded) and, with a history, its conditional acceptance curve."""
    ws_d, ws_s, ws_v = api.Workspace(), api.Workspace(), api.Workspace()
    anchors = torch.as_tensor(np.asarray(x0, dtype=np.int32) if not torch.is_tensor(x0) else x0)
    anchors = anchors.to(W1.device, dtype=torch.int32).contiguous()
    R = anchors.numel()
    streams = [[] for _ in range(R)]
    rec = dict(ell=[], n_acc=[], y=[], theta=[], n_admitted=[], x=[], c=[], a=[], tau_pred=[],
               tau_real=[])
    hist, past = None, []
    for i in range(rounds):
        t = first_round + i
        U = U_of_round(t)
        gamma = U.shape[1]
        if history is not None and hist is None:
            hist = AcceptanceHistory(R, gamma, *history)
        d = api.draft(U, W1, W2, anchors, temp=temp, seed=seed, round=t, ws=ws_d, stream=stream)
        if hist is not None:
            past.append(hist.confidences())
            c = torch.from_numpy(past[-1]).to(W1.device)
            # round t - 2's estimate; before round 2, the prior alone
            cp = (torch.from_numpy(past[-3] if i >= 2 else past[0]).to(W1.device)
                  if mode == A.DSPARK_SCHED_ASYNC_TOPK else None)
        else:
            c = conf_of_round(t) if conf_of_round is not None else None
            # the asynchronous top-K scheduler reads round t - 2's confidences
            # (for the first rounds the callable supplies an earlier history)
            cp = conf_of_round(t - 2) if (c is not None and mode == A.DSPARK_SCHED_ASYNC_TOPK) else None
        s = api.schedule(c, SPS, mode if c is not None else 0, c_prev2=cp, R=R, gamma=gamma,
                         ws=ws_s, stream=stream, threshold=threshold)
        ell = s["ell"].cpu().numpy()
        x = d["x"].cpu().numpy()
        a = anchors.cpu().numpy()
        # target row of (rho, k), k = 1..ell+1, is the target after x_{k-1} (x_0 = anchor)
        prev = np.concatenate([np.concatenate(([a[rho]], x[rho, : ell[rho]]))
                               for rho in range(R)]).astype(np.int64)
        P = target_rows(prev)
        v = api.verify(s["ell"], s["row_offset"], P, U, W1, W2, anchors, d["x"], d["q_stats"],
                       d["q_x"], temp=temp, seed=seed, round=t, ws=ws_v, stream=stream)
        n = v["n_acc"].cpu().numpy()
        y = v["y"].cpu().numpy()
        for rho in range(R):
            streams[rho].extend(int(tok) for tok in y[rho, : n[rho] + 1])
        anchors = torch.as_tensor(y[np.arange(R), n]).to(W1.device, dtype=torch.int32)
        rec["ell"].append(ell)
        rec["n_acc"].append(n)
        rec["y"].append(y)
        rec["x"].append(x)
        rec["theta"].append(float(s["theta"].cpu().numpy()[0]))
        rec["n_admitted"].append(int(s["n_admitted"].cpu().numpy()[0]))
        rec["tau_real"].append(int((n + 1).sum()))
        if c is not None and s["a"] is not None:
            a_host = s["a"].cpu().numpy()
            rec["c"].append(c.cpu().numpy())
            rec["a"].append(a_host)
            kk = np.arange(1, gamma + 1)[None, :]
            rec["tau_pred"].append(float(R + np.where(kk <= ell[:, None], a_host.astype(np.float64),
                                                      0.0).sum()))
        if hist is not None:
            hist.record(ell, n)
    out = {k: np.asarray(v) for k, v in rec.items()}
    out["streams"] = streams
    if hist is not None:
        out["cond_accept"] = hist.curve()
        out["history"] = hist
    errs = (ws_d.error_code(stream), ws_s.error_code(stream), ws_v.error_code(stream))
    out["device_errors"] = errs
    return out
