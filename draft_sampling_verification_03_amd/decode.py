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
"""
import numpy as np
import torch

from . import _abi as A
from . import api


def decode(rounds, x0, W1, W2, U_of_round, target_rows, *, SPS=None, mode=0, threshold=0.0,
           conf_of_round=None, temp=1.0, seed=0, first_round=0, stream=None):
    """Run `rounds` rounds for R requests.

    x0            [R] int32 anchors of the first round (host or device)
    W1, W2        draft head factors, device tensors as for api.draft
    U_of_round    t -> U [R][gamma][V] device tensor of round t
    target_rows   prev (host int64 array of previous tokens) -> [len(prev)][V]
                  device tensor: the target logits after each given token
    conf_of_round t -> c [R][gamma] float32 device tensor (None: scheduler off)
    mode          scheduler mode (ASYNC_TOPK reads the confidences of round t - 2;
                  THRESHOLD keeps each request's leading drafts with c >= threshold)

    Returns a dict of per-round host arrays (ell, n_acc, y, theta, n_admitted)
    and the emitted token stream of every request (anchors excluded)."""
    ws_d, ws_s, ws_v = api.Workspace(), api.Workspace(), api.Workspace()
    anchors = torch.as_tensor(np.asarray(x0, dtype=np.int32) if not torch.is_tensor(x0) else x0)
    anchors = anchors.to(W1.device, dtype=torch.int32).contiguous()
    R = anchors.numel()
    streams = [[] for _ in range(R)]
    rec = dict(ell=[], n_acc=[], y=[], theta=[], n_admitted=[], x=[])
    for i in range(rounds):
        t = first_round + i
        U = U_of_round(t)
        gamma = U.shape[1]
        d = api.draft(U, W1, W2, anchors, temp=temp, seed=seed, round=t, ws=ws_d, stream=stream)
        c = conf_of_round(t) if conf_of_round is not None else None
        # the asynchronous top-K scheduler reads round t - 2's confidences (for
        # the first rounds the callable supplies an earlier history)
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
    out = {k: np.asarray(v) for k, v in rec.items()}
    out["streams"] = streams
    errs = (ws_d.error_code(stream), ws_s.error_code(stream), ws_v.error_code(stream))
    out["device_errors"] = errs
    return out
