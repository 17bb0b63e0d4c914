#!/usr/bin/env python3
"""Benchmark of the DSpark per-round hot path on one MI355X.

One step = one round of the whole path on resident synthetic inputs:
dspark_draft (gamma Markov-head steps) -> dspark_schedule -> dspark_verify over
the flattened sum(1 + ell) target rows.  The target forward itself is outside
the path: its logits for the scheduled rows are laid out once, before timing
(the schedule is a deterministic function of the inputs, so every step
admits the same rows; the bench checks that after timing).

Prints ONE JSON line: draft+verify positions/s (R * gamma per step), the
per-kernel rooflines (average launch durations measured with HIP events on
the launch stream), the achieved HBM bandwidth of the round, and the CPU
oracle's rate on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft+verify positions/sec at V=151936,R=128,γ=16; achieved HBM GB/s"
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix cores
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload id (3 = R=128, gamma=16)")
    ap.add_argument("--cpu-requests", type=int, default=10,
                    help="requests in the CPU-oracle sample (0 disables)")
    ap.add_argument("--workers", type=int, default=16, help="host threads drawing the inputs")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the recurrent-head and training-reduction passes")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters); not part of the timed steps")
    return ap.parse_args()


def source_hash():
    """Hash of the library's code (comments and blank lines dropped), to tell
    whether hardware counters collected earlier still describe its kernels."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_sampling_verification_03_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f)) as fh:
            code = [re.sub(r"//.*", "", line).rstrip() for line in fh]
        h.update(f.encode() + "\n".join(line for line in code if line).encode())
    return h.hexdigest()[:16]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the hot path has no collective and this build runs on a single MI355X",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_sampling_verification_03_amd as ds
    import synth

    cfg = synth.CONFIGS[args.config]
    R, gamma, V, r = cfg.R, cfg.gamma, cfg.V, cfg.r
    s_el = cfg.elem_bytes()
    nT = (V + 127) // 128
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    t0 = time.time()
    U, T = synth.generate(cfg, workers=args.workers)
    W1, W2, x0 = synth.W1(cfg), synth.W2(cfg), synth.anchors(cfg)
    c, cp, sps = synth.confidences(cfg), synth.confidences(cfg, older=True), synth.sps_table(cfg)
    h = w_conf = b_conf = None
    if cfg.conf == "head":
        h, w_conf, b_conf = synth.head(cfg)
    dU, dW1, dW2, dx0 = up(U), up(W1), up(W2), up(x0)
    dT = up(T.reshape(R * (gamma + 1), V))
    dc = up(c) if c is not None else None
    dcp = up(cp) if (cp is not None and cfg.mode == synth.SCHED_ASYNC_TOPK) else None
    dsps = up(sps) if sps is not None else None
    dh = up(h) if h is not None else None
    dw = up(w_conf) if w_conf is not None else None
    torch.cuda.synchronize()
    print(f"[bench] inputs for {cfg.name} ready in {time.time() - t0:.1f} s", file=sys.stderr,
          flush=True)

    stream = torch.cuda.current_stream()
    wsd, wss, wsv, wso = ds.Workspace(), ds.Workspace(), ds.Workspace(), ds.Workspace()
    if args.copy_calibration_mib > 0:
        # a plain elementwise copy kernel: bf16 -> fp32 conversion of n/2 elements
        # reads n bytes and writes 2n bytes
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
        dst = src.float()
        torch.cuda.synchronize()
        del src, dst

    def draft():
        return ds.draft(dU, dW1, dW2, dx0, temp=cfg.temp, seed=cfg.seed, round=cfg.round, h=dh,
                        w_conf=dw, b_conf=0.0 if b_conf is None else float(b_conf), ws=wsd,
                        stream=stream, out=dout)

    dout = None
    dout = draft()
    c_in = dout["c"] if dh is not None else dc
    sout = ds.schedule(c_in, dsps, cfg.mode, c_prev2=dcp, R=R, gamma=gamma, ws=wss, stream=stream)
    torch.cuda.synchronize()
    ell = sout["ell"].cpu().numpy().copy()
    sum_ell = int(ell.sum())
    idx = np.concatenate([rho * (gamma + 1) + np.arange(int(ell[rho]) + 1) for rho in range(R)])
    P = torch.zeros((cfg.rows_capacity, V), dtype=dT.dtype, device=dev)
    P[: idx.size] = dT.index_select(0, torch.from_numpy(idx).to(dev))
    vout = None

    def schedule():
        return ds.schedule(c_in, dsps, cfg.mode, c_prev2=dcp, R=R, gamma=gamma, ws=wss,
                           stream=stream, out=sout)

    def verify():
        return ds.verify(sout["ell"], sout["row_offset"], P, dU, dW1, dW2, dx0, dout["x"],
                         dout["q_stats"], dout["q_x"], temp=cfg.temp, seed=cfg.seed,
                         round=cfg.round, ws=wsv, stream=stream, out=vout)

    vout = verify()

    def step():
        draft()
        schedule()
        verify()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps back to back, one event pair around
    #      them (an event between entry points costs the stream several us)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for k in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps
    ms_step = max(ms_step, 1e3 * wall / args.steps)

    # ---- per-entry-point breakdown (separate pass, events around each call)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record(stream)
        draft()
        ev[k][1].record(stream)
        schedule()
        ev[k][2].record(stream)
        verify()
        ev[k][3].record(stream)
    torch.cuda.synchronize()
    t_draft = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    t_sched = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    t_ver = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps
    assert np.array_equal(sout["ell"].cpu().numpy(), ell), "schedule changed during timing"
    errs = (wsd.error_code(), wss.error_code(), wsv.error_code())
    assert errs == (0, 0, 0), f"device error words {errs}"

    # ---- the same workload with the scheduler off (ell = gamma for every request:
    #      R * (1 + gamma) target rows, the flattened layout of all positions),
    #      a figure that does not depend on the schedule; separate timed pass
    wss_off, wsv_off = ds.Workspace(), ds.Workspace()
    sout_off = ds.schedule(None, None, synth.SCHED_OFF, R=R, gamma=gamma, ws=wss_off,
                           stream=stream)
    vout_off = None

    def step_off():
        nonlocal vout_off
        draft()
        ds.schedule(None, None, synth.SCHED_OFF, R=R, gamma=gamma, ws=wss_off, stream=stream,
                    out=sout_off)
        vout_off = ds.verify(sout_off["ell"], sout_off["row_offset"], dT, dU, dW1, dW2, dx0,
                             dout["x"], dout["q_stats"], dout["q_x"], temp=cfg.temp,
                             seed=cfg.seed, round=cfg.round, ws=wsv_off, stream=stream,
                             out=vout_off)

    step_off()
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_off = max(1, args.steps // 2)
    e2.record(stream)
    for _ in range(n_off):
        step_off()
    e3.record(stream)
    torch.cuda.synchronize()
    ms_off = e2.elapsed_time(e3) / n_off
    rows_off = R * (gamma + 1)
    assert wsv_off.error_code() == 0, "device error word set in the scheduler-off pass"

    # ---- per-kernel launch durations (HIP events on the launch stream, separate pass)
    ds.dspark_trace_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ds.dspark_trace_enable(False)
    kern = ds.trace_summary()

    # ---- standalone TV overlap on R * gamma logit pairs (statistics supplied)
    n_pairs = R * gamma
    Pp = P[:n_pairs] if P.shape[0] >= n_pairs else P
    Qp = dU.reshape(R * gamma, V)[: Pp.shape[0]]

    def stats(t):
        z = t.float()
        m = z.max(dim=1).values
        return torch.stack([m, torch.exp(z - m[:, None]).sum(dim=1)], dim=1).contiguous()

    ps, qs = stats(Pp), stats(Qp)
    ov_out = ds.tv_overlap(Pp, Qp, p_stats=ps, q_stats=qs, ws=wso, stream=stream)
    ds.dspark_trace_enable(True)
    for _ in range(args.steps):
        ds.tv_overlap(Pp, Qp, p_stats=ps, q_stats=qs, ws=wso, stream=stream, out=ov_out)
    torch.cuda.synchronize()
    ds.dspark_trace_enable(False)
    kern_ov = ds.trace_summary()

    # ---- secondary figures of the next rows on the same workload, separate passes:
    #      a round with the recurrent head (scheduler off, every position verified:
    #      compare with the scheduler-off round above) and the forward-only
    #      training reductions on label prefixes (teacher-forced draft + c*)
    next_rows = None
    if not args.no_next_rows:
        GE, Gh, Whh, bhh, s0, Wo = synth.rnn_head(cfg)
        dGE, dGh, dWhh, dbhh, ds0, dWo = up(GE), up(Gh), up(Whh), up(bhh), up(s0), up(Wo)
        wsr, wsrv, wst = ds.Workspace(), ds.Workspace(), ds.Workspace()
        y_lab = up(np.random.default_rng(11).integers(0, V, (R, gamma)).astype(np.int32))
        c_lab = up(np.random.default_rng(12).uniform(0.05, 0.95, (R, gamma)).astype(np.float32))
        keep = {}

        def rnn_round():
            d = ds.draft_rnn(dU, dWo, dGE, dGh, dWhh, dbhh, dx0, s0=ds0, temp=cfg.temp,
                             seed=cfg.seed, round=cfg.round, ws=wsr, stream=stream,
                             out=keep.get("d"))
            keep["d"] = d
            keep["v"] = ds.verify_rnn(sout_off["ell"], sout_off["row_offset"], dT, dU, d["A"], dWo,
                                      dx0, d["x"], d["q_stats"], d["q_x"], temp=cfg.temp,
                                      seed=cfg.seed, round=cfg.round, ws=wsrv, stream=stream,
                                      out=keep.get("v"))

        def train():
            keep["t"] = ds.train_losses(dU, dW1, dW2, dT, dx0, y_lab, c_lab, temp=cfg.temp,
                                        ws=wst, stream=stream, out=keep.get("t"))

        def timed(fn, n):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n

        n_next = max(1, args.steps // 2)
        ms_rnn, ms_train = timed(rnn_round, n_next), timed(train, n_next)
        assert wsr.error_code() == 0 and wsrv.error_code() == 0 and wst.error_code() == 0, \
            "device error word set in a next-row pass"
        ds.dspark_trace_enable(True)
        rnn_round()
        torch.cuda.synchronize()
        ds.dspark_trace_enable(False)
        kr = ds.trace_summary()
        gru_ms, gru_n = kr.get("gru_step", (float("nan"), 1))
        next_rows = {
            "rnn_head": {"ms_per_round": round(ms_rnn, 4),
                         "positions_per_s": round(R * gamma / (ms_rnn / 1e3), 1),
                         "verify_rows": rows_off, "gru_step_us": round(gru_ms / gru_n * 1e3, 3),
                         "markov_same_rows_ms": round(ms_off, 4)},
            "train_losses": {"ms_per_call": round(ms_train, 4),
                             "positions_per_s": round(R * gamma / (ms_train / 1e3), 1)},
        }
        print(f"[bench] next rows: recurrent-head round {ms_rnn:.3f} ms, "
              f"training reductions {ms_train:.3f} ms", file=sys.stderr, flush=True)

    # ---- algorithmic work per launch of each kernel
    rows_used = R + sum_ell
    n_ov = Pp.shape[0]
    # The fused tile kernels do 2*M*r*V flops on (M + r)*V*s bytes (M rows of U or
    # U and P, plus W2): 2*128*256/((128 + 256)*2) = 85 flop/B for the draft step,
    # below the MI355X ridge (~312 flop/B), so their roofline is HBM bandwidth;
    # their matrix-core use is reported beside it.
    work = {
        "bias_tile_draft": dict(bytes=R * V * s_el + r * V * s_el + R * r * s_el + R * nT * 8,
                                flops=2.0 * R * r * V, bound="hbm"),
        "draft_sample": dict(bytes=R * nT * 8 + R * 128 * (r + 1) * s_el, flops=0.0, bound="hbm"),
        "head_hidden_dot": dict(bytes=R * gamma * cfg.d * s_el, flops=2.0 * R * gamma * cfg.d,
                                bound="hbm"),
        "schedule": dict(bytes=R * gamma * 4 * 2, flops=0.0, bound="hbm"),
        "row_chunk_stats": dict(bytes=rows_used * V * s_el + rows_used * 32, flops=0.0, bound="hbm"),
        "bias_tile_verify": dict(bytes=2 * sum_ell * V * s_el + r * V * s_el + sum_ell * nT * 8,
                                 flops=2.0 * sum_ell * r * V, bound="hbm"),
        "verify_finalize": dict(bytes=sum_ell * nT * 8 + R * nT * 8, flops=0.0, bound="hbm"),
        "overlap_chunk": dict(bytes=2 * n_ov * V * s_el, flops=0.0, bound="hbm"),
        "overlap_combine": dict(bytes=n_ov * 20, flops=0.0, bound="hbm"),
    }
    kernels = {}
    for name, (ms, n) in list(kern.items()) + list(kern_ov.items()):
        w = work.get(name, dict(bytes=0, flops=0.0, bound="hbm"))
        avg_s = ms / n / 1e3
        kernels[name] = dict(launches_per_step=n // args.steps, avg_us=round(avg_s * 1e6, 3),
                             gbps=round(w["bytes"] / avg_s / 1e9, 1),
                             tflops=round(w["flops"] / avg_s / 1e12, 2),
                             bytes_per_launch=int(w["bytes"]), flops_per_launch=w["flops"],
                             bound=w["bound"])
    step_kernels = {k: v for k, v in kernels.items() if not k.startswith("overlap")}
    dom = max(step_kernels, key=lambda k: step_kernels[k]["avg_us"] * step_kernels[k]["launches_per_step"])
    dk = kernels[dom]
    if dk["bound"] == "mfma":
        roof = dict(bound="mfma", achieved=dk["tflops"], peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(dk["tflops"] / PEAK_BF16_TFLOPS, 4))
    else:
        roof = dict(bound="hbm", achieved=dk["gbps"], peak=PEAK_HBM_GBPS, unit="GB/s",
                    frac=round(dk["gbps"] / PEAK_HBM_GBPS, 4))
    roof["kernel"] = dom
    roof["mfma_frac"] = round(dk["tflops"] / PEAK_BF16_TFLOPS, 4)
    roof["traffic"] = None
    traffic_file = os.path.join(PROFILE_DIR, f"traffic_{dom}_{cfg.name.replace('-', '_')}.json")
    if os.path.exists(traffic_file):
        with open(traffic_file) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash():
            roof["traffic"] = tr.get("bytes_per_launch")

    # ---- the round's algorithmic HBM bytes (each input read once per call)
    round_bytes = (s_el * V * (R * gamma + sum_ell + rows_used) + 2 * s_el * r * V
                   + (R * gamma * cfg.d * s_el if cfg.d else 0))
    positions = R * gamma
    value = positions / (ms_step / 1e3)

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if args.cpu_requests > 0:
        import oracle
        nreq = min(args.cpu_requests, R)
        o_ell = ell  # the verified lengths of this workload (sets the sample's size only)
        t1 = time.perf_counter()
        for rho in range(nreq):
            hq = h[rho] if h is not None else None
            dr = oracle.draft_request(U[rho], W1, W2, int(x0[rho]), cfg.seed, cfg.round, rho,
                                      temp=cfg.temp, h_req=hq, w_conf=w_conf,
                                      b_conf=0.0 if b_conf is None else float(b_conf))
            oracle.verify_request(T[rho, : int(o_ell[rho]) + 1], U[rho], W1, W2, int(x0[rho]),
                                  dr["x"], int(o_ell[rho]), cfg.seed, cfg.round, rho, temp=cfg.temp)
        if c is not None:
            oracle.schedule(c, sps, cfg.mode, c_prev2=cp)
        cpu_s = time.perf_counter() - t1
        cpu = dict(value=round(nreq * gamma / cpu_s, 3), unit="positions/s", cores=1,
                   kind="oracle",
                   sample=f"{nreq} of {R} requests (draft of {gamma} positions + verify of the "
                          f"scheduled rows each) plus the full schedule; {cpu_s:.1f} s on 1 thread")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == synth.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: R={R} gamma={gamma} V={V} r={r}, "
                               f"scheduler mode {cfg.mode}, seeded synthetic logits",
                   "R": R, "gamma": gamma, "V": V, "r": r, "sum_ell": sum_ell,
                   "verify_rows": rows_used},
        "achieved_hbm_gbps": round(round_bytes / (ms_step / 1e3) / 1e9, 1),
        "round_bytes": int(round_bytes),
        "draft_positions_per_s": round(positions / (t_draft / 1e3), 1),
        "verify_rows_per_s": round(rows_used / (t_ver / 1e3), 1),
        "scheduler_off": {"ms_per_step": round(ms_off, 4),
                          "positions_per_s": round(positions / (ms_off / 1e3), 1),
                          "verify_rows": rows_off,
                          "achieved_hbm_gbps": round(
                              (s_el * V * (R * gamma + R * gamma + rows_off) + 2 * s_el * r * V
                               + (R * gamma * cfg.d * s_el if cfg.d else 0)) / (ms_off / 1e3) / 1e9, 1)},
        "breakdown_ms": {"draft": round(t_draft, 4), "schedule": round(t_sched, 4),
                         "verify": round(t_ver, 4)},
        "roofline": roof,
        "kernels": kernels,
        "next_rows": next_rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
