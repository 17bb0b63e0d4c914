"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Small configuration (config 1, fp32): every position, request and mode.
Full-size configurations (2-5, bf16): the launch shapes the benchmark times,
with the oracle on sampled positions and requests (it recomputes each row one
by one) plus invariants at every position.  Tokens, lengths, schedules and
theta are compared bit for bit, except draws whose uniform lies within 1e-6 of
an oracle CDF boundary (counted); probabilities and c* within 1e-5 (fp32) or
2e-3 (bf16).
"""
import numpy as np
import pytest
import torch

import draft_sampling_verification_03_amd as ds
import oracle
import synth
from gpu_common import (Inputs, check_draft_position, check_properties, check_schedule,
                        check_verify_request, dev, prob_tol, run_round)

pytestmark = pytest.mark.gpu

_cache = {}


def inputs(cid_or_cfg):
    key = cid_or_cfg if isinstance(cid_or_cfg, int) else repr(cid_or_cfg)
    if key not in _cache:
        cfg = synth.CONFIGS[cid_or_cfg] if isinstance(cid_or_cfg, int) else cid_or_cfg
        _cache.clear()  # keep one configuration resident at a time
        torch.cuda.empty_cache()
        _cache[key] = Inputs(cfg)
    return _cache[key]


def new_stats():
    return dict(draws=0, draw_exempt=0, accept_exempt=0, requests=0)


def full_check(inp, g, stats):
    cfg = inp.cfg
    check_properties(inp, g)
    for rho in range(cfg.R):
        for k in range(1, cfg.gamma + 1):
            check_draft_position(inp, g, rho, k, stats)
    check_schedule(inp, g)
    for rho in range(cfg.R):
        check_verify_request(inp, g, rho, stats)


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_tiny_config_every_position_and_mode(mode):
    inp = inputs(1)
    stats = new_stats()
    g = run_round(inp, mode=mode)
    full_check(inp, g, stats)
    print(f"config 1 mode {mode}: {stats}", flush=True)


@pytest.mark.parametrize("rnd", [1, 2, 3])
def test_tiny_config_other_rounds(rnd):
    inp = inputs(1)
    stats = new_stats()
    g = run_round(inp, rnd=rnd)
    full_check(inp, g, stats)


@pytest.mark.parametrize("over", [
    dict(V=1000, R=3, gamma=1),                     # ragged last tile, gamma = 1
    dict(V=8, R=2, gamma=3, r=16),                  # a vocabulary smaller than one tile
    dict(R=1, gamma=6, V=2056),                     # one request
    dict(R=33, gamma=2, V=1032),                    # 64-row tiles
    dict(R=100, gamma=2, V=776),                    # 128-row tiles with padding rows
    dict(R=5, gamma=3, V=1024, temp=0.7),           # temperature
    dict(R=6, gamma=4, V=2048, dtype=synth.BF16, r=32, target_sd=3.0, weight_sd=0.05),
    dict(R=4, gamma=5, V=1024, dtype=synth.BF16, r=256, weight_sd=0.05),
    dict(R=4, gamma=4, V=1024, r=128),              # fp32 rank limit
    dict(R=5, gamma=64, V=1024),                    # the longest block
    dict(R=128, gamma=64, V=264),                   # the largest candidate count, 8192
    # the single-launch draft (bf16, r = 256): a masked last tile, fewer
    # workgroups than requests (each draws several), one request, a partly
    # filled last row block, and five tiles per workgroup with a masked one
    dict(R=3, gamma=4, V=1000, dtype=synth.BF16, r=256, weight_sd=0.05),
    dict(R=10, gamma=3, V=384, dtype=synth.BF16, r=256, weight_sd=0.05),
    dict(R=1, gamma=5, V=2056, dtype=synth.BF16, r=256, weight_sd=0.05),
    dict(R=97, gamma=2, V=4000, dtype=synth.BF16, r=256, weight_sd=0.05),
    dict(R=4, gamma=2, V=131848, dtype=synth.BF16, r=256, weight_sd=0.02),
    dict(R=2, gamma=1, V=1024, dtype=synth.BF16, r=256, weight_sd=0.05),
    dict(R=7, gamma=3, V=2048, dtype=synth.BF16, r=256, weight_sd=0.05, temp=0.6),
    # bf16, r = 256 past five tiles per compute unit (1281 tiles): the
    # streaming draft and the streaming verify product
    dict(R=2, gamma=2, V=163968, dtype=synth.BF16, r=256, weight_sd=0.02),
    # bf16, r = 256 past 512 requests: the per-step kernels (8-wave row
    # groups), and the W2-stationary verify over 1040 possible rows
    dict(R=520, gamma=2, V=2048, dtype=synth.BF16, r=256, weight_sd=0.05),
])
def test_edge_shapes(over):
    cfg = synth.make_config(1, cid=50 + len(_cache), **over)
    inp = inputs(cfg)
    stats = new_stats()
    for mode in (1, 2):
        g = run_round(inp, mode=mode)
        full_check(inp, g, stats)
    print(f"edge {over}: {stats}", flush=True)


def test_zero_and_full_lengths():
    """ell = 0 everywhere (bonus from p_1) and ell = gamma everywhere."""
    cfg = synth.make_config(1, cid=70, R=6, gamma=3, V=1024)
    inp = inputs(cfg)
    stats = new_stats()
    sps_zero = np.ones(cfg.B_max + 1)
    sps_zero[cfg.R + 1:] = 1e-3          # admitting anything costs more than it gains
    inp.sps, inp.dsps = sps_zero, dev(sps_zero)
    g = run_round(inp, mode=2)
    assert (g["ell"] == 0).all()
    full_check(inp, g, stats)
    g = run_round(inp, mode=0)
    assert (g["ell"] == cfg.gamma).all()
    full_check(inp, g, stats)


SAMPLED = {2: [0, 1, 17, 31], 3: [0, 5, 64, 127], 4: [0, 3, 128, 255], 5: [0, 7, 300, 511]}


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_size_config(cid):
    inp = inputs(cid)
    cfg = inp.cfg
    stats = new_stats()
    print(f"[run] config {cid}", flush=True)
    g = run_round(inp)
    check_properties(inp, g)
    check_schedule(inp, g)
    rng = np.random.default_rng(cid)
    reqs = list(SAMPLED[cid])
    # requests at the extremes of the schedule, when present
    for L in (0, cfg.gamma):
        hit = np.flatnonzero(g["ell"] == L)
        if hit.size:
            reqs.append(int(hit[0]))
    for rho in reqs[:6]:
        for k in range(1, cfg.gamma + 1):
            check_draft_position(inp, g, rho, k, stats)
    for rho, k in zip(rng.integers(0, cfg.R, 8), rng.integers(1, cfg.gamma + 1, 8)):
        check_draft_position(inp, g, int(rho), int(k), stats)
    for rho in reqs:
        check_verify_request(inp, g, rho, stats)
    print(f"config {cid}: sum ell={int(g['ell'].sum())} n*={g['n_admitted']} {stats}", flush=True)


@pytest.mark.parametrize("over,reqs", [
    # one masked tile per workgroup (157 tiles), every request checked
    (dict(R=40, gamma=7, V=20000), None),
    # five tiles per workgroup with a masked one, sampled requests
    (dict(R=33, gamma=8, V=131848), (0, 16, 32)),
    # a temperature other than 1 (both the draft's and the verify's z / T)
    (dict(R=36, gamma=8, V=20000, temp=0.7), None),
])
def test_stationary_verify_shapes(over, reqs):
    """The W2-stationary verify product (bf16, r = 256, R gamma > 256) with
    every position admitted: 9 row blocks of 32, the last one partly filled,
    and masked vocabulary tails; draws, c* and the final tokens against the
    oracle."""
    cfg = synth.make_config(1, cid=80 + over["R"], dtype=synth.BF16, r=256, weight_sd=0.05, **over)
    inp = inputs(cfg)
    stats = new_stats()
    g = run_round(inp, mode=0)
    assert (g["ell"] == cfg.gamma).all()
    check_properties(inp, g)
    check_schedule(inp, g)
    reqs = range(cfg.R) if reqs is None else reqs
    for rho in reqs:
        for k in range(1, cfg.gamma + 1):
            check_draft_position(inp, g, rho, k, stats)
        check_verify_request(inp, g, rho, stats)
    print(f"stationary verify {over}: {stats}", flush=True)


@pytest.mark.parametrize("over", [
    # two chunks, the last partly filled (72 rows); 157 workgroups, a masked tile
    dict(R=200, gamma=3, V=20000),
    # two chunks, the last of one request; 129 workgroups of one tile each
    dict(R=129, gamma=2, V=16512),
    # past 128 requests with fewer than 128 tiles: the per-step kernels
    dict(R=150, gamma=2, V=4096),
])
def test_chunked_persistent_draft(over):
    """The single-launch draft past 128 requests (bf16, r = 256): requests in
    chunks of 128, each chunk's draws after the next chunk's products; every
    draw, q(x), normalizer and the verification against the oracle."""
    cfg = synth.make_config(1, cid=90 + over["R"], dtype=synth.BF16, r=256, weight_sd=0.05, **over)
    inp = inputs(cfg)
    stats = new_stats()
    g = run_round(inp, mode=2)
    full_check(inp, g, stats)
    print(f"chunked draft {over}: sum ell={int(g['ell'].sum())} {stats}", flush=True)


def test_persistent_draft_peaky_logits_ragged_rows():
    """The single-launch draft (bf16, r = 256, R <= 128) on the stress
    workload's peaky logits (target sd 8, draft noise sd up to 4) with a
    partly filled last row block (R = 100): every q(x) stays in (0, 1], and
    the draws, q(x) and normalizers of sampled requests match the oracle."""
    cfg = synth.Config(cid=16, name="peaky-r100", R=100, gamma=6, V=151936, r=256,
                       dtype=synth.BF16, target_sd=8.0, noise="uniform:0.1:4", weight_sd=0.02,
                       conf="sigmoid:2:1.5", sps="smooth", mode=synth.SCHED_EARLY_STOP)
    inp = inputs(cfg)
    stats = new_stats()
    g = run_round(inp)
    check_properties(inp, g)
    check_schedule(inp, g)
    for rho in (0, 31, 32, 63, 96, 99):
        for k in range(1, cfg.gamma + 1):
            check_draft_position(inp, g, rho, k, stats)
    for rho in (0, 57, 99):
        check_verify_request(inp, g, rho, stats)
    print(f"peaky R=100: {stats}", flush=True)


@pytest.mark.parametrize("cid", [1, 3])
def test_tv_overlap_against_oracle(cid):
    inp = inputs(cid)
    cfg = inp.cfg
    n = min(64, cfg.R * cfg.gamma)
    rows = [(i % cfg.R, i % cfg.gamma) for i in range(n)]
    P = np.stack([inp.T[r, k] for r, k in rows])
    Q = np.stack([inp.U[r, k] for r, k in rows])
    dP, dQ = dev(P), dev(Q)
    c1 = ds.tv_overlap(dP, dQ).cpu().numpy()
    # statistics supplied (computed with torch in fp64 as plain inputs)
    def stats(t):
        z = t.double()
        m = z.max(dim=1).values
        return torch.stack([m, torch.exp(z - m[:, None]).sum(dim=1)], dim=1).float().contiguous()
    c2 = ds.tv_overlap(dP, dQ, p_stats=stats(dP), q_stats=stats(dQ)).cpu().numpy()
    tol = prob_tol(cfg)
    for i in range(n):
        o = oracle.overlap(P[i], Q[i])
        assert abs(c1[i] - o) <= tol and abs(c2[i] - o) <= tol


def test_tv_overlap_full_launch_sampled_rows():
    """The standalone overlap in the launch the benchmark times: all 2048
    (target row, draft row) pairs of the R = 128, gamma = 16, V = 151936
    workload in one call, statistics supplied and computed on the device;
    sampled rows (first, last, chunk-straddling middle ones) against the
    oracle, and every value in [0, 1]."""
    inp = inputs(3)
    cfg = inp.cfg
    R, gamma, V = cfg.R, cfg.gamma, cfg.V
    n = R * gamma
    P = inp.T.reshape(R * (gamma + 1), V)[:n]
    Q = inp.U.reshape(n, V)
    dP, dQ = inp.dT[:n], inp.dU.reshape(n, V)  # the same bytes, already on the device

    def stats(t):
        z = t.float()
        m = z.max(dim=1).values
        return torch.stack([m, torch.exp(z - m[:, None]).sum(dim=1)], dim=1).contiguous()

    c = ds.tv_overlap(dP, dQ, p_stats=stats(dP), q_stats=stats(dQ)).cpu().numpy()
    assert c.shape == (n,) and np.isfinite(c).all()
    assert ((c >= -1e-6) & (c <= 1 + 1e-5)).all()
    tol = prob_tol(cfg)
    for i in (0, 1, 255, 256, 1023, 1024, 1537, n - 1):
        assert abs(c[i] - oracle.overlap(P[i], Q[i])) <= tol, i


@pytest.mark.parametrize("V,bf16", [
    (8, False),      # one tile narrower than itself: three of the four row chunks empty
    (264, True),     # three tiles: the last chunk empty, its start past V
    (1144, True),    # nine tiles, V not a multiple of 128: an empty last chunk
    (1144, False),
    (20000, True),   # chunks of 40 tiles, a masked last tile
])
def test_tv_overlap_small_vocabularies(V, bf16):
    """dspark_tv_overlap where some row chunks hold no tile (their loads are
    clamped to the row's last piece and their sums are empty) against the
    oracle, with the statistics computed on the device and supplied."""
    rng = np.random.default_rng(V + 7 * bf16)
    n = 6
    P = rng.normal(0.0, 3.0, (n, V)).astype(np.float32)
    Q = (P + rng.normal(0.0, 1.5, (n, V))).astype(np.float32)
    P[1] = Q[1]                      # p = q: overlap 1
    if bf16:
        P, Q = synth.to_bf16_bits(P), synth.to_bf16_bits(Q)
    dP, dQ = dev(P), dev(Q)
    tol = 2e-3 if bf16 else 1e-5

    def stats(t):
        z = t.double()
        m = z.max(dim=1).values
        return torch.stack([m, torch.exp(z - m[:, None]).sum(dim=1)], dim=1).float().contiguous()

    for c in (ds.tv_overlap(dP, dQ).cpu().numpy(),
              ds.tv_overlap(dP, dQ, p_stats=stats(dP), q_stats=stats(dQ)).cpu().numpy()):
        for i in range(n):
            assert abs(c[i] - oracle.overlap(P[i], Q[i])) <= tol, (V, bf16, i)


def test_determinism_bitwise():
    inp = inputs(3)
    outs = [run_round(inp) for _ in range(3)]
    for key in ("x", "q_stats", "q_x", "ell", "row_offset", "a", "n_acc", "y", "c_star"):
        for o in outs[1:]:
            assert np.array_equal(outs[0][key], o[key], equal_nan=True), key
    assert outs[0]["theta"] == outs[1]["theta"] == outs[2]["theta"]


def test_device_error_word_flags_bad_tokens_and_confidences():
    inp = inputs(1)
    cfg = inp.cfg
    bad_x0 = inp.dx0.clone()
    bad_x0[1] = cfg.V + 5
    ws = ds.Workspace()
    ds.draft(inp.dU, inp.dW1, inp.dW2, bad_x0, ws=ws)
    assert ws.error_code() & 1
    ws.clear_error()
    assert ws.error_code() == 0
    c = dev(inp.c)
    c[0, 1] = 1.5
    wss = ds.Workspace()
    ds.schedule(c, inp.dsps, 1, ws=wss)
    assert wss.error_code() & 2


def test_verify_output_law_chi2_on_gpu():
    """Many requests with identical inputs are independent rounds (the Philox
    counter carries the request index): the first output token has the target
    law p1 and, after an accepted first draft, the second has p2."""
    from scipy import special, stats as st
    R, gamma, V, r = 4096, 2, 8, 16
    rng = np.random.default_rng(12)
    W1 = (0.8 * rng.standard_normal((V, r))).astype(np.float32)
    W2 = (0.8 * rng.standard_normal((V, r))).astype(np.float32)
    U1 = (1.2 * rng.standard_normal((gamma, V))).astype(np.float32)
    T1 = (1.2 * rng.standard_normal((gamma + 1, V))).astype(np.float32)
    U = np.broadcast_to(U1, (R, gamma, V)).copy()
    x0 = np.full(R, 3, dtype=np.int32)
    d = ds.draft(dev(U), dev(W1), dev(W2), dev(x0), seed=5, round=9)
    s = ds.schedule(None, None, 0, R=R, gamma=gamma)
    P = np.broadcast_to(T1, (R, gamma + 1, V)).reshape(R * (gamma + 1), V).copy()
    v = ds.verify(s["ell"], s["row_offset"], dev(P), dev(U), dev(W1), dev(W2), dev(x0), d["x"],
                  d["q_stats"], d["q_x"], seed=5, round=9)
    y = v["y"].cpu().numpy()
    n = v["n_acc"].cpu().numpy()
    p1 = special.softmax(T1[0].astype(np.float64))
    assert st.chisquare(np.bincount(y[:, 0], minlength=V), p1 * R).pvalue > 1e-3
    p2 = special.softmax(T1[1].astype(np.float64))
    sel = y[n >= 1, 1]
    assert st.chisquare(np.bincount(sel, minlength=V), p2 * sel.size).pvalue > 1e-3
    # position-1 acceptance frequency against c*_1 (binomial 99.9 % interval)
    c1 = float(v["c_star"].cpu().numpy()[0, 0])
    acc = float(np.mean(n >= 1))
    assert abs(acc - c1) < 3.29 * np.sqrt(c1 * (1 - c1) / R)


# ----------------------------------------------- next rows: STS and thresholds
@pytest.mark.gpu
@pytest.mark.parametrize("dtype,r", [(np.float32, 16), ("bf16", 16), ("bf16", 256)])
def test_confidence_head_position_temperatures(dtype, r):
    """c_k = sigmoid(z_k / T_k) against the oracle's head at the GPU's tokens;
    a temperature that is not a finite positive number is flagged and taken as 1.
    (bf16 with r = 256 runs the single-launch draft.)"""
    rng = np.random.default_rng(21)
    R, gamma, V, d = 16, 5, 512, 64
    store = (lambda a: synth.to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    U = store(rng.standard_normal((R, gamma, V)).astype(np.float32))
    W1 = store((0.3 * rng.standard_normal((V, r)) * np.sqrt(16 / r)).astype(np.float32))
    W2 = store((0.3 * rng.standard_normal((V, r)) * np.sqrt(16 / r)).astype(np.float32))
    h = store(rng.standard_normal((R, gamma, d)).astype(np.float32))
    w = (0.2 * rng.standard_normal(d + r)).astype(np.float32)
    x0 = rng.integers(0, V, R).astype(np.int32)
    T = np.array([0.6, 1.0, 1.7, 3.0, 0.9], dtype=np.float32)
    ws = ds.Workspace()
    g = ds.draft(dev(U), dev(W1), dev(W2), dev(x0), h=dev(h), w_conf=dev(w), b_conf=0.25,
                 conf_temp=dev(T), seed=3, round=1, ws=ws)
    x, c = g["x"].cpu().numpy(), g["c"].cpu().numpy()
    assert ws.error_code() == 0
    tol = 1e-5 if dtype == np.float32 else 2e-3
    for rho in range(R):
        for k in range(gamma):
            prev = int(x0[rho]) if k == 0 else int(x[rho, k - 1])
            o = oracle.conf_head(h[rho, k], w, np.float32(0.25), W1, prev, T=float(T[k]))
            assert abs(c[rho, k] - o) <= tol
    bad = T.copy()
    bad[2] = 0.0
    ws2 = ds.Workspace()
    g2 = ds.draft(dev(U), dev(W1), dev(W2), dev(x0), h=dev(h), w_conf=dev(w), b_conf=0.25,
                  conf_temp=dev(bad), seed=3, round=1, ws=ws2)
    assert ws2.error_code() & 2
    c2 = g2["c"].cpu().numpy()
    for rho in range(R):
        o = oracle.conf_head(h[rho, 2], w, np.float32(0.25), W1, int(x[rho, 1]), T=1.0)
        assert abs(c2[rho, 2] - o) <= tol


@pytest.mark.gpu
@pytest.mark.parametrize("R,gamma", [(4, 4), (128, 16), (512, 15), (1024, 8)])
def test_threshold_schedule_matches_oracle(R, gamma):
    rng = np.random.default_rng(R + gamma)
    c = (1.0 / (1.0 + np.exp(-(2.0 + 1.5 * rng.standard_normal((R, gamma)))))).astype(np.float32)
    sps = 60.0 * 1024.0 / (1024.0 + np.arange(R * (gamma + 1) + 1, dtype=np.float64))
    for thr in np.float32([0.0, 0.6, 0.85, 0.97, 1.5]):
        for table in (sps, None):
            o = oracle.schedule(c, table, oracle.SCHED_THRESHOLD, threshold=thr)
            ws = ds.Workspace()
            g = ds.schedule(dev(c), dev(table) if table is not None else None,
                            ds.DSPARK_SCHED_THRESHOLD, threshold=float(thr), ws=ws)
            assert ws.error_code() == 0
            assert np.array_equal(g["ell"].cpu().numpy(), o["ell"])
            assert np.array_equal(g["row_offset"].cpu().numpy(), o["row_offset"])
            assert int(g["n_admitted"].cpu().numpy()[0]) == o["n_admitted"]
            assert np.array_equal(g["a"].cpu().numpy(), o["a"])
            th = float(g["theta"].cpu().numpy()[0])
            assert (np.isnan(th) and np.isnan(o["theta"])) or th == o["theta"]


def _schedule_against_oracle(c, sps, mode, c_prev2=None, threshold=0.0):
    o = oracle.schedule(c, sps, mode, c_prev2=c_prev2, threshold=threshold)
    ws = ds.Workspace()
    g = ds.schedule(dev(c), dev(sps), mode, c_prev2=dev(c_prev2) if c_prev2 is not None else None,
                    threshold=float(threshold), ws=ws)
    assert ws.error_code() == 0
    assert np.array_equal(g["ell"].cpu().numpy(), o["ell"])
    assert np.array_equal(g["row_offset"].cpu().numpy(), o["row_offset"])
    assert int(g["n_admitted"].cpu().numpy()[0]) == o["n_admitted"]
    assert np.array_equal(g["a"].cpu().numpy().view(np.uint32), o["a"].view(np.uint32))
    th = float(g["theta"].cpu().numpy()[0])
    assert (np.isnan(th) and np.isnan(o["theta"])) or th == o["theta"]
    return o


@pytest.mark.parametrize("case", ["plateau", "rise_after_plateau", "equal_maxima"])
def test_schedule_tie_rules_match_oracle(case):
    """Exact theta ties: early stop halts at the first non-increase, the full
    search takes the smallest maximiser (the oracle's pinned readings)."""
    if case == "plateau":
        c = np.array([[1.0, 1.0], [0.0, 0.0]], dtype=np.float32)
        sps, expect = np.ones(7), {1: 2, 2: 2}
    elif case == "rise_after_plateau":
        c = np.ones((1, 3), dtype=np.float32)
        sps, expect = np.array([0.0, 4.0, 3.0, 2.0, 2.0]), {1: 1, 2: 3}
    else:
        c = np.ones((1, 3), dtype=np.float32)
        sps, expect = np.array([0.0, 1.0, 1.0, 0.5, 0.5]), {1: 1, 2: 1}
    for mode, n in expect.items():
        assert _schedule_against_oracle(c, sps, mode)["n_admitted"] == n
    _schedule_against_oracle(c, sps, 3, c_prev2=c)


@pytest.mark.parametrize("R,gamma", [(128, 16), (512, 15)])
def test_schedule_zero_and_negative_zero_confidences(R, gamma):
    """Many zero-weight candidates (theta plateaus under a stepped SPS) and
    -0.0 confidences, which rank exactly like +0.0: bit-exact against the oracle."""
    rng = np.random.default_rng(R)
    c = (1.0 / (1.0 + np.exp(-(2.0 + 1.5 * rng.standard_normal((R, gamma)))))).astype(np.float32)
    zero = rng.random((R, gamma)) < 0.3
    c[zero] = np.where(rng.random(int(zero.sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
    B = np.arange(R * (gamma + 1) + 1, dtype=np.float64)
    for sps in (60.0 * 1024.0 / (1024.0 + 64.0 * np.ceil(B / 64.0)), np.full(B.size, 3.0)):
        for mode in (1, 2):
            _schedule_against_oracle(c, sps, mode)
        _schedule_against_oracle(c, sps, 3, c_prev2=c[::-1].copy())
        _schedule_against_oracle(c, sps, ds.DSPARK_SCHED_THRESHOLD, threshold=0.0)
