"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None of them compares the oracle with
itself: each checks a value printed on the pages (tests/golden/*.json, with
their citations), a closed form, an invariant, a library routine that the
special case reduces to (numpy's Philox, scipy's softmax and logsumexp, numpy
matmul / searchsorted / lexsort), brute force, exact enumeration, or a
Monte Carlo statistic with a stated interval.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ Philox RNG
@pytest.mark.parametrize("ctr,key", [
    ([1, 0, 0, 0], [0, 0]),
    ([3, 3, 4, 9], [5, 7]),
    ([17, 2, 1, 0], [0, 0]),
    ([2**63, 2**64 - 1, 12345, 2**40 + 3], [0xDEADBEEFCAFEF00D, 0x0123456789ABCDEF]),
])
def test_philox_matches_numpy_library(ctr, key):
    """numpy.random.Philox is a Philox4x64-10 implementation; its state counter
    is incremented before each block, so the block after state c is philox(c+1)."""
    prev = list(ctr)
    prev[0] -= 1  # ctr[0] >= 1 in every case, no borrow
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array(prev, dtype=np.uint64))
    expect = bg.random_raw(4)
    got = oracle.philox4x64_10(ctr, key)
    assert [int(v) for v in got] == [int(v) for v in expect]


def test_uniform_is_top_24_bits_and_uniform():
    us = np.array([oracle.uniform(0, 0, pos, req, s) for pos in range(1, 40) for req in range(40)
                   for s in range(3)])
    assert np.all(us >= 0) and np.all(us < 1)
    assert np.all(us * 2**24 == np.floor(us * 2**24))  # 24-bit dyadic
    # same number from the library generator: top 24 bits of the first word
    bg = np.random.Philox(key=np.array([9, 0], dtype=np.uint64),
                          counter=np.array([4, 5, 1, 7], dtype=np.uint64))
    w0 = int(bg.random_raw(4)[0])
    assert oracle.uniform(9, 7, 5, 5, 1) == (w0 >> 40) / 2**24
    # distribution: Kolmogorov-Smirnov against U[0,1)
    assert stats.kstest(us, "uniform").pvalue > 1e-3


# ------------------------------------------------------------------ widening
def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F, 0x0001], dtype=np.uint16)
    expect = [1.0, -1.0, 3.140625, 0.0, 3.3895313892515355e38, 9.183549615799121e-41]
    assert list(oracle.widen(bits)) == expect


# ------------------------------------------------------------------ softmax stats
def test_row_stats_closed_forms_and_logsumexp():
    V = 1000
    const = np.full(V, 1.25, dtype=np.float32)
    m, S = oracle.row_stats(const)
    assert m == 1.25 and S == pytest.approx(V, rel=1e-15)
    two = np.array([0.0, math.log(3.0)], dtype=np.float32)  # p = (1/4, 3/4)
    m, S = oracle.row_stats(two)
    assert m == np.float64(np.float32(math.log(3.0)))
    assert 1.0 / S == pytest.approx(0.75, rel=1e-7)
    rng = np.random.default_rng(1)
    x = (3 * rng.standard_normal(5000)).astype(np.float32)
    for temp in (1.0, 0.7, 2.0):
        m, S = oracle.row_stats(x, temp)
        z = x.astype(np.float64) / temp
        assert m == z.max() and S >= 1.0
        assert m + math.log(S) == pytest.approx(special.logsumexp(z), rel=1e-13)


# ------------------------------------------------------------------ inverse CDF
def test_inverse_cdf_brute_force_grid():
    w = np.array([0.0, 0.3, 0.0, 1.2, 0.5, 0.0, 2.0, 0.0])
    M = 100_000
    picks = np.array([oracle.inverse_cdf(w, (i + 0.5) / M) for i in range(0, M, 7)])
    assert np.all(w[picks] > 0), "a zero-mass token was drawn"
    frac = np.bincount(picks, minlength=w.size) / picks.size
    assert np.allclose(frac, w / w.sum(), atol=3e-4)
    # the definition reduces to a right-sided search in the cumulative sum
    for u in np.random.default_rng(2).random(500):
        assert oracle.inverse_cdf(w, u) == np.searchsorted(np.cumsum(w), u * w.sum(),
                                                           side="right")


# ------------------------------------------------------------------ Markov head
def _small_head(V=32, r=8, seed=3, w_scale=0.5):
    rng = np.random.default_rng(seed)
    W1 = (w_scale * rng.standard_normal((V, r))).astype(np.float32)
    W2 = (w_scale * rng.standard_normal((V, r))).astype(np.float32)  # column-major r x V
    U = (2 * rng.standard_normal(V)).astype(np.float32)
    return U, W1, W2


@pytest.mark.parametrize("temp", [1.0, 0.8])
def test_draft_law_is_softmax_of_bias_gemm(temp):
    U, W1, W2 = _small_head()
    prev = 5
    out = oracle.draft_position(U, W1, W2, prev, 0.5, temp=temp, want_law=True)
    bias = W2.astype(np.float64) @ W1[prev].astype(np.float64)  # B(prev, v) = W1[prev,:] W2[:, v]
    q = special.softmax((U.astype(np.float64) + bias) / temp)
    assert np.allclose(out["q"], q, rtol=1e-12, atol=1e-15)
    z = (U.astype(np.float64) + bias) / temp
    assert out["m"] == pytest.approx(z.max(), rel=1e-14)
    assert out["qx"] == pytest.approx(q[out["x"]], rel=1e-12)


def test_draft_with_zero_transition_is_independent_softmax():
    U, W1, W2 = _small_head()
    W1[:] = 0
    for prev in (0, 7, 31):
        out = oracle.draft_position(U, W1, W2, prev, 0.25, want_law=True)
        assert np.allclose(out["q"], special.softmax(U.astype(np.float64)), rtol=1e-13)


def test_draft_draws_follow_markov_conditional_chi2():
    V, r = 8, 4
    U, W1, W2 = _small_head(V=V, r=r, seed=4, w_scale=0.8)
    prev = 3
    law = oracle.draft_position(U, W1, W2, prev, 0.0, want_law=True)["q"]
    n = 20000
    xs = [oracle.draft_position(U, W1, W2, prev, oracle.uniform(11, t, 1, 0, 0))["x"]
          for t in range(n)]
    counts = np.bincount(xs, minlength=V)
    assert stats.chisquare(counts, law * n).pvalue > 1e-3


def test_confidence_head_is_sigmoid_of_linear_layer():
    rng = np.random.default_rng(5)
    V, r, d = 16, 8, 24
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    h = rng.standard_normal(d).astype(np.float32)
    w = (0.3 * rng.standard_normal(d + r)).astype(np.float32)
    b = np.float32(0.7)
    prev = 9
    feat = np.concatenate([h, W1[prev]]).astype(np.float64)
    expect = special.expit(feat @ w.astype(np.float64) + float(b))
    assert oracle.conf_head(h, w, b, W1, prev) == pytest.approx(expect, rel=1e-13)


# ------------------------------------------------------------------ c* / TV
def test_overlap_printed_example():
    g = golden("overlap_example.json")
    P = np.log(np.array(g["p_target"])).astype(np.float32)
    Q = np.log(np.array(g["p_draft"])).astype(np.float32)
    assert oracle.overlap(P, Q) == pytest.approx(g["overlap"], abs=1e-6)


def test_overlap_identities():
    rng = np.random.default_rng(6)
    V = 4096
    for _ in range(5):
        P = (3 * rng.standard_normal(V)).astype(np.float32)
        Q = (P + rng.standard_normal(V)).astype(np.float32)
        c, tv = oracle.overlap(P, Q, with_tv=True)
        assert c == pytest.approx(1.0 - tv, abs=1e-12)  # sum min = 1 - TV
        assert 0.0 < c < 1.0
    assert oracle.overlap(P, P) == pytest.approx(1.0, abs=1e-12)
    a = np.array([0.0, -1e4], dtype=np.float32)
    b = np.array([-1e4, 0.0], dtype=np.float32)
    assert oracle.overlap(a, b) == pytest.approx(0.0, abs=1e-300)  # disjoint supports


# ------------------------------------------------------------------ verification
def _verify_setup_one_token(q, p):
    V = len(q)
    U = np.log(np.array([q], dtype=np.float64)).astype(np.float32)      # [gamma=1][V]
    P = np.log(np.array([p, p], dtype=np.float64)).astype(np.float32)   # rows 1 and 2 (bonus)
    W1 = np.zeros((V, 2), dtype=np.float32)
    W2 = np.zeros((V, 2), dtype=np.float32)
    return U, P, W1, W2


def test_verify_printed_example():
    g = golden("spec_sampling_example.json")
    q, p = np.array(g["q_draft"]), np.array(g["p_target"])
    U, P, W1, W2 = _verify_setup_one_token(q, p)
    acc_prob, law = [], np.zeros(3)
    for x in range(3):
        res = oracle.verify_request(P, U, W1, W2, 0, [x], 1, 0, 0, 0, want_cdf=True)
        a = min(1.0, res["ratio"][0])
        acc_prob.append(a)
        resid = oracle.verify_request(P, U, W1, W2, 0, [x], 1, 0, 0, 0, force_n=0, want_cdf=True)
        r_law = np.diff(np.concatenate([[0.0], resid["final_cdf"]]))
        assert np.allclose(r_law, g["residual_normalized"], atol=1e-6)
        assert res["c_star"][0] == pytest.approx(g["alpha"], abs=1e-6)
        law += q[x] * (a * np.eye(3)[x] + (1 - a) * r_law)
    assert np.allclose(acc_prob, g["acceptance_probability"], atol=1e-6)
    assert np.allclose(q * np.array(acc_prob), g["accepted_mass"], atol=1e-6)
    assert np.allclose(law, g["final_law"], atol=1e-6)


def test_verify_exact_enumeration_gamma2():
    """Sum over every drafted pair the acceptance, residual and bonus branches
    of the oracle's verification: the first output token has the target law p1,
    and the second, given the first draft was accepted, has p2(. | x1)."""
    V, r = 4, 2
    rng = np.random.default_rng(7)
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    W2 = rng.standard_normal((V, r)).astype(np.float32)
    U = (1.5 * rng.standard_normal((2, V))).astype(np.float32)
    T1 = (1.5 * rng.standard_normal(V)).astype(np.float32)
    T2 = (1.5 * rng.standard_normal((V, V))).astype(np.float32)      # target at 2 given x1
    T3 = (1.5 * rng.standard_normal((V, V, V))).astype(np.float32)   # target at 3 given x1, x2
    x0 = 2

    def q_law(k, prev):
        return special.softmax(U[k - 1].astype(np.float64) + W2.astype(np.float64) @ W1[prev])

    def law_of(res):
        return np.diff(np.concatenate([[0.0], res["final_cdf"]]))

    law_y1 = np.zeros(V)
    law_y2 = np.zeros((V, V))
    mass_acc1 = np.zeros(V)
    q1 = q_law(1, x0)
    for x1 in range(V):
        q2 = q_law(2, x1)
        for x2 in range(V):
            wgt = q1[x1] * q2[x2]
            P = np.stack([T1, T2[x1], T3[x1, x2]])
            args = (P, U, W1, W2, x0, [x1, x2], 2, 0, 0, 0)
            base = oracle.verify_request(*args)
            a1, a2 = min(1.0, base["ratio"][0]), min(1.0, base["ratio"][1])
            r1 = law_of(oracle.verify_request(*args, force_n=0, want_cdf=True))
            r2 = law_of(oracle.verify_request(*args, force_n=1, want_cdf=True))
            law_y1 += wgt * ((1 - a1) * r1 + a1 * np.eye(V)[x1])
            law_y2[x1] += wgt * a1 * ((1 - a2) * r2 + a2 * np.eye(V)[x2])
            mass_acc1[x1] += wgt * a1
    assert np.allclose(law_y1, special.softmax(T1.astype(np.float64)), atol=1e-12)
    for x1 in range(V):
        assert np.allclose(law_y2[x1] / mass_acc1[x1], special.softmax(T2[x1].astype(np.float64)),
                           atol=1e-12)


def _mc_pipeline(n_trials, V=8, r=4, gamma=3, seed=8, zero_transition=False, markov_target=True):
    rng = np.random.default_rng(seed)
    W1 = (0.8 * rng.standard_normal((V, r))).astype(np.float32)
    if zero_transition:
        W1[:] = 0
    W2 = (0.8 * rng.standard_normal((V, r))).astype(np.float32)
    U = (1.2 * rng.standard_normal((gamma, V))).astype(np.float32)
    Tt = (1.2 * rng.standard_normal((gamma + 1, V, V))).astype(np.float32)  # target k given x_{k-1}
    x0 = 1
    out = []
    for t in range(n_trials):
        d = oracle.draft_request(U, W1, W2, x0, 21, t, 0)
        x = d["x"]
        prevs = [x0] + list(x)
        P = np.stack([Tt[k][prevs[k] if markov_target else x0] for k in range(gamma + 1)])
        v = oracle.verify_request(P, U, W1, W2, x0, x, gamma, 21, t, 0)
        out.append((x, v))
    return out, Tt, x0


def test_verify_output_law_chi2_and_first_acceptance_rate():
    n = 20000
    runs, Tt, x0 = _mc_pipeline(n)
    p1 = special.softmax(Tt[0][x0].astype(np.float64))
    y1 = np.array([v["y"][0] for _, v in runs])
    counts = np.bincount(y1, minlength=p1.size)
    assert stats.chisquare(counts, p1 * n).pvalue > 1e-3
    # second token given the first draft accepted: p2(. | x1)
    pv = []
    for x1 in range(p1.size):
        sel = [v["y"][1] for x, v in runs if v["n_acc"] >= 1 and x[0] == x1]
        if len(sel) < 300:
            continue
        p2 = special.softmax(Tt[1][x1].astype(np.float64))
        pv.append(stats.chisquare(np.bincount(sel, minlength=p2.size), p2 * len(sel)).pvalue)
    assert len(pv) >= 2 and min(pv) > 1e-3 / len(pv)
    # position-1 acceptance frequency equals c*_1 (binomial 99.9 % interval)
    c1 = runs[0][1]["c_star"][0]
    acc = np.mean([v["n_acc"] >= 1 for _, v in runs])
    half = 3.29 * math.sqrt(c1 * (1 - c1) / n)
    assert abs(acc - c1) < half


def test_expected_accepted_length_matches_survival_sum():
    """With a prefix-free draft and target the acceptances are independent with
    probability c*_k, so E[n + 1] = 1 + sum_j prod_{i<=j} c*_i."""
    n = 12000
    runs, _, _ = _mc_pipeline(n, seed=9, zero_transition=True, markov_target=False)
    c = runs[0][1]["c_star"]
    expect = 1.0 + sum(np.prod(c[:j]) for j in range(1, len(c) + 1))
    L = np.array([v["n_acc"] + 1 for _, v in runs], dtype=np.float64)
    assert abs(L.mean() - expect) < 4.0 * L.std() / math.sqrt(n)
    assert all(np.allclose(v["c_star"], c, atol=1e-12) for _, v in runs[:50])


# ------------------------------------------------------------------ scheduler
def _survival(c):
    c = np.asarray(c, dtype=np.float32)
    ones = np.ones(2 * c.size + 2)
    return oracle.schedule(np.asarray(c, dtype=np.float32)[None, :], ones, oracle.SCHED_OFF)["a"][0]


def test_survival_printed_examples():
    g = golden("survival_examples.json")
    first, second, third = g["cases"]
    a = _survival(first["c"])
    for val, printed, dec in zip(a, first["printed_reach"], first["printed_decimals"]):
        assert round(float(val), dec) == printed
    assert round(float(_survival(second["c"])[-1]), second["printed_decimals_last"]) == \
        second["printed_last"]
    assert round(float(_survival(third["c"])[-1]), third["printed_decimals_last"]) == \
        third["printed_last"]
    # to binary32 rounding of the exact products
    for case in g["cases"]:
        exact = np.cumprod(np.array(case["c"], dtype=np.float32).astype(np.float64))
        assert np.allclose(_survival(case["c"]), exact, rtol=4e-7)


def test_survival_non_increasing():
    rng = np.random.default_rng(10)
    c = rng.random((50, 16)).astype(np.float32)
    c[3, 4] = 1.0
    c[7, :] = 1.0
    a = oracle.schedule(c, np.ones(50 * 17 + 1), oracle.SCHED_OFF)["a"]
    assert np.all(np.diff(a, axis=1) <= 0)


def test_throughput_printed_example():
    g = golden("throughput_example.json")
    base, high, low = g["rows"]
    for row in g["rows"]:
        assert row["tau"] * row["sps"] == pytest.approx(row["theta"])
    for mode in (oracle.SCHED_EARLY_STOP, oracle.SCHED_FULL_SEARCH):
        assert oracle.select_n([base["tau"] * base["sps"], high["tau"] * high["sps"]], mode) == 1
        assert oracle.select_n([base["tau"] * base["sps"], low["tau"] * low["sps"]], mode) == 0


def test_greedy_order_printed_example():
    g = golden("greedy_order_example.json")
    A, B = g["cumulative_survival"]["A"], g["cumulative_survival"]["B"]
    c = np.array([[A[0], A[1] / A[0]], [B[0], B[1] / B[0]]], dtype=np.float32)
    R, gamma = c.shape
    # one SPS table per budget: flat up to B = R + n, then a cliff
    expect = {1: [1, 0], 2: [1, 1], 3: [2, 1]}   # A1 | A1 B1 | A1 B1 A2
    for n, ell in expect.items():
        sps = np.ones(R * (1 + gamma) + 1)
        sps[R + n + 1:] = 0.01
        for mode in (oracle.SCHED_EARLY_STOP, oracle.SCHED_FULL_SEARCH):
            out = oracle.schedule(c, sps, mode)
            assert out["n_admitted"] == n and list(out["ell"]) == ell


def _check_prefix_closed_top_n(c, out):
    a = out["a"]
    R, gamma = a.shape
    rho, j = np.meshgrid(np.arange(R), np.arange(1, gamma + 1), indexing="ij")
    order = np.lexsort((rho.ravel(), j.ravel(), -a.ravel().astype(np.float64)))
    n = out["n_admitted"]
    admitted = np.zeros(R * gamma, dtype=bool)
    admitted[order[:n]] = True
    admitted = admitted.reshape(R, gamma)
    for p in range(R):
        L = int(out["ell"][p])
        assert admitted[p].sum() == L and admitted[p, :L].all(), "admitted set not a prefix"
    assert list(out["row_offset"]) == list(np.concatenate([[0], np.cumsum(1 + out["ell"])]))


@pytest.mark.parametrize("seed", range(6))
def test_schedule_full_search_equals_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    R, gamma = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    c = rng.random((R, gamma)).astype(np.float32)
    if seed % 2:
        c[0, :] = 1.0  # repeated survival values exercise the tie order
        c[-1, 0] = c[0, 0]
    B = np.arange(R * (1 + gamma) + 1, dtype=np.float64)
    sps = (100.0 / (1.0 + B / rng.uniform(1, 8))) if seed < 3 else \
        60.0 * 16 / (16 + 4 * np.ceil(B / 4))
    best, ell_b = oracle.schedule_bruteforce(c, sps)
    full = oracle.schedule(c, sps, oracle.SCHED_FULL_SEARCH)
    assert full["theta"] == best  # bitwise: same fixed-point tau and fp64 product
    assert full["n_admitted"] == int(ell_b.sum())
    early = oracle.schedule(c, sps, oracle.SCHED_EARLY_STOP)
    assert early["theta"] <= full["theta"]
    for out in (full, early):
        _check_prefix_closed_top_n(c, out)


def test_schedule_modes_on_config_shapes():
    import synth
    cfg = synth.CONFIGS[4]
    c, cp = synth.confidences(cfg), synth.confidences(cfg, older=True)
    sps = synth.sps_table(cfg)
    asy = oracle.schedule(c, sps, oracle.SCHED_ASYNC_TOPK, c_prev2=cp)
    K = oracle.schedule(cp, sps, oracle.SCHED_FULL_SEARCH)["n_admitted"]
    assert asy["n_admitted"] == K and int(asy["ell"].sum()) == K
    _check_prefix_closed_top_n(c, asy)
    full = oracle.schedule(c, sps, oracle.SCHED_FULL_SEARCH)
    early = oracle.schedule(c, sps, oracle.SCHED_EARLY_STOP)
    # stepped SPS: theta is flat in SPS inside a bucket and tau grows, so the
    # full-search optimum sits on a bucket edge unless the candidates run out
    B_star = cfg.R + full["n_admitted"]
    assert B_star % 64 == 0 or full["n_admitted"] == cfg.R * cfg.gamma
    assert early["theta"] <= full["theta"]
    off = oracle.schedule(None, None, oracle.SCHED_OFF, R=cfg.R, gamma=cfg.gamma)
    assert np.all(off["ell"] == cfg.gamma) and off["n_admitted"] == cfg.R * cfg.gamma
    assert np.isnan(off["theta"])


def test_schedule_rejects_bad_confidence():
    c = np.array([[0.5, 1.5]], dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.schedule(c, np.ones(8), oracle.SCHED_EARLY_STOP)
    c = np.array([[0.5, np.nan]], dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.schedule(c, np.ones(8), oracle.SCHED_EARLY_STOP)


# ------------------------------------------- scheduler tie rules (readings)
# KB section 4 stops the non-anticipating scheduler the first time theta does
# not increase, so a plateau ends admission; Bangkok 4.2.2's "stops once it
# drops" would admit through it.  The pins below take the first reading, and
# the full search returns the smallest maximiser (no extra verify slot for the
# same expected throughput).  Each case has an exact fp64 tie.
def test_select_n_tie_rules_on_theta_paths():
    # a plateau, then a rise: early stop halts at the plateau, full search
    # finds the later maximum
    assert oracle.select_n([4.0, 6.0, 6.0, 8.0], oracle.SCHED_EARLY_STOP) == 1
    assert oracle.select_n([4.0, 6.0, 6.0, 8.0], oracle.SCHED_FULL_SEARCH) == 3
    # equal maxima apart: the smaller admission count wins
    assert oracle.select_n([1.0, 2.0, 1.5, 2.0], oracle.SCHED_FULL_SEARCH) == 1
    assert oracle.select_n([1.0, 2.0, 1.5, 2.0], oracle.SCHED_EARLY_STOP) == 1
    # a flat start admits nothing under either rule
    assert oracle.select_n([3.0, 3.0, 5.0], oracle.SCHED_EARLY_STOP) == 0
    assert oracle.select_n([3.0, 3.0, 2.0], oracle.SCHED_FULL_SEARCH) == 0


def test_schedule_zero_confidence_plateau():
    """Zero-confidence candidates add nothing to tau; under a flat SPS they
    leave theta unchanged, so neither rule admits them."""
    c = np.array([[1.0, 1.0], [0.0, 0.0]], dtype=np.float32)
    sps = np.ones(2 * 3 + 1)
    for mode in (oracle.SCHED_EARLY_STOP, oracle.SCHED_FULL_SEARCH):
        out = oracle.schedule(c, sps, mode)
        assert out["n_admitted"] == 2 and list(out["ell"]) == [2, 0]
        assert out["theta"] == 4.0
    best, ell_b = oracle.schedule_bruteforce(c, sps)
    assert best == 4.0 and list(ell_b) == [2, 0]


def test_schedule_plateau_before_a_rise():
    """One request, c = 1 everywhere (tau_n = 1 + n), SPS chosen so that
    theta = 4, 6, 6, 8: early stop admits 1, full search 3."""
    c = np.ones((1, 3), dtype=np.float32)
    sps = np.array([0.0, 4.0, 3.0, 2.0, 2.0])
    assert oracle.schedule(c, sps, oracle.SCHED_EARLY_STOP)["n_admitted"] == 1
    full = oracle.schedule(c, sps, oracle.SCHED_FULL_SEARCH)
    assert full["n_admitted"] == 3 and full["theta"] == 8.0


def test_schedule_full_search_two_equal_maxima():
    """theta = 1, 2, 1.5, 2: the smallest maximiser (1) and the brute force
    over allocations, whose own tie rule prefers fewer admitted drafts, agree."""
    c = np.ones((1, 3), dtype=np.float32)
    sps = np.array([0.0, 1.0, 1.0, 0.5, 0.5])
    full = oracle.schedule(c, sps, oracle.SCHED_FULL_SEARCH)
    assert full["n_admitted"] == 1 and full["theta"] == 2.0
    best, ell_b = oracle.schedule_bruteforce(c, sps)
    assert best == 2.0 and list(ell_b) == [1]
    asy = oracle.schedule(c, sps, oracle.SCHED_ASYNC_TOPK, c_prev2=c)
    assert asy["n_admitted"] == 1


def test_threshold_keeps_a_confidence_equal_to_the_cutoff():
    """Only drafts below the cutoff are dropped (Bangkok 5.3): c equal to it is kept."""
    c = np.array([[0.5, 0.5, 0.25], [0.25, 0.5, 0.5]], dtype=np.float32)
    out = oracle.schedule(c, None, oracle.SCHED_THRESHOLD, threshold=0.5)
    assert list(out["ell"]) == [2, 0]


def test_negative_zero_confidence_is_zero():
    """-0.0 is the probability 0: every output equals that of +0.0 bit for bit,
    and the survival products carry no negative sign."""
    rng = np.random.default_rng(17)
    c = rng.uniform(0.2, 1.0, (6, 4)).astype(np.float32)
    c[1, 0] = c[3, 2] = c[4, 3] = 0.0
    cn = c.copy()
    cn[1, 0] = cn[3, 2] = cn[4, 3] = np.float32(-0.0)
    sps = np.ones(6 * 5 + 1)
    sps[6 + 20:] = 0.5
    for mode in (oracle.SCHED_OFF, oracle.SCHED_EARLY_STOP, oracle.SCHED_FULL_SEARCH,
                 oracle.SCHED_ASYNC_TOPK, oracle.SCHED_THRESHOLD):
        kw = dict(c_prev2=cn) if mode == oracle.SCHED_ASYNC_TOPK else {}
        o_pos = oracle.schedule(c, sps, mode, threshold=0.3, **({"c_prev2": c} if kw else {}))
        o_neg = oracle.schedule(cn, sps, mode, threshold=0.3, **kw)
        for key in ("ell", "row_offset"):
            assert np.array_equal(o_pos[key], o_neg[key])
        assert o_pos["n_admitted"] == o_neg["n_admitted"] and o_pos["theta"] == o_neg["theta"]
        assert np.array_equal(o_pos["a"].view(np.uint32), o_neg["a"].view(np.uint32))
        assert not np.signbit(o_neg["a"]).any()


# ---------------------------------------- sequential temperature scaling (STS)
def test_sts_head_divides_the_logit():
    """c = sigmoid(z / T): against the T = 1 head of the same inputs."""
    rng = np.random.default_rng(6)
    V, r, d = 16, 8, 24
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    h = rng.standard_normal(d).astype(np.float32)
    w = (0.3 * rng.standard_normal(d + r)).astype(np.float32)
    c1 = oracle.conf_head(h, w, np.float32(0.4), W1, 5)
    z = special.logit(c1)
    for T in (0.5, 2.0, 7.0):
        assert oracle.conf_head(h, w, np.float32(0.4), W1, 5, T=T) == \
            pytest.approx(special.expit(z / T), rel=1e-12)
    # a very hot position says nothing: 1/2
    assert abs(oracle.conf_head(h, w, np.float32(0.4), W1, 5, T=1e6) - 0.5) < 1e-5


def test_sts_printed_example():
    """Blog, "Sequential temperature scaling": raw confidences 0.98, 0.92, 0.80
    against empirical survival 0.94, 0.82, 0.65.  Fitting left to right (each
    position's temperature makes the survival through it match, the earlier
    ones frozen) and applying the temperatures to the raw logits reproduces the
    printed survival, and leaves the ranking of the raw scores unchanged."""
    raw = np.array([0.98, 0.92, 0.80])
    surv = np.array([0.94, 0.82, 0.65])
    d, r, V = 8, 8, 4
    h = np.zeros(d, dtype=np.float32)
    w = np.zeros(d + r, dtype=np.float32)
    W1 = np.zeros((V, r), dtype=np.float32)
    T = []
    a = 1.0
    for k in range(3):
        target = surv[k] / a                        # conditional c that matches survival k
        T.append(special.logit(raw[k]) / special.logit(target))
        c = oracle.conf_head(h, w, np.float32(special.logit(raw[k])), W1, 0, T=T[-1])
        a *= c
        assert a == pytest.approx(surv[k], abs=1e-6)
    # the calibration makes the head less confident at every position
    assert all(t > 1.0 for t in T)


def test_draft_request_applies_position_temperatures():
    rng = np.random.default_rng(7)
    gamma, V, r, d = 3, 32, 8, 16
    U = rng.standard_normal((gamma, V)).astype(np.float32)
    W1 = (0.5 * rng.standard_normal((V, r))).astype(np.float32)
    W2 = (0.5 * rng.standard_normal((V, r))).astype(np.float32)
    h = rng.standard_normal((gamma, d)).astype(np.float32)
    w = (0.2 * rng.standard_normal(d + r)).astype(np.float32)
    T = np.array([0.7, 1.0, 3.0], dtype=np.float32)
    out = oracle.draft_request(U, W1, W2, 2, 1, 0, 0, h_req=h, w_conf=w, b_conf=0.3, conf_temp=T)
    prev = [2, out["x"][0], out["x"][1]]
    for k in range(gamma):
        assert out["c"][k] == oracle.conf_head(h[k], w, np.float32(0.3), W1, prev[k], T=float(T[k]))
    with pytest.raises(AssertionError):
        oracle.draft_request(U, W1, W2, 2, 1, 0, 0, h_req=h, w_conf=w, b_conf=0.3,
                             conf_temp=np.array([1.0, 0.0, 1.0], dtype=np.float32))


# ------------------------------------------ static confidence-threshold admission
def test_threshold_schedule_prefixes_and_limits():
    rng = np.random.default_rng(8)
    R, gamma = 12, 6
    c = rng.uniform(0.05, 1.0, (R, gamma)).astype(np.float32)
    sps = 100.0 / (1.0 + np.arange(R * (gamma + 1) + 1) / 8.0)
    prev_ell = np.full(R, gamma + 1)
    for thr in np.float32([0.0, 0.2, 0.5, 0.7, 0.9, 1.01]):
        s = oracle.schedule(c, sps, oracle.SCHED_THRESHOLD, threshold=thr)
        ell = s["ell"]
        for rho in range(R):
            kept = c[rho, : ell[rho]]
            assert np.all(kept >= thr)                              # kept tokens pass
            assert ell[rho] == gamma or c[rho, ell[rho]] < thr      # stopped at the first miss
        assert np.all(ell <= prev_ell)                              # monotone in the cutoff
        prev_ell = ell
        assert s["n_admitted"] == ell.sum()
        assert np.array_equal(s["row_offset"], np.concatenate(([0], np.cumsum(1 + ell))))
    assert np.all(oracle.schedule(c, sps, oracle.SCHED_THRESHOLD, threshold=0.0)["ell"] == gamma)
    assert np.all(oracle.schedule(c, sps, oracle.SCHED_THRESHOLD, threshold=1.01)["ell"] == 0)


def test_threshold_theta_agrees_with_other_modes():
    """Every token kept: theta is the scheduler-off theta of the same c; none
    kept: R * SPS[R], the full path's theta_0; no SPS table: NaN."""
    rng = np.random.default_rng(9)
    R, gamma = 10, 5
    c = rng.uniform(0.3, 1.0, (R, gamma)).astype(np.float32)
    sps = 60.0 * 1024.0 / (1024.0 + np.arange(R * (gamma + 1) + 1))
    all_kept = oracle.schedule(c, sps, oracle.SCHED_THRESHOLD, threshold=0.0)
    off = oracle.schedule(c, sps, oracle.SCHED_OFF)
    assert all_kept["theta"] == off["theta"] and np.array_equal(all_kept["a"], off["a"])
    none_kept = oracle.schedule(c, sps, oracle.SCHED_THRESHOLD, threshold=1.5)
    assert none_kept["theta"] == R * sps[R]
    assert np.isnan(oracle.schedule(c, None, oracle.SCHED_THRESHOLD, threshold=0.5)["theta"])


# ------------------------------------------------------------ training losses
# Blog, "Training objective", and the knowledge-base summary of the paper's
# training recipe: L = a_ce L_ce + a_tv L_tv + a_conf L_conf with defaults
# (0.1, 0.9, 1.0), position weights w_k = exp(-(k - 1) / gamma), hard CE, an
# L1 target/draft distance, BCE of the confidence against c*, all on the
# ground-truth prefix.
def _train_inputs(R, gamma, V, r, seed=0):
    g = np.random.default_rng(seed)
    U = g.normal(0, 1.0, (R, gamma, V)).astype(np.float32)
    W1 = g.normal(0, 0.5, (V, r)).astype(np.float32)
    W2 = g.normal(0, 0.5, (V, r)).astype(np.float32)  # column-major r x V factor
    P = g.normal(0, 1.5, (R, gamma + 1, V)).astype(np.float32)
    x0 = g.integers(0, V, R).astype(np.int32)
    y = g.integers(0, V, (R, gamma)).astype(np.int32)
    c = g.uniform(0.05, 0.95, (R, gamma)).astype(np.float32)
    return U, W1, W2, x0, y, P, c


def test_train_losses_uniform_case():
    """All-zero logits on both sides: q = p = uniform, so CE = log V, the L1
    distance is 0, c* = 1 and the BCE reduces to -log c.  Equal per-position
    values make every weighted mean equal to that value."""
    R, gamma, V, r = 2, 5, 8, 3
    U = np.zeros((R, gamma, V), np.float32)
    W1 = np.zeros((V, r), np.float32)
    W2 = np.zeros((V, r), np.float32)
    P = np.zeros((R, gamma + 1, V), np.float32)
    x0 = np.array([1, 6], np.int32)
    y = np.arange(R * gamma, dtype=np.int32).reshape(R, gamma) % V
    c = np.full((R, gamma), 0.8, np.float32)
    per, tot = oracle.train_losses(U, W1, W2, x0, y, P, c)
    np.testing.assert_allclose(per[0], math.log(V), rtol=1e-14)
    np.testing.assert_allclose(per[1], 0.0, atol=1e-15)
    np.testing.assert_allclose(per[2], -math.log(np.float32(0.8)), rtol=1e-12)
    lce, lconf = math.log(V), -math.log(np.float32(0.8))
    np.testing.assert_allclose(tot, [lce, 0.0, lconf, 0.1 * lce + lconf], rtol=1e-12, atol=1e-15)


def test_train_losses_teacher_forced_prefix_and_weights():
    """A head whose bias only lifts token 2 after token 1: with W2 row (0, 0,
    40, 0) and W1[1] = 1 (other rows 0) the draft is uniform unless the
    previous token is 1.  The prefix must come from the labels (x0, then
    y_{k-1}), and the label scored at position k is y_k.  Request 0 sees
    CE = (log 4, ~0, log 4); request 1 scores token 3 after token 1, CE ~ 40.
    The totals are position-weighted means with w_k = exp(-(k - 1) / gamma),
    averaged over requests."""
    R, gamma, V, r = 2, 3, 4, 1
    U = np.zeros((R, gamma, V), np.float32)
    W1 = np.array([[0.0], [1.0], [0.0], [0.0]], np.float32)
    W2 = np.array([[0.0, 0.0, 40.0, 0.0]], np.float32)
    P = np.zeros((R, gamma + 1, V), np.float32)
    x0 = np.array([0, 1], np.int32)
    y = np.array([[1, 2, 3], [3, 0, 0]], np.int32)
    c = np.full((R, gamma), 0.5, np.float32)
    per, tot = oracle.train_losses(U, W1, W2, x0, y, P, c)
    peak = 40.0 - math.log(math.exp(40.0) + 3.0)  # log q(2) after token 1
    low = -math.log(math.exp(40.0) + 3.0)         # log q(v != 2) after token 1
    np.testing.assert_allclose(per[0][0], [math.log(4), -peak, math.log(4)], rtol=1e-12)
    np.testing.assert_allclose(per[0][1], [-low, math.log(4), math.log(4)], rtol=1e-12)
    w = np.exp(-np.arange(gamma) / gamma)
    req = (per[0] * w).sum(1) / w.sum()
    np.testing.assert_allclose(tot[0], req.mean(), rtol=1e-14)
    # weights favour early positions: the first request's loss sits at k = 1, 3
    np.testing.assert_allclose(req[0], math.log(4) * (w[0] + w[2]) / w.sum(), rtol=1e-12)


def test_train_losses_l1_is_twice_one_minus_cstar():
    """The L1 distance of two distributions equals 2 (1 - sum min(p, q)) (twice
    the total variation); the BCE is linear in its soft label, so c* can be
    read back from it and the two losses checked against each other."""
    U, W1, W2, x0, y, P, c = _train_inputs(3, 6, 50, 4, seed=11)
    per, _ = oracle.train_losses(U, W1, W2, x0, y, P, c, temp=0.8)
    cd = c.astype(np.float64)
    cs = (per[2] + np.log1p(-cd)) / (np.log1p(-cd) - np.log(cd))
    assert np.all((cs > 0) & (cs < 1))
    np.testing.assert_allclose(per[1], 2.0 * (1.0 - cs), rtol=1e-9, atol=1e-12)


def test_train_losses_temperature_and_library_softmax():
    """With W1 = W2 = 0 the draft logits are U, so CE is scipy's log-softmax of
    U / T at the label; a target row equal to U gives p = q at any T (L1 = 0,
    c* = 1)."""
    R, gamma, V, r = 2, 4, 33, 2
    U, _, _, x0, y, _, c = _train_inputs(R, gamma, V, r, seed=5)
    W1 = np.zeros((V, r), np.float32)
    W2 = np.zeros((V, r), np.float32)
    P = np.zeros((R, gamma + 1, V), np.float32)
    P[:, :gamma] = U
    T = 0.6
    per, tot = oracle.train_losses(U, W1, W2, x0, y, P, c, temp=T)
    ls = special.log_softmax(U.astype(np.float64) / T, axis=-1)
    ce = -np.take_along_axis(ls, y[..., None].astype(np.int64), -1)[..., 0]
    np.testing.assert_allclose(per[0], ce, rtol=1e-12)
    np.testing.assert_allclose(per[1], 0.0, atol=1e-12)
    np.testing.assert_allclose(per[2], -np.log(c.astype(np.float64)), rtol=1e-9)


def test_train_losses_alpha_combination_is_linear():
    args = _train_inputs(2, 4, 40, 3, seed=2)
    _, tot = oracle.train_losses(*args)
    for i, a in enumerate([(1, 0, 0), (0, 1, 0), (0, 0, 1)]):
        _, t = oracle.train_losses(*args, alpha=a)
        assert t[3] == pytest.approx(tot[i], rel=1e-14)
    assert tot[3] == pytest.approx(0.1 * tot[0] + 0.9 * tot[1] + tot[2], rel=1e-14)


# ------------------------------------------------------------ recurrent head
# Blog, "RNN sequential head"; KB section 3: s_k = f(s_{k-1}, E(x_{k-1}), h_k)
# with a gated update, read as the standard GRU.
def _gru_case(V, r, gamma, bf16, seed):
    g = np.random.default_rng(seed)
    GE = g.normal(0, 1.0, (V, 3 * r)).astype(np.float32)
    Gh = g.normal(0, 1.0, (gamma, 3 * r)).astype(np.float32)
    Whh = g.normal(0, 0.4, (r, 3 * r)).astype(np.float32)
    bhh = g.normal(0, 0.5, 3 * r).astype(np.float32)
    s0 = g.normal(0, 0.5, r).astype(np.float32)
    x0 = int(g.integers(0, V))
    x = g.integers(0, V, gamma - 1).astype(np.int32)
    if bf16:
        import synth
        GE, Whh = synth.to_bf16_bits(GE), synth.to_bf16_bits(Whh)
    return GE, Gh, Whh, bhh, s0, x0, x


@pytest.mark.parametrize("bf16", [False, True])
def test_rnn_states_match_library_gru_cell(bf16):
    """torch.nn.GRUCell (float64) with input u = [one-hot(x_{k-1}); G_h[k]],
    input weights [G_E^T | I] and no input bias has input pre-activations
    exactly G_E[x_{k-1}] + G_h[k]; its recurrent weights are W_hh (stored
    column-major here) and b_hh."""
    import torch
    import synth
    V, r, gamma = 11, 8, 6
    GE, Gh, Whh, bhh, s0, x0, x = _gru_case(V, r, gamma, bf16, seed=3)
    wid = (lambda a: synth.bf16_bits_to_f32(a)) if bf16 else (lambda a: a)
    cell = torch.nn.GRUCell(V + 3 * r, r, dtype=torch.float64)
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(np.concatenate(
            [wid(GE).astype(np.float64).T, np.eye(3 * r)], axis=1)))
        cell.bias_ih.zero_()
        cell.weight_hh.copy_(torch.from_numpy(wid(Whh).astype(np.float64).T))
        cell.bias_hh.copy_(torch.from_numpy(bhh.astype(np.float64)))
        s = torch.from_numpy(s0.astype(np.float64))[None]
        ref = []
        for k in range(1, gamma + 1):
            prev = x0 if k == 1 else int(x[k - 2])
            u = torch.zeros(1, V + 3 * r, dtype=torch.float64)
            u[0, prev] = 1.0
            u[0, V:] = torch.from_numpy(Gh[k - 1].astype(np.float64))
            s = cell(u, s)
            ref.append(s[0].numpy().copy())
    got = oracle.rnn_states(GE, Gh, Whh, bhh, x0, x, s0=s0)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-12, atol=1e-14)


def test_rnn_states_closed_forms():
    """A saturated update gate keeps the state (s_k = s_0); a closed update
    gate with zero recurrent weights gives s_k = tanh(g_n) regardless of the
    past; s0 = None starts from zeros."""
    V, r, gamma = 7, 4, 3
    GE, Gh, Whh, bhh, s0, x0, x = _gru_case(V, r, gamma, False, seed=9)
    GEk = GE.copy()
    GEk[:, r:2 * r] = 60.0
    got = oracle.rnn_states(GEk, Gh, Whh, bhh, x0, x, s0=s0)
    np.testing.assert_allclose(got, np.tile(s0.astype(np.float64), (gamma, 1)), atol=1e-12)
    GEo = GE.copy()
    GEo[:, r:2 * r] = -60.0
    Z = np.zeros_like(Whh)
    bz = np.zeros_like(bhh)
    got = oracle.rnn_states(GEo, Gh, Z, bz, x0, x, s0=s0)
    for k in range(1, gamma + 1):
        prev = x0 if k == 1 else int(x[k - 2])
        want = np.tanh(GEo[prev, 2 * r:].astype(np.float64) + Gh[k - 1, 2 * r:])
        np.testing.assert_allclose(got[k - 1], want, rtol=1e-12, atol=1e-14)
    a = oracle.rnn_states(GE, Gh, Whh, bhh, x0, x, s0=None)
    b = oracle.rnn_states(GE, Gh, Whh, bhh, x0, x, s0=np.zeros(r, np.float32))
    assert np.array_equal(a, b)


def test_verify_with_given_rows_equals_table_rows():
    """Verification with the transition rows given explicitly equals the
    table form when the given rows are the table's rows W1[x_{k-1}]."""
    g = np.random.default_rng(4)
    gamma, V, r = 4, 300, 16
    U = g.normal(0, 1, (gamma, V)).astype(np.float32)
    P = g.normal(0, 1, (gamma + 1, V)).astype(np.float32)
    W1 = g.normal(0, 0.5, (V, r)).astype(np.float32)
    W2 = g.normal(0, 0.5, (V, r)).astype(np.float32)
    x0 = 5
    x = g.integers(0, V, gamma).astype(np.int32)
    prevs = np.concatenate([[x0], x[:-1]])
    a = oracle.verify_request(P, U, W1, W2, x0, x, gamma, 1, 2, 0)
    b = oracle.verify_request(P, U, None, W2, x0, x, gamma, 1, 2, 0, A_rows=W1[prevs])
    for key in ("n_acc", "y", "c_star", "ratio"):
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key]), equal_nan=True), key
