"""GPU parity of the forward-only training reductions (dspark_train_losses)
against the oracle's teacher-forced losses.

Small shapes (several vocabulary tiles and a ragged last tile, fp32 and bf16,
two temperatures): every position's (CE, L1, BCE) and the four totals.  The
full b128-long-block shape (R = 128, gamma = 16, V = 151936, r = 256, bf16):
the oracle on sampled requests, and at every position the property that the
totals are the position-weighted request means of the per-position values.

Tolerances: c* is a sum over V in fp32 on the device, so L1 = 2 (1 - c*) gets
twice the c* bound (1e-5 fp32 inputs, 2e-3 bf16 inputs), and the BCE that
bound times |log(c / (1 - c))|; CE = -log q(y) from fp32 logits and an fp32
normaliser: 1e-4 absolute plus 1e-5 relative.
"""
import math

import numpy as np
import pytest
import torch

import draft_sampling_verification_03_amd as ds
import oracle
import synth
from gpu_common import dev, prob_tol

pytestmark = pytest.mark.gpu

ALPHA = (0.1, 0.9, 1.0)


def labels_and_conf(cfg, T):
    """Labels: the target row's argmax at about half of the positions, a
    uniform token elsewhere; confidences uniform in (0.02, 0.98)."""
    g = np.random.default_rng(np.random.SeedSequence([77, cfg.R, cfg.gamma, cfg.V]))
    Tf = synth.as_f32(cfg, T[:, : cfg.gamma])
    y = np.where(g.random((cfg.R, cfg.gamma)) < 0.5, Tf.argmax(-1),
                 g.integers(0, cfg.V, (cfg.R, cfg.gamma))).astype(np.int32)
    c = g.uniform(0.02, 0.98, (cfg.R, cfg.gamma)).astype(np.float32)
    return y, c


def tolerances(cfg, c):
    pt = prob_tol(cfg)
    lr = np.abs(np.log(c.astype(np.float64)) - np.log1p(-c.astype(np.float64)))
    return 2 * pt, pt * lr + 1e-5


def check_per_pos(cfg, per_gpu, per_orc, c):
    tl1, tbce = tolerances(cfg, c)
    ce_err = np.abs(per_gpu[0] - per_orc[0])
    assert np.all(ce_err <= 1e-4 + 1e-5 * np.abs(per_orc[0])), ce_err.max()
    assert np.all(np.abs(per_gpu[1] - per_orc[1]) <= tl1), np.abs(per_gpu[1] - per_orc[1]).max()
    assert np.all(np.abs(per_gpu[2] - per_orc[2]) <= tbce), np.abs(per_gpu[2] - per_orc[2]).max()


def weighted_totals(per, gamma, alpha=ALPHA):
    w = np.exp(-np.arange(gamma) / gamma)
    t = [float(((per[i] * w).sum(1) / w.sum()).mean()) for i in range(3)]
    return np.array(t + [alpha[0] * t[0] + alpha[1] * t[1] + alpha[2] * t[2]])


@pytest.mark.parametrize("shape,temp", [
    (dict(R=3, gamma=5, V=1000, r=16, dtype=synth.F32), 1.0),
    (dict(R=3, gamma=5, V=1000, r=16, dtype=synth.F32), 0.7),
    (dict(R=5, gamma=7, V=2056, r=32, dtype=synth.BF16), 1.0),
    (dict(R=2, gamma=1, V=136, r=16, dtype=synth.BF16), 1.3),
    (dict(R=4, gamma=3, V=1000, r=256, dtype=synth.BF16, weight_sd=0.05), 1.0),  # single launch
    # the single launch past 128 requests (two chunks) and the W2-stationary
    # verify product (R gamma > 256)
    (dict(R=160, gamma=2, V=20000, r=256, dtype=synth.BF16, weight_sd=0.05), 1.0),
])
def test_train_losses_match_oracle_small(shape, temp):
    cfg = synth.make_config(1, **shape)
    print(f"[train] {shape} temp={temp}", flush=True)
    U, T = synth.generate(cfg, workers=4)
    W1, W2, x0 = synth.W1(cfg), synth.W2(cfg), synth.anchors(cfg)
    y, c = labels_and_conf(cfg, T)
    out = ds.train_losses(dev(U), dev(W1), dev(W2), dev(T), dev(x0), dev(y), dev(c), temp=temp,
                          alpha=ALPHA)
    per_gpu = out["per_pos"].cpu().numpy().astype(np.float64)
    tot_gpu = out["totals"].cpu().numpy()
    per_orc, tot_orc = oracle.train_losses(U, W1, W2, x0, y, T, c, temp=temp, alpha=ALPHA)
    check_per_pos(cfg, per_gpu, per_orc, c)
    tl1, tbce = tolerances(cfg, c)
    np.testing.assert_allclose(tot_gpu[0], tot_orc[0], atol=1e-4, rtol=1e-5)
    assert abs(tot_gpu[1] - tot_orc[1]) <= tl1
    assert abs(tot_gpu[2] - tot_orc[2]) <= tbce.max()
    np.testing.assert_allclose(tot_gpu, weighted_totals(per_gpu, cfg.gamma), rtol=1e-6, atol=1e-7)


def test_train_losses_full_shape_sampled_requests():
    cfg = synth.CONFIGS[3]
    print(f"[train] {cfg.name}", flush=True)
    U, T = synth.generate(cfg, workers=16)
    W1, W2, x0 = synth.W1(cfg), synth.W2(cfg), synth.anchors(cfg)
    y, c = labels_and_conf(cfg, T)
    out = ds.train_losses(dev(U), dev(W1), dev(W2), dev(T), dev(x0), dev(y), dev(c))
    per_gpu = out["per_pos"].cpu().numpy().astype(np.float64)
    tot_gpu = out["totals"].cpu().numpy()
    assert np.all(np.isfinite(per_gpu))
    assert np.all(per_gpu[1] >= -1e-3) and np.all(per_gpu[1] <= 2.0 + 1e-3)
    np.testing.assert_allclose(tot_gpu, weighted_totals(per_gpu, cfg.gamma), rtol=1e-6, atol=1e-7)
    for rho in (0, 77, cfg.R - 1):
        sl = slice(rho, rho + 1)
        per_orc, _ = oracle.train_losses(U[sl], W1, W2, x0[sl], y[sl], T[sl], c[sl], alpha=ALPHA)
        check_per_pos(cfg, per_gpu[:, sl], per_orc, c[sl])
    # the same call twice is bit-identical (fixed-order reductions)
    out2 = ds.train_losses(dev(U), dev(W1), dev(W2), dev(T), dev(x0), dev(y), dev(c))
    assert torch.equal(out["per_pos"], out2["per_pos"])
    assert torch.equal(out["totals"], out2["totals"])


def test_train_losses_equal_distributions_and_bad_label():
    """A target row equal to the draft logits (W1 = W2 = 0, so q = softmax(U))
    gives L1 = 0 and c* = 1 on the device as well; an out-of-range label sets
    the token bit of the device error word."""
    cfg = synth.make_config(1, R=2, gamma=3, V=1024, r=16, dtype=synth.F32)
    U, T = synth.generate(cfg)
    T[:, : cfg.gamma] = U
    W1 = np.zeros_like(synth.W1(cfg))
    W2 = np.zeros_like(synth.W2(cfg))
    x0 = synth.anchors(cfg)
    y, c = labels_and_conf(cfg, T)
    ws = ds.Workspace()
    out = ds.train_losses(dev(U), dev(W1), dev(W2), dev(T), dev(x0), dev(y), dev(c), ws=ws)
    per = out["per_pos"].cpu().numpy()
    assert ws.error_code() == 0
    assert np.all(np.abs(per[1]) <= 2e-5)
    np.testing.assert_allclose(per[2], -np.log(c.astype(np.float64)), rtol=1e-4, atol=2e-5)
    bad = y.copy()
    bad[1, 2] = cfg.V
    ds.train_losses(dev(U), dev(W1), dev(W2), dev(T), dev(x0), dev(bad), dev(c), ws=ws)
    assert ws.error_code() & 1
    ws.clear_error()
    assert ws.error_code() == 0
    assert math.isfinite(float(out["totals"][3]))
