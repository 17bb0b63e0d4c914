"""Seeded synthetic inputs for the DSpark per-round hot path.

This module only draws inputs; it holds none of the method's arithmetic.  Both
the HIP library's tests/benchmark and the CPU oracle take their inputs from
here.  Every tensor row is drawn from its own numpy ``SeedSequence``
([config, tensor, indices...]) so that any single row can be regenerated on
its own (the oracle checks sampled rows of the large configurations without
materializing them), and identical bytes go to both sides.

bf16 tensors are float32 normals rounded to bfloat16 (round to nearest even)
and stored as uint16 bit patterns.

The five workloads stand in for the shapes the pages discuss: batch 128 with
blocks of 4-16 (Bangkok 5.3, cost at batch 128), the fixed 7-token offline
block (Bangkok 5.1), gamma = 15 (Bangkok 5.3), the production V4 drafter's
gamma <= 5 (KB section 7) and a hidden size near 4096 (Blog, "Hidden-state
communication").  No dataset or trained weight is involved.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32, BF16 = 0, 1
SCHED_OFF, SCHED_EARLY_STOP, SCHED_FULL_SEARCH, SCHED_ASYNC_TOPK, SCHED_THRESHOLD = 0, 1, 2, 3, 4

# tensor ids of the seed sequences
_T_TARGET, _T_UNOISE, _T_W1, _T_W2, _T_X0, _T_C, _T_CPREV, _T_SIGMA, _T_H, _T_WCONF = range(10)


@dataclass
class Config:
    cid: int
    name: str
    R: int
    gamma: int
    V: int
    r: int
    dtype: int
    target_sd: float
    noise: str            # "const:<sd>" or "uniform:<lo>:<hi>" (per-request sd)
    weight_sd: float
    conf: Optional[str]   # "beta:4:1", "sigmoid:2:1.5", "head" or None
    sps: Optional[str]    # "tiny", "smooth", "jagged" or None
    mode: int
    temp: float = 1.0
    d: int = 0            # confidence-head input width (config 5)
    seed: int = 0         # Philox key of the method's own draws
    round: int = 0
    modes_tested: tuple = field(default_factory=tuple)

    @property
    def n_positions(self):
        return self.R * self.gamma

    @property
    def rows_capacity(self):
        return self.R * (1 + self.gamma)

    @property
    def B_max(self):
        return self.R * (1 + self.gamma)

    def elem_bytes(self):
        return 4 if self.dtype == F32 else 2


CONFIGS = {
    1: Config(1, "tiny", R=4, gamma=4, V=1024, r=16, dtype=F32, target_sd=2.0, noise="const:0.5",
              weight_sd=0.1, conf="beta:4:1", sps="tiny", mode=SCHED_EARLY_STOP,
              modes_tested=(SCHED_OFF, SCHED_EARLY_STOP, SCHED_FULL_SEARCH, SCHED_ASYNC_TOPK)),
    2: Config(2, "qwen3-8b-round", R=32, gamma=7, V=151936, r=256, dtype=BF16, target_sd=3.0,
              noise="const:1.0", weight_sd=0.02, conf=None, sps=None, mode=SCHED_OFF),
    3: Config(3, "b128-long-block", R=128, gamma=16, V=151936, r=256, dtype=BF16, target_sd=3.0,
              noise="uniform:0.3:2.0", weight_sd=0.02, conf="sigmoid:2:1.5", sps="smooth",
              mode=SCHED_EARLY_STOP),
    4: Config(4, "v4-ragged", R=256, gamma=5, V=129280, r=256, dtype=BF16, target_sd=3.0,
              noise="uniform:0.3:2.0", weight_sd=0.02, conf="sigmoid:2:1.5", sps="jagged",
              mode=SCHED_ASYNC_TOPK),
    5: Config(5, "stress", R=512, gamma=15, V=151936, r=256, dtype=BF16, target_sd=8.0,
              noise="uniform:0.1:4.0", weight_sd=0.02, conf="head", sps="jagged",
              mode=SCHED_FULL_SEARCH, d=4096),
}


def make_config(base: int = 1, **over) -> Config:
    """A variant of a configuration (edge-case shapes for the tests)."""
    c = CONFIGS[base]
    kw = {k: getattr(c, k) for k in c.__dataclass_fields__}
    kw.update(over)
    return Config(**kw)


def _rng(cfg: Config, *ids):
    return np.random.default_rng(np.random.SeedSequence([1000 + cfg.cid, cfg.V, cfg.R, *ids]))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(cfg: Config, x32: np.ndarray) -> np.ndarray:
    return to_bf16_bits(x32) if cfg.dtype == BF16 else np.ascontiguousarray(x32, np.float32)


def as_f32(cfg: Config, stored: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(stored) if cfg.dtype == BF16 else stored


# ------------------------------------------------------------------ per-request
def sigma(cfg: Config) -> np.ndarray:
    """Per-request sd of the draft noise."""
    kind, *par = cfg.noise.split(":")
    if kind == "const":
        return np.full(cfg.R, float(par[0]), dtype=np.float32)
    lo, hi = float(par[0]), float(par[1])
    return _rng(cfg, _T_SIGMA).uniform(lo, hi, cfg.R).astype(np.float32)


def _target_row32(cfg: Config, rho: int, k: int) -> np.ndarray:
    return (cfg.target_sd * _rng(cfg, _T_TARGET, rho, k).standard_normal(cfg.V, dtype=np.float32))


def target_row(cfg: Config, rho: int, k: int) -> np.ndarray:
    """Target logits of request rho at position k = 1..gamma+1."""
    return _store(cfg, _target_row32(cfg, rho, k))


def U_row(cfg: Config, rho: int, k: int, sig: Optional[np.ndarray] = None) -> np.ndarray:
    """Draft base logits U_k of request rho, k = 1..gamma: target + per-request noise."""
    s = sigma(cfg)[rho] if sig is None else sig[rho]
    noise = _rng(cfg, _T_UNOISE, rho, k).standard_normal(cfg.V, dtype=np.float32)
    return _store(cfg, _target_row32(cfg, rho, k) + np.float32(s) * noise)


def U_request(cfg: Config, rho: int, sig=None) -> np.ndarray:
    return np.stack([U_row(cfg, rho, k, sig) for k in range(1, cfg.gamma + 1)])


def target_request(cfg: Config, rho: int) -> np.ndarray:
    """[gamma+1][V] target rows of one request (positions 1..gamma+1)."""
    return np.stack([target_row(cfg, rho, k) for k in range(1, cfg.gamma + 2)])


def W1(cfg: Config) -> np.ndarray:
    """[V][r]: row x is W1[x, :]."""
    w = cfg.weight_sd * _rng(cfg, _T_W1).standard_normal((cfg.V, cfg.r), dtype=np.float32)
    return _store(cfg, w)


def W2(cfg: Config) -> np.ndarray:
    """The r x V factor stored column-major: array[v, i] is element (i, v)."""
    w = cfg.weight_sd * _rng(cfg, _T_W2).standard_normal((cfg.V, cfg.r), dtype=np.float32)
    return _store(cfg, w)


def anchors(cfg: Config) -> np.ndarray:
    return _rng(cfg, _T_X0).integers(0, cfg.V, cfg.R).astype(np.int32)


def confidences(cfg: Config, older: bool = False) -> Optional[np.ndarray]:
    """[R][gamma] conditional confidences c (older=True: the round t-2 history)."""
    if cfg.conf is None or cfg.conf == "head":
        return None
    g = _rng(cfg, _T_CPREV if older else _T_C)
    kind, *par = cfg.conf.split(":")
    if kind == "beta":
        c = g.beta(float(par[0]), float(par[1]), (cfg.R, cfg.gamma))
    else:
        mu, sd = float(par[0]), float(par[1])
        c = 1.0 / (1.0 + np.exp(-(mu + sd * g.standard_normal((cfg.R, cfg.gamma)))))
    return c.astype(np.float32)


def sps_table(cfg: Config) -> Optional[np.ndarray]:
    """Target steps per second indexed by verify batch size B = 0..B_max."""
    if cfg.sps is None:
        return None
    B = np.arange(cfg.B_max + 1, dtype=np.float64)
    if cfg.sps == "tiny":
        return 100.0 / (1.0 + B / 8.0)
    if cfg.sps == "smooth":
        return 60.0 * 1024.0 / (1024.0 + B)
    # plateaus every 64 tokens: the padded bucket size of a graph-replayed step
    return 60.0 * 1024.0 / (1024.0 + 64.0 * np.ceil(B / 64.0))


def head(cfg: Config, rho: Optional[int] = None):
    """Confidence-head inputs: h [R][gamma][d] (or one request's [gamma][d]),
    weights w [d + r] float32 and bias b."""
    d, r = cfg.d, cfg.r
    w = (1.5 / np.sqrt(d + r)) * _rng(cfg, _T_WCONF).standard_normal(d + r)
    b = 2.0
    rows = range(cfg.R) if rho is None else [rho]
    h = np.stack([_store(cfg, _rng(cfg, _T_H, p).standard_normal((cfg.gamma, d), dtype=np.float32))
                  for p in rows])
    return (h if rho is None else h[0]), w.astype(np.float32), np.float32(b)


def full_U(cfg: Config) -> np.ndarray:
    sig = sigma(cfg)
    return np.stack([U_request(cfg, rho, sig) for rho in range(cfg.R)])


def full_target(cfg: Config) -> np.ndarray:
    """[R][gamma+1][V] target rows of every request and position."""
    return np.stack([target_request(cfg, rho) for rho in range(cfg.R)])


def flatten_target(T: np.ndarray, row_offset: np.ndarray, ell: np.ndarray) -> np.ndarray:
    """The verify batch: rows row_offset[rho] + k - 1 = T[rho][k-1], k = 1..ell+1."""
    rows = [T[rho, : int(ell[rho]) + 1] for rho in range(T.shape[0])]
    return np.ascontiguousarray(np.concatenate(rows, axis=0))


def request_rows(cfg: Config, rho: int, sig: Optional[np.ndarray] = None):
    """(U_req [gamma][V], T_req [gamma+1][V]) of one request, each target row drawn once."""
    s = np.float32(sigma(cfg)[rho] if sig is None else sig[rho])
    Tq = np.empty((cfg.gamma + 1, cfg.V), dtype=np.uint16 if cfg.dtype == BF16 else np.float32)
    Uq = np.empty((cfg.gamma, cfg.V), dtype=Tq.dtype)
    for k in range(1, cfg.gamma + 2):
        t32 = _target_row32(cfg, rho, k)
        Tq[k - 1] = _store(cfg, t32)
        if k <= cfg.gamma:
            noise = _rng(cfg, _T_UNOISE, rho, k).standard_normal(cfg.V, dtype=np.float32)
            Uq[k - 1] = _store(cfg, t32 + s * noise)
    return Uq, Tq


def generate(cfg: Config, workers: int = 8, requests=None):
    """U [R][gamma][V] and T [R][gamma+1][V] (or only the listed requests), drawn in
    parallel threads; bytes are identical to the per-row functions above."""
    from concurrent.futures import ThreadPoolExecutor
    reqs = list(range(cfg.R)) if requests is None else list(requests)
    sig = sigma(cfg)
    dt = np.uint16 if cfg.dtype == BF16 else np.float32
    U = np.empty((len(reqs), cfg.gamma, cfg.V), dtype=dt)
    T = np.empty((len(reqs), cfg.gamma + 1, cfg.V), dtype=dt)

    def one(i):
        U[i], T[i] = request_rows(cfg, reqs[i], sig)

    with ThreadPoolExecutor(max(1, workers)) as ex:
        list(ex.map(one, range(len(reqs))))
    return U, T


# ------------------------------------------------------------ multi-round loop
# A prefix-dependent synthetic target for many rounds of decoding: a low-rank
# Markov model whose next-token logits given the previous token are
#     t(prev) = B + Wt1[prev, :] Wt2        (B [V], Wt1 [V][r], Wt2 r x V)
# and a draft that resembles it: the draft head's factors are the target's
# plus noise, and the draft backbone rows U_k of every round are B plus noise.
# The target forward is the environment of the method, not part of it; it is
# given here (fp32, numpy) so that the host can lay out the target rows that a
# round's verify reads.
_T_MB, _T_MW1, _T_MW2, _T_MD1, _T_MD2, _T_MU, _T_MC, _T_MX0 = range(100, 108)


@dataclass
class MarkovLoop:
    R: int = 8
    gamma: int = 4
    V: int = 64
    r: int = 16
    dtype: int = F32
    base_sd: float = 1.5       # B
    factor_sd: float = 0.6     # Wt1, Wt2 entries
    head_noise: float = 0.15   # draft head factors = target's + this * N(0, 1)
    u_noise: float = 0.6       # U_k = B + this * N(0, 1)
    conf: str = "beta:4:1"
    sps: str = "tiny"
    mode: int = SCHED_EARLY_STOP
    temp: float = 1.0
    seed: int = 7              # Philox key of the method's own draws
    key: int = 0               # seed of the synthetic inputs

    @property
    def B_max(self):
        return self.R * (1 + self.gamma)


def _mrng(m: MarkovLoop, *ids):
    return np.random.default_rng(np.random.SeedSequence([7000 + m.key, m.V, m.R, m.r, *ids]))


def _mstore(m: MarkovLoop, x32: np.ndarray) -> np.ndarray:
    return to_bf16_bits(x32) if m.dtype == BF16 else np.ascontiguousarray(x32, np.float32)


def markov_target(m: MarkovLoop):
    """(B [V], Wt1 [V][r], Wt2 stored [V][r] = r x V column-major), float32."""
    B = m.base_sd * _mrng(m, _T_MB).standard_normal(m.V, dtype=np.float32)
    W1t = m.factor_sd * _mrng(m, _T_MW1).standard_normal((m.V, m.r), dtype=np.float32)
    W2t = m.factor_sd * _mrng(m, _T_MW2).standard_normal((m.V, m.r), dtype=np.float32)
    return B, W1t, W2t


def markov_target_rows(m: MarkovLoop, target, prev: np.ndarray) -> np.ndarray:
    """Stored target rows t(prev[i]) for a list of previous tokens."""
    B, W1t, W2t = target
    prev = np.asarray(prev, dtype=np.int64)
    t32 = B[None, :] + W1t[prev] @ W2t.T
    return _mstore(m, t32.astype(np.float32))


def markov_draft_head(m: MarkovLoop, target):
    """Stored draft factors (W1 [V][r], W2 [V][r]): the target's plus noise."""
    _, W1t, W2t = target
    n1 = _mrng(m, _T_MD1).standard_normal((m.V, m.r), dtype=np.float32)
    n2 = _mrng(m, _T_MD2).standard_normal((m.V, m.r), dtype=np.float32)
    return _mstore(m, W1t + m.head_noise * n1), _mstore(m, W2t + m.head_noise * n2)


def markov_U(m: MarkovLoop, target, t: int) -> np.ndarray:
    """Draft backbone rows of round t: [R][gamma][V], B + noise."""
    B = target[0]
    n = _mrng(m, _T_MU, t).standard_normal((m.R, m.gamma, m.V), dtype=np.float32)
    return _mstore(m, B[None, None, :] + m.u_noise * n)


def markov_confidences(m: MarkovLoop, t: int) -> np.ndarray:
    """[R][gamma] conditional confidences of round t (t < 0: an earlier history)."""
    g = _mrng(m, _T_MC, t + 1000)
    kind, *par = m.conf.split(":")
    if kind == "beta":
        c = g.beta(float(par[0]), float(par[1]), (m.R, m.gamma))
    else:
        mu, sd = float(par[0]), float(par[1])
        c = 1.0 / (1.0 + np.exp(-(mu + sd * g.standard_normal((m.R, m.gamma)))))
    return c.astype(np.float32)


def markov_anchors(m: MarkovLoop) -> np.ndarray:
    return _mrng(m, _T_MX0).integers(0, m.V, m.R).astype(np.int32)


def markov_sps(m: MarkovLoop) -> np.ndarray:
    """SPS(B) tables: "tiny" falls steeply (few drafts pay), "knee" at a rate
    where admitting a candidate pays only when its survival is moderate, and
    the default is nearly flat (every draft pays)."""
    B = np.arange(m.B_max + 1, dtype=np.float64)
    if m.sps == "tiny":
        return 100.0 / (1.0 + B / 8.0)
    if m.sps == "knee":
        return 100.0 / (1.0 + B / 48.0)
    return 60.0 * 1024.0 / (1024.0 + B)


# ------------------------------------------------------------ recurrent head
_T_RGE, _T_RGH, _T_RWHH, _T_RBHH, _T_RS0, _T_RWO = range(200, 206)


def rnn_head(cfg: Config):
    """Random weights of a recurrent head of state size r (no trained weights
    exist): the token input projection G_E [V][3r] ~ N(0, 0.5^2) (stored like
    the weights), the hidden-state input projection G_h [R][gamma][3r] fp32
    ~ N(0, 0.5^2), W_hh [r][3r] (column-major storage) ~ N(0, 1/r), b_hh [3r]
    fp32 ~ N(0, 0.1^2), s0 [R][r] fp32 ~ N(0, 0.3^2), and the output factor
    W_o (stored like W2) ~ N(0, 0.15^2)."""
    r3 = 3 * cfg.r
    GE = 0.5 * _rng(cfg, _T_RGE).standard_normal((cfg.V, r3), dtype=np.float32)
    Gh = 0.5 * _rng(cfg, _T_RGH).standard_normal((cfg.R, cfg.gamma, r3), dtype=np.float32)
    Whh = _rng(cfg, _T_RWHH).standard_normal((cfg.r, r3), dtype=np.float32) / np.float32(
        np.sqrt(cfg.r))
    bhh = 0.1 * _rng(cfg, _T_RBHH).standard_normal(r3, dtype=np.float32)
    s0 = 0.3 * _rng(cfg, _T_RS0).standard_normal((cfg.R, cfg.r), dtype=np.float32)
    Wo = 0.15 * _rng(cfg, _T_RWO).standard_normal((cfg.V, cfg.r), dtype=np.float32)
    return (_store(cfg, GE), Gh.astype(np.float32), _store(cfg, Whh.astype(np.float32)),
            bhh.astype(np.float32), s0.astype(np.float32), _store(cfg, Wo))
