"""Seeded input generator for the five verify-path workloads.

Every array is drawn from numpy's PCG64 under a fixed seed
(``1000 * (cfg + 1)`` unless given), so a workload is bit-for-bit reproducible
on any host. Logit rows are generated in independent blocks, each from its own
child ``SeedSequence``, so they can be drawn on several threads and still give
the same bits.

Planted structure (never computed from the data):

* Each target row ``[r, j]`` is N(0, sigma) clipped to ``[-5 sigma, 5 sigma]``,
  then one id ``top[r, j]`` receives the value ``5 sigma + 1``, the row's
  strict maximum. In configs 1-4 a row gets, with probability 0.1, a second
  copy of that value at another uniformly drawn id, an exact tie that the
  lowest-index rule resolves.
* Draft token ``d[r, k]`` (position k, checked against target row k-1)
  equals ``top[r, k-1]`` when a standard logistic draw falls below the raw
  confidence logit ``z[r, k]`` (a Bernoulli with success probability
  sigmoid(z), drawn without evaluating a sigmoid). Otherwise it is a uniform
  id different from ``top[r, k-1]``.
* Config 4 draws draft logits ``q[r, k] = clip(p[r, k-1] + N(0, sigma_r))``
  and plants the draft's own maximum (value ``5 sigma + 5``) at ``d[r, k]``.
  ``d[r, k] = top[r, k-1]`` with probability ``1 - sigma_r / 4``.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

_ROW_BLOCK = 32  # rows per independently seeded logit block


@dataclass(frozen=True)
class ConfigSpec:
    name: str
    B: int
    gamma: int
    V: int
    dtype: str  # "f32" or "bf16": storage type of the logits
    sigma: float  # standard deviation of the target logits
    min_len: int
    max_len: int
    eps: float
    tiers: tuple
    budget: tuple  # (budget_lo, budget_hi) over the extra verify rows b
    kind: str  # "conf_logits" (z + STS temperatures) or "survival" (from TV)


CONFIGS = {
    0: ConfigSpec("tiny", 2, 4, 1024, "f32", 1.0, 1, 5, 0.0, (2, 4, 8, 10), (0, 8), "conf_logits"),
    1: ConfigSpec("b8_g8_v32000_f32", 8, 8, 32000, "f32", 2.0, 1, 9, 1e-3,
                  (8, 16, 32, 64, 72), (0, 64), "conf_logits"),
    2: ConfigSpec("b64_g8_v151936_bf16", 64, 8, 151936, "bf16", 3.0, 1, 9, 1e-3,
                  (64, 128, 256, 384, 576), (0, 512), "conf_logits"),
    3: ConfigSpec("b256_g8_v129280_bf16", 256, 8, 129280, "bf16", 3.0, 1, 9, 1e-3,
                  (256, 512, 1024, 2048, 2304), (0, 2048), "conf_logits"),
    4: ConfigSpec("b256_g16_v129280_bf16_tv", 256, 16, 129280, "bf16", 3.0, 1, 17, 1e-4,
                  (256, 512, 1024, 2048, 4096, 4352), (0, 4096), "survival"),
}


@dataclass
class Workload:
    cfg: int
    spec: ConfigSpec
    seed: int
    B: int
    gamma: int
    V: int
    dtype: str
    conf: Optional[np.ndarray]  # [B, gamma] f32 confidence logits z (None for config 4)
    temps: np.ndarray  # [gamma] f32 STS temperatures
    bias: np.float32
    alpha: np.ndarray  # [B + 1] f32, alpha[bs] in ms
    theta: np.ndarray  # [B * (gamma + 1) + 1] f32, theta[M] in ms
    tiers: np.ndarray  # int32, ascending
    b_lo: int
    b_hi: int
    min_len: int
    max_len: int
    eps: float
    anchors: np.ndarray  # [B] int32, the root row's token per request
    drafts: np.ndarray  # [B, gamma] int32
    prefix_lens: np.ndarray  # [B] int32
    planted_top: np.ndarray  # [B, gamma + 1] int32, id holding the planted row maximum
    target: Optional[np.ndarray]  # [B, gamma + 1, V]: uint16 bf16 bits or float32
    draft_logits: Optional[np.ndarray]  # [B, gamma, V] (config 4 only)

    @property
    def rows_strided(self) -> int:
        return self.B * (self.gamma + 1)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits.

    Inputs here are always finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _other_id(rng: np.random.Generator, avoid: np.ndarray, V: int) -> np.ndarray:
    """Uniform id in [0, V) different from ``avoid`` (elementwise)."""
    u = rng.integers(0, V - 1, size=avoid.shape, dtype=np.int64)
    return (u + (u >= avoid)).astype(np.int32)


def _piecewise_table(knots_m, knot_vals, n):
    """Dense table over M = 0..n-1, linear between knots, extended linearly."""
    m = np.arange(n, dtype=np.float64)
    km = np.asarray(knots_m, dtype=np.float64)
    kv = np.asarray(knot_vals, dtype=np.float64)
    out = np.interp(m, km, kv)
    lo_slope = (kv[1] - kv[0]) / (km[1] - km[0])
    hi_slope = (kv[-1] - kv[-2]) / (km[-1] - km[-2])
    out = np.where(m < km[0], kv[0] + (m - km[0]) * lo_slope, out)
    out = np.where(m > km[-1], kv[-1] + (m - km[-1]) * hi_slope, out)
    return out


def _cost_tables(cfg: int, spec: ConfigSpec, rng: np.random.Generator):
    B, g = spec.B, spec.gamma
    n_theta = B * (g + 1) + 1
    bs = np.arange(B + 1, dtype=np.float64)
    M = np.arange(n_theta, dtype=np.float64)
    bias = 0.5
    if cfg == 0:
        alpha = 0.01 * bs
        theta = 0.02 * M
    elif cfg == 1:
        alpha = 0.01 * bs
        knots = [8, 16, 32, 64]
        slopes = np.sort(rng.uniform(0.01, 0.03, size=len(knots) - 1))
        vals = [0.08]
        for i, s in enumerate(slopes):
            vals.append(vals[-1] + s * (knots[i + 1] - knots[i]))
        theta = _piecewise_table(knots, vals, n_theta)
    elif cfg == 2:
        alpha = 0.02 * bs
        tiers = np.asarray(spec.tiers)
        idx = np.searchsorted(tiers, M, side="left")  # smallest tier >= M
        idx = np.minimum(idx, len(tiers) - 1)
        theta = 0.004 * M + 0.5 * idx
    else:  # configs 3 and 4: convex piecewise-linear with knots at the tiers
        alpha = 0.005 * bs
        knots = list(spec.tiers)
        slopes = np.sort(rng.uniform(5e-4, 4e-3, size=len(knots) - 1))
        vals = [0.5]
        for i, s in enumerate(slopes):
            vals.append(vals[-1] + s * (knots[i + 1] - knots[i]))
        theta = _piecewise_table(knots, vals, n_theta)
    return np.float32(bias), alpha.astype(np.float32), theta.astype(np.float32)


def _fill_blocks(n_rows: int, work, n_threads: Optional[int] = None):
    n_blocks = (n_rows + _ROW_BLOCK - 1) // _ROW_BLOCK
    n_threads = n_threads or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n_threads) as ex:
        list(ex.map(work, range(n_blocks)))


def _target_logits(spec, ss, top, dup):
    """Strided target logits [B, gamma+1, V]; the planted value sits at ``top``."""
    B, g, V = spec.B, spec.gamma, spec.V
    n_rows = B * (g + 1)
    cap = np.float32(5.0 * spec.sigma)
    peak = np.float32(5.0 * spec.sigma + 1.0)
    top_f = top.reshape(-1)
    dup_f = dup.reshape(-1)
    out = np.empty((n_rows, V), dtype=np.uint16 if spec.dtype == "bf16" else np.float32)
    children = ss.spawn((n_rows + _ROW_BLOCK - 1) // _ROW_BLOCK)

    def work(i):
        r0, r1 = i * _ROW_BLOCK, min(n_rows, (i + 1) * _ROW_BLOCK)
        rng = np.random.Generator(np.random.PCG64(children[i]))
        x = rng.standard_normal((r1 - r0, V), dtype=np.float32)
        x *= np.float32(spec.sigma)
        np.clip(x, -cap, cap, out=x)
        rows = np.arange(r1 - r0)
        x[rows, top_f[r0:r1]] = peak
        has = dup_f[r0:r1] >= 0
        x[rows[has], dup_f[r0:r1][has]] = peak
        out[r0:r1] = f32_to_bf16_bits(x) if spec.dtype == "bf16" else x

    _fill_blocks(n_rows, work)
    return out.reshape(B, g + 1, V)


def _draft_logits(spec, ss, target, d_ids, sig_r):
    """Config 4 draft logits q[r, k] = clip(p[r, k-1] + N(0, sigma_r)), peak at d."""
    B, g, V = spec.B, spec.gamma, spec.V
    n_rows = B * g
    bf16 = spec.dtype == "bf16"
    cap = np.float32(5.0 * spec.sigma + 3.0)
    peak = np.float32(5.0 * spec.sigma + 5.0)
    out = np.empty((n_rows, V), dtype=np.uint16 if bf16 else np.float32)
    children = ss.spawn((n_rows + _ROW_BLOCK - 1) // _ROW_BLOCK)
    d_f = d_ids.reshape(-1)

    def work(i):
        q0, q1 = i * _ROW_BLOCK, min(n_rows, (i + 1) * _ROW_BLOCK)
        rng = np.random.Generator(np.random.PCG64(children[i]))
        qi = np.arange(q0, q1)
        r, k0 = qi // g, qi % g  # k0 = k - 1: paired target row
        p = bf16_bits_to_f32(target[r, k0]) if bf16 else target[r, k0]
        noise = rng.standard_normal((q1 - q0, V), dtype=np.float32)
        noise *= sig_r[r].astype(np.float32)[:, None]
        x = p + noise
        np.clip(x, -cap, cap, out=x)
        x[np.arange(q1 - q0), d_f[q0:q1]] = peak
        out[q0:q1] = f32_to_bf16_bits(x) if bf16 else x

    _fill_blocks(n_rows, work)
    return out.reshape(B, g, V)


def make(cfg: int, seed: Optional[int] = None, *, logits: bool = True,
         conf_shift: float = 0.0) -> Workload:
    """Draw workload ``cfg`` (0-4). ``logits=False`` skips the big logit arrays
    (every other array is unchanged by that choice). ``conf_shift`` moves the
    mean of the confidence logits of configs 1-3 (the planted draft matches
    follow the shifted logits)."""
    spec = CONFIGS[cfg]
    seed = 1000 * (cfg + 1) if seed is None else int(seed)
    ss_meta, ss_target, ss_draft = np.random.SeedSequence(seed).spawn(3)
    rng = np.random.Generator(np.random.PCG64(ss_meta))
    B, g, V = spec.B, spec.gamma, spec.V
    k = np.arange(1, g + 1, dtype=np.float64)

    # confidence logits z[r, k] and STS temperatures T[k]
    conf = None
    if cfg == 0:
        c = np.array([[0.9, 0.8, 0.7, 0.6], [0.6, 0.5, 0.4, 0.3]], dtype=np.float64)
        conf = np.log(c / (1.0 - c)).astype(np.float32)
        temps = np.ones(g, dtype=np.float32)
    elif cfg == 1:
        conf = (rng.normal(1.5 + conf_shift, 1.0, size=(B, g)) - 0.25 * k).astype(np.float32)
        temps = rng.uniform(0.8, 1.5, size=g).astype(np.float32)
    elif cfg == 2:
        mu = rng.choice(np.array([2.5, 1.0, -0.5]), size=B)
        conf = (rng.normal(conf_shift, 1.0, size=(B, g)) + mu[:, None] - 0.25 * k).astype(np.float32)
        temps = rng.uniform(0.8, 1.5, size=g).astype(np.float32)
    elif cfg == 3:
        conf = (rng.normal(1.2 + conf_shift, 1.2, size=(B, g)) - 0.3 * k).astype(np.float32)
        temps = rng.uniform(0.7, 2.0, size=g).astype(np.float32)
    else:
        temps = np.ones(g, dtype=np.float32)

    bias, alpha, theta = _cost_tables(cfg, spec, rng)

    # planted maxima and optional exact ties
    top = rng.integers(0, V, size=(B, g + 1), dtype=np.int64).astype(np.int32)
    dup = np.full((B, g + 1), -1, dtype=np.int32)
    if cfg != 0:
        tie = rng.random(size=(B, g + 1)) < 0.1
        cand = _other_id(rng, top, V)
        dup = np.where(tie, cand, -1).astype(np.int32)

    # draft tokens: position k (0-based column k-1) is checked against row k-1
    sig_r = None
    if cfg == 0:
        match = np.array([[1, 1, 1, 0], [1, 0, 0, 0]], dtype=bool)
    elif cfg == 4:
        sig_r = rng.uniform(0.2, 2.0, size=B)
        match = rng.random(size=(B, g)) < (1.0 - sig_r / 4.0)[:, None]
    else:
        match = rng.logistic(0.0, 1.0, size=(B, g)) < conf
    wrong = _other_id(rng, top[:, :g], V)
    drafts = np.where(match, top[:, :g], wrong).astype(np.int32)

    anchors = rng.integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    prefix_lens = rng.integers(16, 4097, size=B, dtype=np.int64).astype(np.int32)

    target = draft_l = None
    if logits:
        target = _target_logits(spec, ss_target, top, dup)
        if cfg == 4:
            draft_l = _draft_logits(spec, ss_draft, target, drafts, sig_r)

    return Workload(
        cfg=cfg, spec=spec, seed=seed, B=B, gamma=g, V=V, dtype=spec.dtype,
        conf=conf, temps=temps, bias=bias, alpha=alpha, theta=theta,
        tiers=np.asarray(spec.tiers, dtype=np.int32),
        b_lo=spec.budget[0], b_hi=spec.budget[1],
        min_len=spec.min_len, max_len=spec.max_len, eps=spec.eps,
        anchors=anchors, drafts=drafts, prefix_lens=prefix_lens,
        planted_top=top, target=target, draft_logits=draft_l,
    )


@dataclass
class SamplingExtras:
    draft_logits: np.ndarray  # [B, gamma, V]: uint16 bf16 bits or float32
    temps: np.ndarray  # [B] f32 per-request sampling temperature (0 = greedy)
    rand_accept: np.ndarray  # [B, gamma] uint32 random words
    rand_sample: np.ndarray  # [B, gamma + 1] uint32 random words


def sampling_extras(w: Workload, seed: Optional[int] = None, greedy_frac: float = 0.0,
                    t_range=(0.6, 1.4)) -> SamplingExtras:
    """Inputs of the sampling accept for workload ``w``: draft logits (config
    4's own, or drawn with config 4's recipe, q[r, k] = clip(p[r, k-1] +
    N(0, sigma_r)) with the draft's maximum planted at d[r, k]), a
    temperature per request (a ``greedy_frac`` share of them 0) and the
    random words."""
    seed = 7919 * (w.cfg + 1) if seed is None else int(seed)
    ss_meta, ss_draft = np.random.SeedSequence(seed).spawn(2)
    rng = np.random.Generator(np.random.PCG64(ss_meta))
    B, g = w.B, w.gamma
    if w.draft_logits is not None:
        dl = w.draft_logits
    else:
        sig_r = rng.uniform(0.2, 2.0, size=B)
        dl = _draft_logits(w.spec, ss_draft, w.target, w.drafts, sig_r)
    temps = rng.uniform(t_range[0], t_range[1], size=B).astype(np.float32)
    temps[rng.random(B) < greedy_frac] = 0.0
    ra = rng.integers(0, 2**32, size=(B, g), dtype=np.uint64).astype(np.uint32)
    rs = rng.integers(0, 2**32, size=(B, g + 1), dtype=np.uint64).astype(np.uint32)
    return SamplingExtras(dl, temps, ra, rs)
