"""GPU parity of dspark_sts_fit against the CPU oracle, through the C ABI.

Bar: bit-exact. The chosen temperatures and indices, the ECE and Brier of the
chosen candidates, the ECE of every candidate, and the fitted survivals all
come from integer sums or correctly rounded operations on both sides.
"""

import numpy as np
import pytest
import torch

import dspark_verify_scheduling_amd as dv
import oracle
from _gpu import DEV, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(hip):
    return hip


def _records(rng, N, gamma, t_true):
    """Confidence logits and greedy prefix labels whose acceptance follows
    sigmoid(z / t_true) position by position (a label needs its predecessors)."""
    z = (rng.normal(1.0, 2.0, (N, gamma)) - 0.3 * np.arange(gamma)).astype(np.float32)
    p = 1.0 / (1.0 + np.exp(-z.astype(np.float64) / t_true[None, :]))
    acc = rng.random((N, gamma)) < p
    return z, np.cumprod(acc, axis=1).astype(np.uint8)


def _fit_both(z, y, grid, nbins, tag, workspace=None):
    say(f"sts_fit {tag} N={z.shape[0]} gamma={z.shape[1]} n_t={len(grid)} bins={nbins}")
    got = dv.dspark_sts_fit(up(z), up(y), grid, nbins, workspace=workspace)
    torch.cuda.synchronize()
    ref = oracle.sts_fit(z, y, np.asarray(grid, np.float32), nbins)
    g = {k: getattr(got, k).cpu().numpy() for k in ("temps", "t_index", "ece", "brier",
                                                    "ece_grid", "survival")}
    for k in ("temps", "t_index", "ece", "brier", "survival"):
        a, b = g[k], ref[k]
        same = (a == b) | (np.isnan(a) & np.isnan(b)) if a.dtype.kind == "f" else a == b
        assert np.all(same), (k, a if a.size < 20 else np.argwhere(~same)[:5], b if b.size < 20 else "")
    N = z.shape[0]
    ref_grid = ref["ece_fx"] / (N * 2.0 ** 40) if N else np.zeros_like(ref["ece_fx"], float)
    assert np.array_equal(g["ece_grid"], ref_grid), "ece_grid"
    return g, ref


GRID = np.exp(np.linspace(np.log(0.4), np.log(3.0), 24)).astype(np.float32)


@pytest.mark.parametrize("N,gamma,nbins", [(5000, 4, 15), (4096, 8, 10), (9000, 3, 64), (1, 2, 1)])
def test_sts_fit_parity(N, gamma, nbins):
    rng = np.random.default_rng(N + gamma)
    t_true = np.linspace(0.8, 1.8, gamma)
    z, y = _records(rng, N, gamma, t_true)
    g, ref = _fit_both(z, y, GRID, nbins, f"N={N}")
    say(f"fitted {g['temps'].round(3).tolist()} for {t_true.round(3).tolist()}")


def test_sts_fit_recovers_the_generating_temperatures():
    rng = np.random.default_rng(7)
    t_true = np.array([0.7, 1.0, 1.5, 2.2])
    z, y = _records(rng, 60000, 4, t_true)
    g, _ = _fit_both(z, y, GRID, 15, "large")
    # statistical, loose: every fitted temperature is within 20% of the truth
    assert np.all(np.abs(g["temps"] / t_true - 1) < 0.2), g["temps"]


def test_sts_fit_edge_cases():
    rng = np.random.default_rng(3)
    z, y = _records(rng, 700, 5, np.ones(5))
    z[3, 1] = np.inf
    z[4, 2] = -np.inf
    z[5, 0] = np.nan  # a NaN survival is binned and summed as 0
    _fit_both(z, y, GRID, 15, "inf and nan logits")
    _fit_both(z, y, GRID[:1], 15, "one candidate")
    grid128 = np.exp(np.linspace(np.log(0.2), np.log(5.0), 128)).astype(np.float32)
    _fit_both(z, y, grid128, 64, "largest grid and bins")
    _fit_both(np.zeros((0, 3), np.float32), np.zeros((0, 3), np.uint8), GRID, 15, "no records")


@pytest.mark.parametrize("n_t", [2, 3, 4, 5, 7, 9, 63])
def test_sts_fit_grid_sizes(n_t):
    """Candidate counts around the four threads per record and the two
    candidates a thread takes per step: fewer candidates than threads, an odd
    count per thread, and counts that leave a thread's last step half used."""
    rng = np.random.default_rng(100 + n_t)
    z, y = _records(rng, 2000, 3, np.array([0.9, 1.3, 1.7]))
    grid = np.exp(np.linspace(np.log(0.5), np.log(2.5), n_t)).astype(np.float32)
    _fit_both(z, y, grid, 12, f"n_t={n_t}")


def test_sts_fit_reuses_a_dirty_workspace():
    """The workspace's contents on entry do not matter: a garbage-filled
    workspace, then a second, smaller fit on the same one (its histogram
    buffers hold the first fit's sums), both equal the oracle."""
    rng = np.random.default_rng(21)
    z1, y1 = _records(rng, 3000, 6, np.linspace(0.8, 1.6, 6))
    z2, y2 = _records(rng, 700, 5, np.linspace(1.2, 0.9, 5))
    size = max(dv.dspark_sts_workspace_size(3000, 6, len(GRID), 15),
               dv.dspark_sts_workspace_size(700, 5, len(GRID), 15))
    ws = torch.full((size,), 0x5A, dtype=torch.uint8, device=DEV)
    _fit_both(z1, y1, GRID, 15, "garbage workspace", workspace=ws)
    _fit_both(z2, y2, GRID, 15, "reused workspace", workspace=ws)
