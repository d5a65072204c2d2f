"""Pins for the soft accept-rate oracle ``a = 1 - TV(softmax(q), softmax(p))``.

The pages print no TV values, so the pins are mathematical:

* identical rows give a = 1; the rejection-sampling identity
  ``sum_x min(p, q) = 1 - TV`` holds (the oracle asserts it internally);
* softmax is invariant under adding a constant to a row;
* closed form for a uniform q against a one-hot-ish p (one logit L, the
  rest 0): ``a = 1/V + (V-1)/(e^L + V - 1)``;
* closed form for two disjoint spikes;
* the cumulative product S equals the running product of a.
"""

import math

import numpy as np

import oracle
from oracle.tv import tv_pair
from workloads import f32_to_bf16_bits


def test_identical_rows_give_one():
    rng = np.random.default_rng(0)
    q = rng.normal(0, 3, size=1000).astype(np.float32)
    assert tv_pair(q, q.copy()) == 1.0


def test_translation_invariance():
    rng = np.random.default_rng(1)
    # values on a 2**-10 grid so that the shifts below are exact in float32
    q = (np.round(rng.normal(0, 2, size=500) * 1024) / 1024).astype(np.float32)
    p = (np.round(rng.normal(0, 2, size=500) * 1024) / 1024).astype(np.float32)
    a0 = tv_pair(q, p)
    a1 = tv_pair(q + np.float32(4.0), p - np.float32(2.0))
    a2 = tv_pair(q + np.float32(800.0), p + np.float32(900.0))  # exp would overflow unshifted
    assert abs(a0 - a1) < 1e-12 and abs(a0 - a2) < 1e-12


def test_uniform_vs_spike_closed_form():
    V, L = 1000, 6.0
    q = np.zeros(V, np.float32)
    p = np.zeros(V, np.float32)
    p[17] = L
    expect = 1.0 / V + (V - 1) / (math.exp(L) + V - 1)
    assert abs(tv_pair(q, p) - expect) < 1e-13


def test_disjoint_spikes_closed_form():
    V, L = 64, 20.0
    q = np.zeros(V, np.float32)
    p = np.zeros(V, np.float32)
    q[3], p[40] = L, L
    Z = math.exp(L) + V - 1
    # both distributions put e^L/Z on their own spike and 1/Z elsewhere
    expect = (V - 2) / Z + 2.0 / Z
    assert abs(tv_pair(q, p) - expect) < 1e-13


def test_bf16_rows_and_cumprod():
    rng = np.random.default_rng(2)
    B, gamma, V = 2, 3, 257
    p = f32_to_bf16_bits(rng.normal(0, 3, size=(B, gamma + 1, V)).astype(np.float32))
    q = f32_to_bf16_bits(rng.normal(0, 3, size=(B, gamma, V)).astype(np.float32))
    a, S = oracle.tv_accept(B, gamma, q, p, "bf16")
    assert np.all((a >= 0) & (a <= 1))
    for r in range(B):
        assert np.allclose(S[r], np.cumprod(a[r]), rtol=0, atol=1e-15)
    # q paired with target row k-1: make q[r, 1] equal to p[r, 1] -> a[r, 1] = 1
    q2 = q.copy()
    q2[1, 1] = p[1, 1]
    a2, _ = oracle.tv_accept(B, gamma, q2, p, "bf16")
    assert a2[1, 1] == 1.0
