"""Pins for the oracle's decay gate (oracle/gate.py; K3 README, roadmap row L5 and the
key-constraints table's exp-underflow row).

The forward is tied to library routines and closed forms, not to a restatement of its
formula: at A_log = 0 the decay factor exp(g) is the logistic function of -z (scipy's
expit) and g is torch's softplus negated; the workloads' recipe max(-5, -softplus(x)) is the
safe gate at A_log = 0, dt_bias = 0; exp(A_log) acts as a power on the decay factor; dt_bias
is a shift of the input per (head, channel); hand-worked values. The backward is tied to
central finite differences of the forward, element by element, and the check is shown to
catch plausible mistakes planted into a copy of it."""

import math

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle.gate import gate, gate_bwd


def _inputs(seed, lead=(2, 5), HV=3, K=4, spread=2.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(lead + (HV, K)) * spread
    A_log = rng.uniform(-1.0, 1.0, HV)
    dt_bias = rng.uniform(-1.0, 1.0, (HV, K))
    return x, A_log, dt_bias


def test_unit_rate_gate_is_the_logistic_decay():
    x, _, _ = _inputs(0)
    g = gate(x, np.zeros(x.shape[-2]))
    np.testing.assert_allclose(np.exp(g), expit(-x), rtol=1e-13, atol=0)
    ref = -torch.nn.functional.softplus(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(g, ref, rtol=1e-13, atol=1e-15)


def test_safe_gate_is_the_workload_recipe():
    # the workloads draw g = max(-5, -softplus(N(0, 1))); with a wide spread many
    # entries sit on the bound
    x, _, _ = _inputs(1, lead=(8, 5), spread=5.0)
    g = gate(x, np.zeros(x.shape[-2]), None, lower_bound=-5.0)
    t = torch.from_numpy(x)
    ref = torch.clamp(-torch.nn.functional.softplus(t), min=-5.0).numpy()
    np.testing.assert_allclose(g, ref, rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(g == -5.0, ref == -5.0)
    assert np.mean(g == -5.0) > 0.05


def test_rate_is_a_power_on_the_decay_factor():
    x, _, _ = _inputs(2)
    HV = x.shape[-2]
    a = np.array([0.5, 2.0, 3.7])[:HV]
    g = gate(x, np.log(a))
    np.testing.assert_allclose(np.exp(g), expit(-x) ** a[:, None], rtol=1e-12)


def test_bias_is_a_per_head_channel_shift():
    x, A_log, dt_bias = _inputs(3)  # HV=3 != K=4: a transposed bias fails
    np.testing.assert_allclose(gate(x, A_log, dt_bias), gate(x + dt_bias, A_log), rtol=1e-14)
    assert not np.allclose(gate(x, A_log, dt_bias), gate(x + dt_bias.T.reshape(3, 4), A_log))


def test_hand_worked_values():
    # softplus(0) = ln 2; softplus(ln(e - 1)) = 1; rate exp(ln 2) = 2 doubles g
    assert gate(np.zeros((1, 1)), np.zeros(1))[0, 0] == pytest.approx(-math.log(2.0), abs=1e-15)
    x1 = np.full((1, 1), math.log(math.e - 1.0))
    assert gate(x1, np.zeros(1))[0, 0] == pytest.approx(-1.0, abs=1e-15)
    assert gate(np.zeros((1, 1)), np.log([2.0]))[0, 0] == pytest.approx(-math.log(4.0), abs=1e-15)
    # large inputs: softplus(z) -> z; very negative: softplus(z) -> e^z, no overflow
    assert gate(np.full((1, 1), 800.0), np.zeros(1))[0, 0] == pytest.approx(-800.0, rel=1e-15)
    assert gate(np.full((1, 1), -800.0), np.zeros(1))[0, 0] == 0.0


def test_range_and_monotonicity():
    x, A_log, dt_bias = _inputs(4, lead=(400,), spread=6.0)
    g = gate(x, A_log, dt_bias)
    assert np.all(g < 0.0)
    gs = gate(x, A_log, dt_bias, lower_bound=-5.0)
    assert np.all(gs >= -5.0) and np.all(gs <= 0.0)
    np.testing.assert_array_equal(gs[g >= -5.0], g[g >= -5.0])
    # a larger gate input forgets more
    assert np.all(gate(x + 0.25, A_log, dt_bias) < g)


def _fd_errors(bwd, x, A_log, dt_bias, dg, lb, eps=1e-6):
    """Largest |analytic - central difference| over every element of x, A_log, dt_bias."""
    dx, dA, db = bwd(x, A_log, dt_bias, dg, lb)
    f = lambda x_, a_, b_: np.sum(gate(x_, a_, b_, lb) * dg)
    worst = 0.0
    for arr, grad, pos in ((x, dx, 0), (A_log, dA, 1), (dt_bias, db, 2)):
        for idx in np.ndindex(arr.shape):
            args = [x.copy(), A_log.copy(), dt_bias.copy()]
            args[pos][idx] += eps
            fp = f(*args)
            args[pos][idx] -= 2 * eps
            fm = f(*args)
            worst = max(worst, abs((fp - fm) / (2 * eps) - grad[idx]))
    return worst


def _away_from_bound(x, A_log, dt_bias, lb, margin=1e-3):
    g = gate(x, A_log, dt_bias)
    return np.abs(g - lb) > margin


@pytest.mark.parametrize("lb", [None, -1.5])
def test_backward_matches_finite_differences(lb):
    x, A_log, dt_bias = _inputs(5, lead=(2, 3), spread=2.5)
    if lb is not None:
        ok = _away_from_bound(x, A_log, dt_bias, lb)
        x = np.where(ok, x, x + 0.1)
        assert np.all(_away_from_bound(x, A_log, dt_bias, lb))
        assert 0.1 < np.mean(gate(x, A_log, dt_bias) < lb) < 0.9  # both sides exercised
    dg = np.random.default_rng(6).standard_normal(x.shape)
    assert _fd_errors(gate_bwd, x, A_log, dt_bias, dg, lb) < 1e-7


def test_finite_differences_catch_planted_mistakes():
    x, A_log, dt_bias = _inputs(7, lead=(2, 3), spread=2.5)
    lb = -1.5
    x = np.where(_away_from_bound(x, A_log, dt_bias, lb), x, x + 0.1)
    dg = np.random.default_rng(8).standard_normal(x.shape)

    def no_chain_on_rate(x_, a_, b_, dg_, lb_):   # d/dA_log taken as -softplus, not -a softplus
        dx, dA, db = gate_bwd(x_, a_, b_, dg_, lb_)
        return dx, dA / np.exp(a_), db

    def clamp_passes_everywhere(x_, a_, b_, dg_, lb_):
        return gate_bwd(x_, a_, b_, dg_, None)

    def bias_sums_one_batch(x_, a_, b_, dg_, lb_):  # reduction over too few tokens
        dx, dA, db = gate_bwd(x_, a_, b_, dg_, lb_)
        return dx, dA, dx[0].sum(axis=0)

    assert _fd_errors(gate_bwd, x, A_log, dt_bias, dg, lb) < 1e-7
    for wrong in (no_chain_on_rate, clamp_passes_everywhere, bias_sums_one_batch):
        assert _fd_errors(wrong, x, A_log, dt_bias, dg, lb) > 1e-2, wrong.__name__
