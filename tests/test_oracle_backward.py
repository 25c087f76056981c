"""Pins of oracle.recurrent_bwd (hand-written reverse mode of the recurrence).

* Central finite differences of the forward oracle ``recurrent``, the check the
  K3 README page's roadmap table prescribes for row L1 (gradcheck in float64 with
  eps 1e-6 and atol 1e-4): every input element on a small shape, and random
  directions over all inputs at once on the pages' naive-test shape
  (T=16, B=2, H=2, HV=4, K=V=8; key-constraints table).
* A one-token closed form with a zero initial state.
* Independence of the checkpoint interval.
* Sensitivity: an error of 1e-3 in any one gradient fails the finite-difference
  check, so the check is not vacuous.
* Gradients through the in-operator transforms (q/k L2 normalisation, beta sigmoid):
  every element against central differences of the forward oracle with the same
  transforms, on raw q, k and beta logits.
"""

import numpy as np
import pytest

from oracle import recurrent, recurrent_bwd
from synth import prefill_inputs

EPS = 1e-6
ATOL = 1e-4


def _inputs(B, T, H, HV, K, V, seed):
    inp = prefill_inputs(B, T, H, HV, K, V, "fp32", True, seed)
    x = {n: inp[n].double().numpy() for n in ("q", "k", "v", "g", "beta", "initial_state")}
    rng = np.random.default_rng(seed)
    x["do"] = rng.standard_normal((B, T, HV, V))
    x["dht"] = rng.standard_normal((B, HV, K, V))
    return x, inp["scale"]


def _loss(x, scale):
    o, s = recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["initial_state"])
    return float(np.sum(o * x["do"]) + np.sum(s * x["dht"]))


def _grads(x, scale, ckpt=64):
    dq, dk, dv, dg, db, dh0 = recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], scale,
                                            x["do"], x["initial_state"], x["dht"], ckpt=ckpt)
    return {"q": dq, "k": dk, "v": dv, "g": dg, "beta": db, "initial_state": dh0}


NAMES = ("q", "k", "v", "g", "beta", "initial_state")


def _fd_element(x, scale, name, idx):
    xp = {n: a.copy() for n, a in x.items()}
    xm = {n: a.copy() for n, a in x.items()}
    xp[name][idx] += EPS
    xm[name][idx] -= EPS
    return (_loss(xp, scale) - _loss(xm, scale)) / (2 * EPS)


def test_every_element_matches_finite_differences():
    x, scale = _inputs(1, 6, 1, 2, 4, 3, seed=11)
    gr = _grads(x, scale)
    worst = 0.0
    for name in NAMES:
        for idx in np.ndindex(x[name].shape):
            fd = _fd_element(x, scale, name, idx)
            err = abs(fd - gr[name][idx])
            worst = max(worst, err)
            assert err <= ATOL, f"d{name}{idx}: analytic {gr[name][idx]:.8f} vs fd {fd:.8f}"
    assert worst < 1e-6  # central differences in float64 are far better than atol here


@pytest.mark.parametrize("seed", [3, 4])
def test_directional_derivatives_on_the_naive_test_shape(seed):
    x, scale = _inputs(2, 16, 2, 4, 8, 8, seed=seed)
    gr = _grads(x, scale)
    rng = np.random.default_rng(100 + seed)
    for _ in range(6):
        d = {n: rng.standard_normal(x[n].shape) for n in NAMES}
        xp = dict(x)
        xm = dict(x)
        for n in NAMES:
            xp[n] = x[n] + EPS * d[n]
            xm[n] = x[n] - EPS * d[n]
        fd = (_loss(xp, scale) - _loss(xm, scale)) / (2 * EPS)
        an = sum(float(np.sum(gr[n] * d[n])) for n in NAMES)
        assert abs(fd - an) <= ATOL * max(1.0, abs(fd)), (fd, an)


def test_one_token_closed_form():
    # S_1 = k (beta v)^T from zero, o = scale (q . k) beta v
    rng = np.random.default_rng(5)
    K, V = 5, 4
    q, k = rng.standard_normal((1, 1, 1, K)), rng.standard_normal((1, 1, 1, K))
    v, g = rng.standard_normal((1, 1, 1, V)), -rng.random((1, 1, 1, K))
    beta, do = np.array([[[0.7]]]), rng.standard_normal((1, 1, 1, V))
    scale = 0.3
    dq, dk, dv, dg, db, dh0 = recurrent_bwd(q, k, v, g, beta, scale, do)
    qk, vdo = float(q.ravel() @ k.ravel()), float(v.ravel() @ do.ravel())
    np.testing.assert_allclose(dv.ravel(), scale * 0.7 * qk * do.ravel(), rtol=1e-12)
    np.testing.assert_allclose(dq.ravel(), scale * 0.7 * vdo * k.ravel(), rtol=1e-12)
    np.testing.assert_allclose(dk.ravel(), scale * 0.7 * vdo * q.ravel(), rtol=1e-12)
    np.testing.assert_allclose(db.ravel(), [scale * qk * vdo], rtol=1e-12)
    np.testing.assert_array_equal(dg, 0.0)  # the decay acts on a zero state
    # dh0: o = scale S1^T q with S1 = exp(g) S0 + k (beta (v - (exp(g) S0)^T k))^T
    e = np.exp(g.ravel())
    P = np.eye(K) - 0.7 * np.outer(k.ravel(), k.ravel())  # d S1 / d s, applied on the left
    want = np.outer(e * (P @ (scale * q.ravel())), do.ravel())
    np.testing.assert_allclose(dh0[0, 0], want, rtol=1e-12, atol=1e-14)


def test_checkpoint_interval_does_not_matter():
    x, scale = _inputs(1, 37, 1, 2, 8, 6, seed=21)
    ref = _grads(x, scale, ckpt=1)
    for ck in (5, 16, 64):
        got = _grads(x, scale, ckpt=ck)
        for n in NAMES:
            np.testing.assert_allclose(got[n], ref[n], rtol=1e-11, atol=1e-12)


def test_finite_difference_check_catches_small_errors():
    x, scale = _inputs(1, 6, 1, 2, 4, 3, seed=11)
    gr = _grads(x, scale)
    rng = np.random.default_rng(9)
    for name in NAMES:
        idx = tuple(rng.integers(0, s) for s in x[name].shape)
        fd = _fd_element(x, scale, name, idx)
        assert abs(fd - (gr[name][idx] + 1e-3)) > ATOL  # a planted 1e-3 error shows


def _loss_t(x, scale, flags):
    o, s = recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["initial_state"], **flags)
    return float(np.sum(o * x["do"]) + np.sum(s * x["dht"]))


@pytest.mark.parametrize("flags", [dict(qk_l2norm=True, beta_sigmoid=False),
                                   dict(qk_l2norm=False, beta_sigmoid=True),
                                   dict(qk_l2norm=True, beta_sigmoid=True)])
def test_transformed_gradients_match_finite_differences(flags):
    """Gradients through the in-operator transforms, element by element against central
    differences of the forward oracle applying the same transforms (raw q, k; beta logits)."""
    x, scale = _inputs(1, 5, 1, 2, 4, 3, seed=13)
    rng = np.random.default_rng(14)
    x["q"] = 3.0 * rng.standard_normal(x["q"].shape)
    x["k"] = 0.5 * rng.standard_normal(x["k"].shape)
    x["beta"] = 2.0 * rng.standard_normal(x["beta"].shape)
    dq, dk, dv, dg, db, dh0 = recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], scale,
                                            x["do"], x["initial_state"], x["dht"], **flags)
    gr = {"q": dq, "k": dk, "v": dv, "g": dg, "beta": db, "initial_state": dh0}
    for name in NAMES:
        for idx in np.ndindex(x[name].shape):
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += EPS
            xm[name][idx] -= EPS
            fd = (_loss_t(xp, scale, flags) - _loss_t(xm, scale, flags)) / (2 * EPS)
            assert abs(fd - gr[name][idx]) <= ATOL, f"d{name}{idx}: {gr[name][idx]:.8f} vs {fd:.8f}"
