"""Pins for the oracle's optional input transforms (q/k L2 normalisation, beta sigmoid).

Each pin ties the transform to a property or closed form, not to a restatement of its
formula: normalisation makes the operator blind to per-token rescaling of q and k and
leaves unit vectors alone; the sigmoid maps logit 0 to beta = 1/2 and a very negative
logit to beta = 0, whose output is the pure decayed readout."""

import numpy as np
import pytest

from oracle import l2_normalize, recurrent, sigmoid
from synth import prefill_inputs


def _inp(seed, **kw):
    shape = dict(B=2, T=24, H=2, HV=4, K=8, V=6)
    shape.update(kw)
    return prefill_inputs(**shape, dtype="fp32", init_state=True, seed=seed)


def _np(x):
    return x.double().numpy()


def test_l2_normalize_unit_norm_and_direction():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 16)) * rng.uniform(0.5, 20.0, (5, 3, 1))
    y = l2_normalize(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-8)
    cos = np.sum(x * y, axis=-1) / (np.linalg.norm(x, axis=-1) * np.linalg.norm(y, axis=-1))
    np.testing.assert_allclose(cos, 1.0, atol=1e-12)
    assert np.all(l2_normalize(np.zeros((2, 8))) == 0.0)  # a zero vector stays zero


def test_qk_l2norm_is_blind_to_per_token_rescaling():
    inp = _inp(1)
    rng = np.random.default_rng(1)
    q, k = _np(inp["q"]), _np(inp["k"])
    # with EPS in the norm, a rescale by c >= 1/2 of a unit vector moves the normalised
    # vector by at most EPS / (2 c^2) = 2e-6 relatively, far below a missing normalisation
    cq = rng.uniform(0.5, 30.0, q.shape[:-1] + (1,))
    ck = rng.uniform(0.5, 30.0, k.shape[:-1] + (1,))
    args = dict(v=inp["v"], g=inp["g"], beta=inp["beta"], scale=inp["scale"],
                initial_state=inp["initial_state"], qk_l2norm=True)
    o1, s1 = recurrent(q=q, k=k, **args)
    o2, s2 = recurrent(q=q * cq, k=k * ck, **args)
    np.testing.assert_allclose(o2, o1, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(s2, s1, rtol=1e-5, atol=1e-7)


def test_qk_l2norm_leaves_unit_vectors_alone():
    inp = _inp(2)  # synth's q, k are unit vectors (float32)
    o0, s0 = recurrent(**inp)
    o1, s1 = recurrent(**inp, qk_l2norm=True)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-5)
    np.testing.assert_allclose(s1, s0, rtol=0, atol=1e-5)


def test_qk_l2norm_changes_non_unit_inputs():
    inp = _inp(3)
    inp["q"], inp["k"] = inp["q"] * 3.0, inp["k"] * 0.5
    o0, _ = recurrent(**inp)
    o1, _ = recurrent(**inp, qk_l2norm=True)
    assert np.max(np.abs(o1 - o0)) > 1e-2


def test_sigmoid_values():
    np.testing.assert_allclose(sigmoid(np.array([0.0])), [0.5])
    x = np.array([-800.0, -30.0, -1.0, 1.0, 30.0, 800.0])
    y = sigmoid(x)
    assert np.all(np.isfinite(y)) and np.all((y >= 0) & (y <= 1))
    np.testing.assert_allclose(y + sigmoid(-x), 1.0, atol=1e-15)  # symmetry
    np.testing.assert_allclose(y[2], 1.0 / (1.0 + np.e), rtol=1e-15)


def test_beta_sigmoid_logit_zero_is_one_half():
    inp = _inp(4)
    logits = inp["beta"] * 0.0
    o1, s1 = recurrent(**{**inp, "beta": logits}, beta_sigmoid=True)
    o0, s0 = recurrent(**{**inp, "beta": logits + 0.5})
    np.testing.assert_allclose(o1, o0, atol=1e-12)
    np.testing.assert_allclose(s1, s0, atol=1e-12)


@pytest.mark.parametrize("seed", [5, 6])
def test_beta_sigmoid_very_negative_logit_is_pure_decayed_readout(seed):
    inp = _inp(seed)
    o1, s1 = recurrent(**{**inp, "beta": inp["beta"] * 0.0 - 200.0}, beta_sigmoid=True)
    # beta = 0: no writes; the state only decays, o_t = (prod_{r<=t} exp(g_r) S0)^T (scale q_t)
    q = np.repeat(_np(inp["q"]), 2, axis=2) * inp["scale"]
    g, s = _np(inp["g"]), _np(inp["initial_state"])
    for t in range(q.shape[1]):
        s = np.exp(g[:, t])[..., None] * s
        np.testing.assert_allclose(o1[:, t], np.einsum("bhkv,bhk->bhv", s, q[:, t]), atol=1e-12)
    np.testing.assert_allclose(s1, s, atol=1e-12)
