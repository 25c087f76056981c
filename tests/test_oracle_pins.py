"""Pins for the CPU oracle (runs without a GPU).

Each test ties the oracle to something other than itself: a hand-worked
example, brute-force composition of affine maps, a separately written chunked
form, a library solver, closed forms and invariants of the recurrence. The
last test plants plausible mistakes into copies of the recurrence step and
checks that these pins catch every one of them.
"""

import os

import numpy as np
import pytest
import torch

from oracle import brute, chunked, decode_step, forward_substitution_inverse, recurrent
from synth import prefill_inputs

TOL = dict(rtol=1e-10, atol=1e-12)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.txt")


def _read_golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, rhs = line.split("=", 1)
            vals[name.strip()] = np.array([float(x) for x in rhs.split(",")])
    return vals


def _golden_inputs():
    gv = _read_golden()
    q = gv["q"].reshape(1, 2, 1, 2)
    k = gv["k"].reshape(1, 2, 1, 2)
    v = gv["v"].reshape(1, 2, 1, 3)
    g = np.log(gv["decay"]).reshape(1, 2, 1, 2)
    beta = gv["beta"].reshape(1, 2, 1)
    s0 = gv["S0"].reshape(1, 1, 2, 3)
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=s0, scale=gv["scale"][0]), gv


def _rand(seed, B=2, T=16, H=2, HV=4, K=8, V=8, s0=True, **kw):
    return prefill_inputs(B, T, H, HV, K, V, dtype="fp32", init_state=s0, seed=seed, **kw)


def _np(d):
    out = {}
    for key, val in d.items():
        out[key] = val.double().numpy() if isinstance(val, torch.Tensor) else val
    return out


# ---------------------------------------------------------------- hand example

@pytest.mark.parametrize("impl", ["recurrent", "chunked1", "chunked2", "brute"])
def test_hand_worked_example(impl):
    inp, gv = _golden_inputs()
    if impl == "recurrent":
        o, s = recurrent(**inp)
    elif impl == "brute":
        o, s = brute(**inp)
    else:
        o, s = chunked(**inp, chunk_size=int(impl[-1]))
    np.testing.assert_allclose(o.reshape(-1), gv["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(s.reshape(-1), gv["S_final"], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- cross-formulations

@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("s0", [False, True])
def test_recurrent_equals_brute_force(seed, s0):
    inp = _np(_rand(seed, s0=s0))
    o1, s1 = recurrent(**inp)
    o3, s3 = brute(**inp)
    np.testing.assert_allclose(o1, o3, **TOL)
    np.testing.assert_allclose(s1, s3, **TOL)


@pytest.mark.parametrize("chunk", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("solver", ["forward", "numpy"])
def test_recurrent_equals_chunked(chunk, solver):
    inp = _np(_rand(10 + chunk))
    o1, s1 = recurrent(**inp)
    o2, s2 = chunked(**inp, chunk_size=chunk, solver=solver)
    np.testing.assert_allclose(o1, o2, **TOL)
    np.testing.assert_allclose(s1, s2, **TOL)


def test_recurrent_equals_chunked_long_slow_gate():
    # a slow gate keeps old state alive across many chunks
    inp = _np(prefill_inputs(1, 96, 1, 2, 16, 12, dtype="fp32", seed=7, gate="slow"))
    o1, s1 = recurrent(**inp)
    o2, s2 = chunked(**inp, chunk_size=32)
    np.testing.assert_allclose(o1, o2, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(s1, s2, rtol=1e-9, atol=1e-11)


def test_forward_substitution_matches_library_inverse():
    rng = np.random.default_rng(3)
    for c in (1, 5, 16, 64):
        m = np.tril(rng.standard_normal((c, c)) * 0.3, -1)
        t = forward_substitution_inverse(m)
        np.testing.assert_allclose(t, np.linalg.inv(np.eye(c) + m), rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(t @ (np.eye(c) + m), np.eye(c), atol=1e-10)


# ---------------------------------------------------------------- closed forms

def test_beta_zero_is_pure_decayed_readout():
    inp = _np(_rand(21))
    inp["beta"] = np.zeros_like(inp["beta"])
    o, s = recurrent(**inp)
    B, T, H, K = inp["q"].shape
    HV = inp["v"].shape[2]
    G = HV // H
    gsum = np.cumsum(inp["g"], axis=1)                         # global cumsum over time
    s0 = inp["initial_state"]
    for b in range(B):
        for hv in range(HV):
            for t in range(T):
                qt = inp["scale"] * inp["q"][b, t, hv // G]
                ref = s0[b, hv].T @ (np.exp(gsum[b, t, hv]) * qt)
                np.testing.assert_allclose(o[b, t, hv], ref, **TOL)
            np.testing.assert_allclose(s[b, hv], np.exp(gsum[b, -1, hv])[:, None] * s0[b, hv], **TOL)
    # and with a zero state nothing is ever read
    inp["initial_state"] = None
    o, s = recurrent(**inp)
    assert np.all(o == 0) and np.all(s == 0)


def test_key_value_recall_with_orthonormal_keys():
    rng = np.random.default_rng(4)
    K, V, T = 8, 5, 6
    basis, _ = np.linalg.qr(rng.standard_normal((K, K)))
    keys = basis[:, :T].T                                       # T orthonormal keys
    vals = rng.standard_normal((T, V))
    q = rng.standard_normal((1, T, 1, K))
    inp = dict(q=q, k=keys.reshape(1, T, 1, K), v=vals.reshape(1, T, 1, V),
               g=np.zeros((1, T, 1, K)), beta=np.ones((1, T, 1)), scale=0.3)
    o, s = recurrent(**inp)
    np.testing.assert_allclose(s[0, 0], keys.T @ vals, atol=1e-12)
    # first token reads the state it just wrote: o_1 = scale (q_1 . k_1) v_1
    np.testing.assert_allclose(o[0, 0, 0], 0.3 * (q[0, 0, 0] @ keys[0]) * vals[0], atol=1e-12)
    # querying with key j returns scale * v_j from the final state
    for j in range(T):
        oj, _ = decode_step(keys[j].reshape(1, 1, K), np.zeros((1, 1, K)), np.zeros((1, 1, V)),
                            np.zeros((1, 1, K)), np.zeros((1, 1)), s, 0.3)
        np.testing.assert_allclose(oj[0, 0], 0.3 * vals[j], atol=1e-12)


def test_delta_rule_overwrites_same_key():
    K, V = 4, 3
    key = np.array([0.5, -0.5, 0.5, 0.5])
    v1, v2 = np.array([1.0, 2.0, 3.0]), np.array([-4.0, 0.5, 7.0])
    inp = dict(q=np.tile(key, (1, 2, 1, 1)), k=np.tile(key, (1, 2, 1, 1)),
               v=np.stack([v1, v2]).reshape(1, 2, 1, V), g=np.zeros((1, 2, 1, K)),
               beta=np.ones((1, 2, 1)), scale=1.0)
    o, s = recurrent(**inp)
    np.testing.assert_allclose(s[0, 0], np.outer(key, v2), atol=1e-14)
    np.testing.assert_allclose(o[0, 1, 0], v2, atol=1e-14)


def test_zero_input_leaves_state_unchanged():
    inp = _np(_rand(5))
    for name in ("q", "k", "v", "g"):
        inp[name] = np.zeros_like(inp[name])
    o, s = recurrent(**inp)
    assert np.all(o == 0)
    np.testing.assert_array_equal(s, inp["initial_state"])


def test_state_passing_split_equals_whole():
    inp = _np(_rand(6, T=16))
    o, s = recurrent(**inp)
    first = {k: (v[:, :6] if isinstance(v, np.ndarray) and k != "initial_state" else v) for k, v in inp.items()}
    o_a, s_a = recurrent(**first)
    second = {k: (v[:, 6:] if isinstance(v, np.ndarray) and k != "initial_state" else v) for k, v in inp.items()}
    second["initial_state"] = s_a
    o_b, s_b = recurrent(**second)
    np.testing.assert_allclose(np.concatenate([o_a, o_b], axis=1), o, **TOL)
    np.testing.assert_allclose(s_b, s, **TOL)


def test_gva_equals_explicit_repeat_interleave():
    inp = _np(_rand(8, H=2, HV=6))
    o, s = recurrent(**inp)
    rep = dict(inp)
    rep["q"] = np.repeat(inp["q"], 3, axis=2)                  # [q0,q0,q0,q1,q1,q1]
    rep["k"] = np.repeat(inp["k"], 3, axis=2)
    o_r, s_r = recurrent(**rep)
    np.testing.assert_allclose(o, o_r, **TOL)
    np.testing.assert_allclose(s, s_r, **TOL)
    # and the map really is hv // G: head 1 uses q/k head 0, head 3 uses head 1
    swapped = dict(rep)
    swapped["q"] = rep["q"][:, :, [0, 3, 1, 4, 2, 5]]
    o_w, _ = recurrent(**swapped)
    assert not np.allclose(o_w, o)


def test_linearity_in_values_and_state_and_scale():
    a = _np(_rand(9))
    b = _np(_rand(19))
    mix = dict(a)
    mix["v"] = 2.0 * a["v"] - 0.5 * b["v"]
    mix["initial_state"] = 2.0 * a["initial_state"] - 0.5 * b["initial_state"]
    ob = dict(a)
    ob["v"], ob["initial_state"] = b["v"], b["initial_state"]
    o_a, s_a = recurrent(**a)
    o_b, s_b = recurrent(**ob)
    o_m, s_m = recurrent(**mix)
    np.testing.assert_allclose(o_m, 2.0 * o_a - 0.5 * o_b, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(s_m, 2.0 * s_a - 0.5 * s_b, rtol=1e-9, atol=1e-12)
    sc = dict(a)
    sc["scale"] = 3.0 * a["scale"]
    o_s, s_s = recurrent(**sc)
    np.testing.assert_allclose(o_s, 3.0 * o_a, **TOL)
    np.testing.assert_allclose(s_s, s_a, **TOL)


def test_decode_step_single_token_closed_form():
    # g = 0, beta = 1, S = 0: S_new = k v^T and o = scale (q . k) v
    rng = np.random.default_rng(11)
    B, H, HV, K, V = 3, 2, 4, 6, 5
    q, k = rng.standard_normal((B, H, K)), rng.standard_normal((B, H, K))
    v = rng.standard_normal((B, HV, V))
    o, s = decode_step(q, k, v, np.zeros((B, HV, K)), np.ones((B, HV)), np.zeros((B, HV, K, V)), 0.7)
    for b in range(B):
        for hv in range(HV):
            h = hv // 2
            np.testing.assert_allclose(s[b, hv], np.outer(k[b, h], v[b, hv]), atol=1e-13)
            np.testing.assert_allclose(o[b, hv], 0.7 * (q[b, h] @ k[b, h]) * v[b, hv], atol=1e-13)


# ---------------------------------------------------------------- the pins catch planted mistakes

def _mutant_recurrent(step, inp):
    q, k, v, g, beta = (np.asarray(inp[n], dtype=np.float64) for n in ("q", "k", "v", "g", "beta"))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    s = np.zeros((B, HV, K, V)) if inp.get("initial_state") is None else np.array(inp["initial_state"], dtype=np.float64)
    o = np.zeros((B, T, HV, V))
    for t in range(T):
        o[:, t], s = step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], s, inp["scale"])
    return o, s


def _m_undecayed_prediction(q, k, v, g, beta, s, scale):
    G = v.shape[1] // q.shape[1]
    kh, qh = np.repeat(k, G, 1), np.repeat(q, G, 1) * scale
    pred = np.einsum("bhkv,bhk->bhv", s, kh)                      # prediction before decay
    s = np.exp(g)[..., None] * s
    s = s + kh[..., None] * (beta[..., None] * (v - pred))[:, :, None, :]
    return np.einsum("bhkv,bhk->bhv", s, qh), s


def _m_read_before_write(q, k, v, g, beta, s, scale):
    G = v.shape[1] // q.shape[1]
    kh, qh = np.repeat(k, G, 1), np.repeat(q, G, 1) * scale
    s = np.exp(g)[..., None] * s
    o = np.einsum("bhkv,bhk->bhv", s, qh)                         # reads the old state
    s = s + kh[..., None] * (beta[..., None] * (v - np.einsum("bhkv,bhk->bhv", s, kh)))[:, :, None, :]
    return o, s


def _m_gva_modulo(q, k, v, g, beta, s, scale):
    HV, H = v.shape[1], q.shape[1]
    idx = np.arange(HV) % H                                       # hv % H instead of hv // G
    kh, qh = k[:, idx], q[:, idx] * scale
    s = np.exp(g)[..., None] * s
    s = s + kh[..., None] * (beta[..., None] * (v - np.einsum("bhkv,bhk->bhv", s, kh)))[:, :, None, :]
    return np.einsum("bhkv,bhk->bhv", s, qh), s


def _m_decay_on_value_axis(q, k, v, g, beta, s, scale):
    G = v.shape[1] // q.shape[1]
    kh, qh = np.repeat(k, G, 1), np.repeat(q, G, 1) * scale
    kd, vd = s.shape[2], s.shape[3]
    gv = np.resize(g, (g.shape[0], g.shape[1], vd)) if vd != kd else g
    s = np.exp(gv)[:, :, None, :] * s                             # decays value columns
    s = s + kh[..., None] * (beta[..., None] * (v - np.einsum("bhkv,bhk->bhv", s, kh)))[:, :, None, :]
    return np.einsum("bhkv,bhk->bhv", s, qh), s


def _m_beta_on_write_only_error_sign(q, k, v, g, beta, s, scale):
    G = v.shape[1] // q.shape[1]
    kh, qh = np.repeat(k, G, 1), np.repeat(q, G, 1) * scale
    s = np.exp(g)[..., None] * s
    s = s + kh[..., None] * (beta[..., None] * (v + np.einsum("bhkv,bhk->bhv", s, kh)))[:, :, None, :]
    return np.einsum("bhkv,bhk->bhv", s, qh), s


@pytest.mark.parametrize("mutant", [_m_undecayed_prediction, _m_read_before_write, _m_gva_modulo,
                                    _m_decay_on_value_axis, _m_beta_on_write_only_error_sign])
def test_pins_catch_planted_mistakes(mutant):
    caught = []
    inp, gv = _golden_inputs()
    o, s = _mutant_recurrent(mutant, inp)
    caught.append(not (np.allclose(o.reshape(-1), gv["o"]) and np.allclose(s.reshape(-1), gv["S_final"])))
    rnd = _np(_rand(31, H=2, HV=4, K=8, V=6))
    o, s = _mutant_recurrent(mutant, rnd)
    o3, s3 = brute(**rnd)
    caught.append(not (np.allclose(o, o3) and np.allclose(s, s3)))
    assert any(caught), "no pin distinguishes this planted mistake"
