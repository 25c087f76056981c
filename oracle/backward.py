"""Gradients of the KDA recurrence, one token at a time, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The K3 README page ("KDA 训练 → 推理 手写实现") lists, in its roadmap table,
hand-written gradients dq, dk, dv, dg, dbeta for the recurrence (row L1) and an
end-to-end backward of the chunked kernels checked against it (row L4); its
key-constraints table fixes where they land: dv, dg, dbeta per value head, dq
and dk computed per value head and then summed over the G value heads that share
a q/k head.

``recurrent_bwd`` is reverse-mode differentiation of ``recurrent.decode_step``
written out by hand, step by step in reverse order. For one token, with
``s = exp(g) * S_prev`` (rows decayed), ``a = s^T k``, ``u = beta (v - a)``,
``S = s + k u^T`` and ``o = S^T (scale q)``, and dS the gradient reaching S:

    dS     += scale q do^T        dq  = scale S do
    du      = dS^T k              dk  = dS u
    dv      = beta du             dbeta = du . (v - a)
    da      = -beta du            ds  = dS + k da^T,   dk += s da
    dg      = rowsum(ds * s)      dS_prev = exp(g) * ds

The gradient of the final state (``dht``) seeds dS; the one reaching the
initial state is returned as ``dh0``. Forward states are recomputed from
checkpoints every ``ckpt`` tokens, so memory stays at T/ckpt states.

With ``qk_l2norm`` / ``beta_sigmoid`` (the input transforms of ``oracle.transforms``)
the gradients are taken through the transforms by the chain rule: for
``x_hat = x r`` with ``r = (sum x^2 + EPS)^(-1/2)``, ``dx = r (dx_hat - x_hat (x_hat . dx_hat))``;
for ``beta = sigmoid(b)``, ``db = dbeta * beta (1 - beta)``.

Pinned (tests/test_oracle_backward.py) against central finite differences of the
forward oracle ``recurrent``, the pages' gradcheck (float64, eps 1e-6, atol 1e-4).
"""

import numpy as np

from .recurrent import _expand_heads, _f64
from .transforms import EPS, l2_normalize, sigmoid


def _step(q, k, v, g, beta, s_prev, scale):
    """Forward of one token for every (b, hv); q, k already expanded to HV."""
    s = np.exp(g)[:, :, :, None] * s_prev
    a = np.einsum("bhkv,bhk->bhv", s, k)
    u = beta[:, :, None] * (v - a)
    s_new = s + k[:, :, :, None] * u[:, :, None, :]
    return s, a, u, s_new


def recurrent_bwd(q, k, v, g, beta, scale, do, initial_state=None, dht=None, ckpt=64,
                  qk_l2norm=False, beta_sigmoid=False):
    """Gradients of L = sum(o * do) + sum(S_T * dht) with respect to every input.

    Shapes as in ``recurrent``; do [B, T, HV, V]; dht [B, HV, K, V] or None (zeros).
    Returns ``(dq [B,T,H,K], dk [B,T,H,K], dv [B,T,HV,V], dg [B,T,HV,K],
    dbeta [B,T,HV], dh0 [B,HV,K,V])`` in float64. ``qk_l2norm`` / ``beta_sigmoid``:
    the forward applied those transforms (``recurrent``'s flags); the gradients are with
    respect to the raw inputs.
    """
    if qk_l2norm or beta_sigmoid:
        q, k, beta = (_f64(a) for a in (q, k, beta))
        qn = l2_normalize(q) if qk_l2norm else q
        kn = l2_normalize(k) if qk_l2norm else k
        bn = sigmoid(beta) if beta_sigmoid else beta
        dq, dk, dv, dg, db, dh0 = recurrent_bwd(qn, kn, v, g, bn, scale, do, initial_state,
                                                dht, ckpt)
        if qk_l2norm:
            def through_norm(x, xn, dxn):
                r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)
                return r * (dxn - xn * np.sum(xn * dxn, axis=-1, keepdims=True))
            dq, dk = through_norm(q, qn, dq), through_norm(k, kn, dk)
        if beta_sigmoid:
            db = db * bn * (1.0 - bn)
        return dq, dk, dv, dg, db, dh0
    q, k, v, g, beta, do = (_f64(a) for a in (q, k, v, g, beta, do))
    b, t_len, h, kd = q.shape
    hv, vd = v.shape[2], v.shape[3]
    G = hv // h
    s0 = np.zeros((b, hv, kd, vd)) if initial_state is None else _f64(initial_state)
    qe = np.stack([_expand_heads(q[:, t], hv) for t in range(t_len)], axis=1)
    ke = np.stack([_expand_heads(k[:, t], hv) for t in range(t_len)], axis=1)

    # forward checkpoints: the state before tokens 0, ckpt, 2 ckpt, ...
    marks = list(range(0, t_len, ckpt))
    saved = {}
    s = s0
    for t in range(t_len):
        if t % ckpt == 0:
            saved[t] = s
        s = _step(qe[:, t], ke[:, t], v[:, t], g[:, t], beta[:, t], s, scale)[3]

    dqe = np.zeros_like(qe)
    dke = np.zeros_like(ke)
    dv = np.zeros_like(v)
    dg = np.zeros_like(g)
    dbeta = np.zeros_like(beta)
    dS = np.zeros((b, hv, kd, vd)) if dht is None else _f64(dht)
    for m in reversed(marks):
        end = min(m + ckpt, t_len)
        # states before each token of the segment
        states = [saved[m]]
        for t in range(m, end - 1):
            states.append(_step(qe[:, t], ke[:, t], v[:, t], g[:, t], beta[:, t], states[-1],
                                scale)[3])
        for t in reversed(range(m, end)):
            qt, kt, vt, gt, bt = qe[:, t], ke[:, t], v[:, t], g[:, t], beta[:, t]
            s, a, u, s_new = _step(qt, kt, vt, gt, bt, states[t - m], scale)
            dot = do[:, t]
            dqe[:, t] = scale * np.einsum("bhkv,bhv->bhk", s_new, dot)
            dS = dS + scale * qt[:, :, :, None] * dot[:, :, None, :]
            du = np.einsum("bhkv,bhk->bhv", dS, kt)
            dk_t = np.einsum("bhkv,bhv->bhk", dS, u)
            dv[:, t] = bt[:, :, None] * du
            dbeta[:, t] = np.sum(du * (vt - a), axis=-1)
            da = -bt[:, :, None] * du
            ds = dS + kt[:, :, :, None] * da[:, :, None, :]
            dk_t = dk_t + np.einsum("bhkv,bhv->bhk", s, da)
            dke[:, t] = dk_t
            dg[:, t] = np.sum(ds * s, axis=-1)
            dS = np.exp(gt)[:, :, :, None] * ds
    # GVA: value heads hv = h G + j all read q/k head h
    dq = dqe.reshape(b, t_len, h, G, kd).sum(axis=3)
    dk = dke.reshape(b, t_len, h, G, kd).sum(axis=3)
    return dq, dk, dv, dg, dbeta, dS
