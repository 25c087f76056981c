"""O1: the KDA recurrence, one token at a time, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed, per value head ``hv`` with its K x V state ``S``
(K3 README page "KDA 训练 → 推理 手写实现", roadmap table row L1; the order of
operations is the one in the KDA CUDA Trainer README's model paragraph):

1. decay: every key row of ``S`` is multiplied by ``exp(g_t)`` (a per-key-
   channel gate, natural log, one value per key channel);
2. delta-rule write: the prediction ``S'^T k_t`` is read from the *decayed*
   state, and ``S = S' + k_t (beta_t (v_t - S'^T k_t))^T``;
3. read: ``o_t = S_t^T (scale * q_t)`` from the *updated* state.

Grouped value heads (K3 README, key-constraints table, GVA row): q and k are
repeated G = HV/H times along the head axis, element-interleaved, so value
head ``hv`` uses q/k head ``hv // G``. ``scale`` multiplies q at the entry
(same table, scale row); callers pass 1/sqrt(K).

Readings where the pages are terse: beta is one scalar per (token, value head),
used as given (already squashed into (0, 1)); g is used as given (no clamp,
no transform); the initial state defaults to zeros.
"""

import numpy as np

from .transforms import l2_normalize, sigmoid


def _f64(x):
    """Copy any array-like (numpy, or a CPU torch tensor of any float dtype) to float64 numpy."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.array(x, dtype=np.float64, copy=True)


def _expand_heads(x, hv):
    """[B, H, K] -> [B, HV, K] with head h repeated G = HV/H times in place
    (the GVA map of the K3 README's key-constraints table)."""
    h = x.shape[1]
    if hv % h != 0:
        raise ValueError(f"HV={hv} is not a multiple of H={h}")
    return np.repeat(x, hv // h, axis=1)


def decode_step(q, k, v, g, beta, state, scale, qk_l2norm=False, beta_sigmoid=False):
    """One token of the recurrence for every (b, hv).

    Shapes: q, k [B, H, K]; v [B, HV, V]; g [B, HV, K]; beta [B, HV];
    state [B, HV, K, V]. Returns ``(o [B, HV, V], new_state [B, HV, K, V])``
    in float64; the argument ``state`` is not modified.

    This is the single step the K3 README's roadmap row L6 (recurrent decode
    against a [B, HV, K, V] state cache) repeats per generated token.
    ``qk_l2norm`` / ``beta_sigmoid`` first apply the input transforms of
    ``oracle.transforms`` to q, k / beta.
    """
    q, k, v, g, beta, s = (_f64(a) for a in (q, k, v, g, beta, state))
    if qk_l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    if beta_sigmoid:
        beta = sigmoid(beta)
    hv = v.shape[1]
    qh = _expand_heads(q, hv) * float(scale)
    kh = _expand_heads(k, hv)
    # 1. decay each key row of the state
    s = np.exp(g)[:, :, :, None] * s
    # 2. prediction from the decayed state, then the delta-rule write
    pred = np.einsum("bhkv,bhk->bhv", s, kh)
    u = beta[:, :, None] * (v - pred)
    s = s + kh[:, :, :, None] * u[:, :, None, :]
    # 3. read from the updated state
    o = np.einsum("bhkv,bhk->bhv", s, qh)
    return o, s


def recurrent(q, k, v, g, beta, scale, initial_state=None, qk_l2norm=False, beta_sigmoid=False):
    """The whole sequence, token by token.

    Shapes: q, k [B, T, H, K]; v [B, T, HV, V]; g [B, T, HV, K]; beta [B, T, HV];
    initial_state [B, HV, K, V] or None (zeros). Returns ``(o [B, T, HV, V],
    final_state [B, HV, K, V])`` in float64. ``qk_l2norm`` / ``beta_sigmoid`` as in
    ``decode_step``.
    """
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    b, t_len, _, kd = q.shape
    hv, vd = v.shape[2], v.shape[3]
    if initial_state is None:
        s = np.zeros((b, hv, kd, vd))
    else:
        s = _f64(initial_state)
    o = np.zeros((b, t_len, hv, vd))
    for t in range(t_len):
        o[:, t], s = decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], s, scale,
                                 qk_l2norm, beta_sigmoid)
    return o, s
