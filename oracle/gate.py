"""The KDA decay gate and its gradients, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The K3 README page ("KDA 训练 → 推理 手写实现") lists the gate as roadmap row L5:
a standard gate and a safe gate with the upstream semantics, whose hand-written
gradients are those of A_log, dt_bias and the gate input. The key-constraints
table (exp-underflow row) gives the gate path a lower bound of -5.0 and asks for
the clamp to happen before g is applied. The model card (Model table) describes
the KDA layer's gate as a per-channel decay gate.

The pages print no formula. Reading (the one the workloads' own recipe
``g = max(-5, -softplus(x))`` supports, which is this gate at A_log = 0,
dt_bias = 0): per token, value head hv and key channel c, with z = x + dt_bias,

    standard:  g = -exp(A_log[hv]) * softplus(z),   softplus(z) = log(1 + e^z)
    safe:      g = max(lower_bound, standard)        (lower_bound = -5 on the pages)

so exp(g) = (1 + e^z)^(-exp(A_log)) is a per-channel decay factor in (0, 1).
A_log is one value per value head, dt_bias one per (value head, channel).
The gradient of the clamp passes where the standard value is >= lower_bound.
"""

import numpy as np


def softplus(z):
    """log(1 + e^z) in float64 without overflow."""
    return np.logaddexp(0.0, np.asarray(z, dtype=np.float64))


def _logistic(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _prepare(x, A_log, dt_bias):
    x = np.asarray(x, dtype=np.float64)
    HV, K = x.shape[-2], x.shape[-1]
    a = np.exp(np.asarray(A_log, dtype=np.float64).reshape(HV, 1))
    b = np.zeros((HV, K)) if dt_bias is None else np.asarray(dt_bias, np.float64).reshape(HV, K)
    return x, a, x + b


def gate(x, A_log, dt_bias=None, lower_bound=None):
    """g [..., HV, K] from the gate input x [..., HV, K], A_log [HV] and dt_bias [HV, K]
    (None = 0). lower_bound None is the standard gate; a number gives the safe gate."""
    _, a, z = _prepare(x, A_log, dt_bias)
    g = -a * softplus(z)
    if lower_bound is not None:
        g = np.maximum(float(lower_bound), g)
    return g


def gate_bwd(x, A_log, dt_bias, dg, lower_bound=None):
    """Gradients of <g, dg> with respect to x, A_log and dt_bias.

    d softplus(z)/dz is the logistic function, d(-a softplus)/dA_log = -a softplus
    (a = exp(A_log)), and the clamp stops the gradient where the standard value lies
    below lower_bound. dt_bias's gradient sums dx over all leading axes (every token);
    A_log's sums over the tokens and the head's channels.
    Returns (dx [..., HV, K], dA_log [HV], ddt_bias [HV, K])."""
    x, a, z = _prepare(x, A_log, dt_bias)
    dg = np.asarray(dg, dtype=np.float64)
    g_std = -a * softplus(z)
    pass_ = np.ones_like(g_std) if lower_bound is None else (g_std >= float(lower_bound))
    dgm = dg * pass_
    dx = dgm * (-a) * _logistic(z)
    lead = tuple(range(x.ndim - 2))
    ddt_bias = dx.sum(axis=lead)
    dA_log = (dgm * g_std).sum(axis=lead).sum(axis=-1)
    return dx, dA_log, ddt_bias
