"""O3: brute force by explicit composition of per-token affine maps (tiny shapes).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

One token of the KDA recurrence (K3 README page "KDA 训练 → 推理 手写实现",
roadmap row L1, with the KDA CUDA Trainer README's order of operations) maps
the state as ``S_t = A_t S_{t-1} + beta_t k_t v_t^T`` with the K x K matrix
``A_t = (I - beta_t k_t k_t^T) diag(exp(g_t))``. Here every state is formed
from scratch as ``(A_t ... A_1) S_0 + sum_j (A_t ... A_{j+1}) beta_j k_j v_j^T``
and read as ``o_t = S_t^T (scale q_t)``. Cost O(T^2 K^3) per head: use it for
T <= 32, K <= 16 only.
"""

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.array(x, dtype=np.float64, copy=True)


def brute(q, k, v, g, beta, scale, initial_state=None):
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    b, t_len, h, kd = q.shape
    hv, vd = v.shape[2], v.shape[3]
    if t_len > 64 or kd > 32:
        raise ValueError("brute force is for tiny shapes only")
    grp = hv // h
    o = np.zeros((b, t_len, hv, vd))
    s_fin = np.zeros((b, hv, kd, vd))
    eye = np.eye(kd)
    for bi in range(b):
        for vh in range(hv):
            hh = vh // grp
            s0 = np.zeros((kd, vd)) if initial_state is None else _f64(initial_state[bi, vh])
            maps = []
            writes = []
            for t in range(t_len):
                kt = k[bi, t, hh]
                maps.append((eye - beta[bi, t, vh] * np.outer(kt, kt)) @ np.diag(np.exp(g[bi, t, vh])))
                writes.append(beta[bi, t, vh] * np.outer(kt, v[bi, t, vh]))
            for t in range(t_len):
                # product A_t A_{t-1} ... A_1 applied to S_0
                prod = eye.copy()
                for r in range(t, -1, -1):
                    prod = prod @ maps[r]
                s_t = prod @ s0
                for j in range(t + 1):
                    pj = eye.copy()
                    for r in range(t, j, -1):
                        pj = pj @ maps[r]
                    s_t = s_t + pj @ writes[j]
                o[bi, t, vh] = s_t.T @ (float(scale) * q[bi, t, hh])
                if t == t_len - 1:
                    s_fin[bi, vh] = s_t
    return o, s_fin
