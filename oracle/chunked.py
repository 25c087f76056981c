"""O2: the chunk-wise form of the KDA recurrence, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The K3 README page ("KDA 训练 → 推理 手写实现"), roadmap table row L2, lists
four steps for the chunked form: (1) cumulative sum of g inside the chunk,
(2) build a lower-triangular system, (3) solve it, (4) pass the state from
chunk to chunk. Written out for one value head and one chunk of C tokens
(local index i; ``Gam_i = exp(G_i)`` per key channel; S0 = state at chunk
start; q already multiplied by ``scale``), unrolling the recurrence inside the
chunk gives:

* ``u_i = beta_i (v_i - S0^T (Gam_i * k_i) - sum_{j<i} (k_i . (Gam_i/Gam_j) k_j) u_j)``
  i.e. ``(I + M) U = diag(beta) (V - (K * Gam) S0)`` with the strictly lower
  ``M_ij = beta_i sum_c k_i[c] k_j[c] exp(G_i[c] - G_j[c])``;
* ``o_i = S0^T (Gam_i * q_i) + sum_{j<=i} (q_i . (Gam_i/Gam_j) k_j) u_j``;
* ``S_C = diag(Gam_C) S0 + (K * Gam_C/Gam)^T U``.

The solve is written as ``T = (I + M)^-1`` by forward substitution (or numpy's
general solver, as a second path), then ``W = T diag(beta) (K * Gam)`` and
``U' = T diag(beta) V`` so that ``U = U' - W S0`` (the WY form). The exponent
``G_i - G_j`` is only formed for j <= i, where it is <= 0 for g <= 0.
"""

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.array(x, dtype=np.float64, copy=True)


def forward_substitution_inverse(m):
    """Inverse of the unit lower-triangular ``I + m`` (``m`` strictly lower), by
    forward substitution, row by row: ``T[i] = e_i - sum_{j<i} m[i, j] T[j]``."""
    c = m.shape[0]
    t = np.zeros((c, c))
    for i in range(c):
        row = np.zeros(c)
        row[i] = 1.0
        for j in range(i):
            row -= m[i, j] * t[j]
        t[i] = row
    return t


def _chunk(qc, kc, vc, gc, bc, s0, solver):
    """One chunk of one value head. qc (scaled), kc, gc [C, K]; vc [C, V]; bc [C]; s0 [K, V]."""
    c = qc.shape[0]
    big_g = np.cumsum(gc, axis=0)                       # step 1: in-chunk inclusive cumsum
    lower_incl = np.tril(np.ones((c, c), dtype=bool))
    diff = big_g[:, None, :] - big_g[None, :, :]        # G_i - G_j, [C, C, K]
    decay = np.where(lower_incl[:, :, None], np.exp(np.where(lower_incl[:, :, None], diff, 0.0)), 0.0)
    kk = np.einsum("ic,jc,ijc->ij", kc, kc, decay)
    m = np.tril(bc[:, None] * kk, -1)                   # step 2: strictly lower system
    a = np.tril(np.einsum("ic,jc,ijc->ij", qc, kc, decay))
    if solver == "forward":                             # step 3: triangular solve
        t = forward_substitution_inverse(m)
    elif solver == "numpy":
        t = np.linalg.solve(np.eye(c) + m, np.eye(c))
    else:
        raise ValueError(solver)
    gam = np.exp(big_g)
    w = t @ (bc[:, None] * kc * gam)
    u_prime = t @ (bc[:, None] * vc)
    u = u_prime - w @ s0                                # step 4: the state enters here
    o = (qc * gam) @ s0 + a @ u
    k_to_end = kc * np.exp(big_g[-1][None, :] - big_g)
    s1 = np.exp(big_g[-1])[:, None] * s0 + k_to_end.T @ u
    return o, s1


def chunked(q, k, v, g, beta, scale, initial_state=None, chunk_size=64, solver="forward"):
    """Chunked forward over the whole sequence; same shapes and results as
    ``oracle.recurrent`` (up to rounding order). Requires T % chunk_size == 0
    (the K3 README's key-constraints table, chunk_size row)."""
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    b, t_len, h, kd = q.shape
    hv, vd = v.shape[2], v.shape[3]
    if t_len % chunk_size != 0:
        raise ValueError("T must be a multiple of chunk_size")
    grp = hv // h
    o = np.zeros((b, t_len, hv, vd))
    s_out = np.zeros((b, hv, kd, vd))
    for bi in range(b):
        for vh in range(hv):
            hh = vh // grp
            s = np.zeros((kd, vd)) if initial_state is None else _f64(initial_state[bi, vh])
            for t0 in range(0, t_len, chunk_size):
                sl = slice(t0, t0 + chunk_size)
                o[bi, sl, vh], s = _chunk(
                    q[bi, sl, hh] * float(scale), k[bi, sl, hh], v[bi, sl, vh],
                    g[bi, sl, vh], beta[bi, sl, vh], s, solver)
            s_out[bi, vh] = s
    return o, s_out
