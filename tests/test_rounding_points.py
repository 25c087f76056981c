"""Where the bf16 prefill's error comes from: a float64 emulation of the chunked form with
each of the two-kernel path's bf16 rounding points switchable, against the oracle.

The chunked form is the one of the K3 README's roadmap row L2 (per 64-token chunk: the
in-chunk cumsum G, Gam = exp(G), M and Aq from decay-weighted key products, T = (I + M)^-1,
U = T beta (V - (K*Gam) S0), O = (Q*Gam) S0 + Aq U, S_C = Gam_C S0 + (K*Gam_C/Gam)^T U). The
products of M and Aq are formed the way the factors are stored: per 16-token block I, a row
operand x_i exp(G_i - G_rI) and a column operand k_j exp(G_rI - G_j), with r_I the block's
first token. A rounding point rounds one quantity to bf16 (round to nearest even) where the
kernel hands it to a bf16 matrix product or stores it; everything else is exact.

The checks:
* with no rounding point the emulation is the oracle (to 1e-11), so the algebra is right;
* with a single bf16 rounding at every point (the design before the hi + lo pairs), the
  per-element bound |err| <= 2e-2 RMS + 2^-8 |ref| fails on a workload-shaped head, and the
  points that set the excess are the diagonal-tile Aq operands, the stored diagonal Aq
  tiles, beta (V - X) and U: each alone takes more of the bound than the rest together;
* with the points the kernel still rounds once (those four now carried as bf16 hi + lo
  pairs, i.e. exact to ~2^-16), the bound holds with room to spare;
* on the stress input with beta ~ 1e-3, the rounding of Q*Gam and of S in the readout
  (Q*Gam) S each break the bound alone: the reason that case's per-element figure is
  logged but not asserted in the GPU tests.

Test infrastructure: nothing here runs the HIP path.
"""

import numpy as np
import pytest

from oracle import recurrent
from synth import prefill_inputs
from tests.helpers import head_slice

# every rounding point of the two-kernel path
ALL_POINTS = (
    "qg", "kg", "kd",            # stored Q*Gam, K*Gam, (K*Gam_C/Gam)^T tiles
    "m_ops",                     # operands of M's decay-weighted key products
    "aq_ops_diag", "aq_ops_off",  # operands of Aq's products: diagonal / off-diagonal tiles
    "aq_diag", "aq_off",         # stored Aq: diagonal 16 x 16 tiles / the rest
    "t",                         # stored T
    "s_x", "s_p",                # the state as operand of X = (K*Gam) S / P = (Q*Gam) S
    "y",                         # beta (V - X) as operand of U = T Y
    "u_o", "u_s",                # U as operand of Aq U / of the state update
    "o",                         # stored o
)
# carried as bf16 hi + lo pairs by the kernel
SPLIT_POINTS = ("aq_ops_diag", "aq_diag", "y", "u_o", "u_s")
KERNEL_POINTS = tuple(p for p in ALL_POINTS if p not in SPLIT_POINTS)


def bf16_round(x):
    """float64 -> nearest bf16 value (8 significant bits, ties to even), as float64."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def emulate(q, k, v, g, beta, s0, scale, points, C=64, blk=16):
    """One head: q, k, g [T, K]; v [T, V]; beta [T]; s0 [K, V]; float64 arrays."""
    rnd = lambda name, x: bf16_round(x) if name in points else x
    T, K = q.shape
    S = s0.copy()
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        qc, kc, vc, bc = q[c0:c0 + n], k[c0:c0 + n], v[c0:c0 + n], beta[c0:c0 + n]
        G = np.cumsum(g[c0:c0 + n], axis=0)
        gam = np.exp(G)
        M = np.zeros((n, n))
        Aq = np.zeros((n, n))
        diag = np.zeros((n, n), dtype=bool)
        for I in range(0, n, blk):
            rows = slice(I, min(I + blk, n))
            ref = G[I]                                   # the block's first token
            diag[rows, rows] = True
            fr = np.exp(G[rows] - ref)                   # row factors <= 1
            fc = np.exp(ref - G[:rows.stop])             # column factors of tokens <= block end
            krow, qrow, kcol = kc[rows] * fr, qc[rows] * fr, kc[:rows.stop] * fc
            m = rnd("m_ops", krow) @ rnd("m_ops", kcol).T
            a_d = rnd("aq_ops_diag", qrow) @ rnd("aq_ops_diag", kcol).T
            a_o = rnd("aq_ops_off", qrow) @ rnd("aq_ops_off", kcol).T
            M[rows, :rows.stop] = bc[rows, None] * m
            Aq[rows, :rows.stop] = np.where(diag[rows, :rows.stop], a_d, a_o)
        lower = np.tril(np.ones((n, n), dtype=bool))
        M = np.where(lower & ~np.eye(n, dtype=bool), M, 0.0)
        Aq = np.where(lower, Aq, 0.0)
        Tm = rnd("t", np.linalg.inv(np.eye(n) + M))
        Aq = np.where(diag, rnd("aq_diag", Aq), rnd("aq_off", Aq))
        X = rnd("kg", kc * gam) @ rnd("s_x", S)
        U = Tm @ rnd("y", bc[:, None] * (vc - X))
        O = rnd("qg", qc * gam) @ rnd("s_p", S) + Aq @ rnd("u_o", U)
        o[c0:c0 + n] = rnd("o", scale * O)
        S = gam[-1][:, None] * S + rnd("kd", kc * (gam[-1] / gam)).T @ rnd("u_s", U)
    return o, S


def _ratio(got, ref):
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref) / (2e-2 * rms + 2.0 ** -8 * np.abs(ref))))


class Head:
    """One (b = 0, hv) head of a prefill input, as float64 arrays, with its oracle result."""

    def __init__(self, inp, hv):
        one = head_slice(inp, 0, hv, inp["v"].shape[2] // inp["q"].shape[2])
        f = lambda t: t[0, :, 0].double().numpy()
        self.q, self.k, self.v, self.g = (f(one[n]) for n in ("q", "k", "v", "g"))
        self.beta = one["beta"][0, :, 0].double().numpy()
        self.s0 = one["initial_state"][0, 0].double().numpy()
        self.scale = one["scale"]
        ref_o, ref_s = recurrent(**one)
        self.ref_o, self.ref_s = ref_o[0, :, 0], ref_s[0, 0]

    def ratios(self, points):
        o, s = emulate(self.q, self.k, self.v, self.g, self.beta, self.s0, self.scale,
                       frozenset(points))
        return _ratio(o, self.ref_o), _ratio(s, self.ref_s)


@pytest.fixture(scope="module")
def workload_heads():
    # the long-prefill workload's recipe (default gate and beta, S0 ~ N(0, 0.1), K = V = 128),
    # 1,024 tokens of two heads
    inp = prefill_inputs(1, 1024, 2, 2, 128, 128, "bf16", True, 11)
    return [Head(inp, hv) for hv in range(2)]


def test_emulation_without_rounding_is_the_oracle(workload_heads):
    for h in workload_heads:
        o, s = emulate(h.q, h.k, h.v, h.g, h.beta, h.s0, h.scale, frozenset())
        assert np.max(np.abs(o - h.ref_o)) <= 1e-11 * np.max(np.abs(h.ref_o))
        assert np.max(np.abs(s - h.ref_s)) <= 1e-11 * np.max(np.abs(h.ref_s))


def test_single_rounding_everywhere_breaks_the_bound(workload_heads):
    worst = max(max(h.ratios(ALL_POINTS)) for h in workload_heads)
    assert worst > 1.2, worst


def test_split_points_set_the_excess(workload_heads):
    for h in workload_heads:
        # the compute error of the points the kernel still rounds once, together
        rest_o, rest_s = h.ratios(tuple(p for p in KERNEL_POINTS if p != "o"))
        for p in ("aq_ops_diag", "aq_diag", "y", "u_o"):
            assert h.ratios((p,))[0] > rest_o, p
        for p in ("y", "u_s"):
            assert h.ratios((p,))[1] > rest_s, p


def test_kernel_rounding_points_meet_the_bound(workload_heads):
    for h in workload_heads:
        r_o, r_s = h.ratios(KERNEL_POINTS)
        assert r_o <= 0.7 and r_s <= 0.5, (r_o, r_s)


def test_small_beta_readout_breaks_the_bound_through_qg_and_s():
    inp = prefill_inputs(1, 512, 1, 1, 128, 128, "bf16", True, 77, gate="default", beta="small")
    h = Head(inp, 0)
    assert h.ratios(KERNEL_POINTS)[0] > 1.5
    assert h.ratios(("qg",))[0] > 1.0 and h.ratios(("s_p",))[0] > 1.0
    rest = tuple(p for p in KERNEL_POINTS if p not in ("qg", "s_p"))
    assert h.ratios(rest)[0] <= 1.0


def test_short_keys_slow_gate_off_diagonal_aq_sets_the_excess():
    # K = 32, V = 64, slow gate, 2,048 tokens: o's per-element figure comes near the bound on
    # the GPU. The emulation puts it there too, and the off-diagonal Aq points (the operands of
    # its products and the stored tiles, rounded once) are what takes the excess: without them
    # the rest stay where they are at K = 128.
    case = dict(B=1, T=2048, H=1, HV=2, K=32, V=64)
    inp = prefill_inputs(**case, dtype="bf16", init_state=True, seed=sum(case.values()) + 16,
                         gate="slow")
    h = Head(inp, 0)
    assert h.ratios(KERNEL_POINTS)[0] > 0.9
    alone = {p: h.ratios((p,))[0] for p in KERNEL_POINTS}
    assert max(alone, key=alone.get) == "aq_ops_off"
    rest = tuple(p for p in KERNEL_POINTS if p not in ("aq_ops_off", "aq_off"))
    assert h.ratios(rest)[0] <= 0.8
