"""GPU parity of the chunked paths when g leaves the safe gate's range (g < -5).

The K3 README's roadmap row L5 has a standard gate next to the safe one; the standard gate
has no lower bound, and any caller may pass g below -5. Within a 16-token block the chunk
kernels factor the relative decay through the block's first token, which covers a decay
span of up to 2^96 (about 66 nats); wider blocks take a term-by-term route (exact for any
g <= 0). These tests cover:

* constant g = -8, -20 and -100 (every block wide);
* the standard gate (lower_bound = -inf) applied inside the prefill on a wide gate input
  (x ~ 3 N(0, 1)), B1 T1024 HV16 K128;
* "mixed" g: the default gate with about one token in 64 decaying 40 times faster, so that
  chunks mix blocks of both routes;
* the segmented route (few heads) and packed sequences with wide g.

Each is checked against the float64 oracle at the bf16 criterion (tests/helpers.py)."""

import numpy as np
import pytest
import torch

import gated_delta_rule_67_amd as kda
from oracle import gate, recurrent
from synth import gate_inputs, prefill_inputs
from tests.helpers import assert_parity, gpu, log, to64

pytestmark = pytest.mark.gpu


def _fwd_case(B, T, H, HV, K, V, gate_mode, seed, chunk=64, workspace=True, segments=None):
    # segments None: kda_chunk_fwd's own route; else kda_chunk_fwd_segmented with that count
    # (1: the plain two-kernel path)
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, seed, gate=gate_mode)
    d = gpu(inp)
    if segments is None:
        o, s = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                                 d["initial_state"], chunk_size=chunk)
    else:
        o, s = kda.kda_chunk_fwd_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], segments,
                                           d["scale"], d["initial_state"])
    torch.cuda.synchronize()
    ref_o, ref_s = recurrent(**inp)
    assert_parity(to64(o), ref_o, torch.bfloat16, f"o ({gate_mode})")
    assert_parity(to64(s), ref_s, torch.bfloat16, f"state ({gate_mode})")


@pytest.mark.parametrize("segments", [None, 1], ids=["auto-4-segments", "plain"])
@pytest.mark.parametrize("gate_mode", ["const:-8", "const:-20", "const:-100", "mixed"])
def test_two_kernel_prefill_wide_decay(gate_mode, segments):
    # B1 T1024 H16: kda_chunk_fwd's own route is the segmented one (4 segments)
    log(f"prefill B1 T1024 H16 K128 g={gate_mode} segments={segments or 'auto'}")
    _fwd_case(1, 1024, 16, 16, 128, 128, gate_mode, seed=301, segments=segments)


@pytest.mark.parametrize("shape", [
    dict(B=2, T=200, H=2, HV=4, K=64, V=64),   # GVA, ragged last chunk
    dict(B=1, T=136, H=1, HV=3, K=32, V=32),
])
def test_two_kernel_prefill_wide_decay_small_k(shape):
    for mode in ("const:-20", "mixed"):
        log(f"two-kernel prefill {shape} g={mode}")
        _fwd_case(**shape, gate_mode=mode, seed=302, chunk=8)


def test_standard_gate_inside_the_prefill():
    """kda_chunk_fwd_gated with lower_bound = -inf (the standard gate) on x ~ 3 N(0, 1): the
    oracle applies its own gate (float64, then rounded to bf16 as the kernel stores g)."""
    B, T, H, HV, K, V = 1, 1024, 16, 16, 128, 128
    log("standard gate inside the prefill, B1 T1024 HV16 K128, x ~ 3 N(0, 1)")
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, seed=303)
    gi = gate_inputs(B, T, HV, K, "bf16", seed=304, x_std=3.0)
    g_ref = gate(gi["x"].double().numpy(), gi["A_log"].double().numpy(),
                 gi["dt_bias"].double().numpy(), None)
    wide = float(np.mean(g_ref < -5.0))
    log(f"    share of g below -5: {wide:.3f}, min g {g_ref.min():.1f}")
    assert wide > 0.05
    d = gpu(inp)
    o, s = kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], gi["x"].cuda(), gi["A_log"].cuda(),
                                   gi["dt_bias"].cuda(), d["beta"], None, d["scale"],
                                   d["initial_state"])
    torch.cuda.synchronize()
    ref_o, ref_s = recurrent(**dict(inp, g=torch.from_numpy(g_ref).to(torch.bfloat16)))
    # per-element bound not asserted: where the kernel's float32 gate and the oracle's
    # float64 gate round g to neighbouring bf16 values (one ulp of |g| up to ~40), the
    # decay itself differs by a few per cent
    assert_parity(to64(o), ref_o, torch.bfloat16, "o", elem=False)
    assert_parity(to64(s), ref_s, torch.bfloat16, "state", elem=False)


@pytest.mark.parametrize("gate_mode", ["const:-20", "mixed"])
def test_segmented_prefill_wide_decay(gate_mode):
    log(f"segmented prefill B1 T4096 H4 K128 g={gate_mode}")
    inp = prefill_inputs(1, 4096, 4, 4, 128, 128, "bf16", True, 305, gate=gate_mode)
    d = gpu(inp)
    o, s = kda.kda_chunk_fwd_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], 16,
                                       d["scale"], d["initial_state"])
    torch.cuda.synchronize()
    ref_o, ref_s = recurrent(**inp)
    assert_parity(to64(o), ref_o, torch.bfloat16, "o")
    assert_parity(to64(s), ref_s, torch.bfloat16, "state")


def test_packed_sequences_wide_decay():
    lengths = [70, 0, 200, 33]
    log(f"packed sequences {lengths} g=mixed and const:-20")
    for mode, seed in (("mixed", 306), ("const:-20", 307)):
        T = sum(lengths)
        inp = prefill_inputs(1, T, 2, 4, 64, 64, "bf16", True, seed, gate=mode)
        gen = torch.Generator().manual_seed(seed + 1)
        s0 = 0.1 * torch.randn((len(lengths), 4, 64, 64), generator=gen)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
        d = gpu(inp)
        o, sT = kda.kda_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu.cuda(),
                                         d["scale"], s0.cuda(), True)
        torch.cuda.synchronize()
        for sq in range(len(lengths)):
            a, b = int(cu[sq]), int(cu[sq + 1])
            if a == b:
                continue
            one = {n: inp[n][:, a:b] for n in ("q", "k", "v", "g", "beta")}
            ref_o, ref_s = recurrent(**one, scale=inp["scale"], initial_state=s0[sq:sq + 1])
            assert_parity(to64(o[:, a:b]), ref_o, torch.bfloat16, f"o of sequence {sq} ({mode})")
            assert_parity(to64(sT[sq:sq + 1]), ref_s, torch.bfloat16, f"state of sequence {sq}")


@pytest.mark.parametrize("gate_mode", ["const:-20", "mixed"])
def test_two_kernel_prefill_wide_decay_with_l2norm(gate_mode):
    """The in-kernel q/k L2 normalisation on the wide route: every token's own norm."""
    log(f"two-kernel prefill with q/k L2-norm, B1 T256 H2 HV4 K64, g={gate_mode}")
    inp = prefill_inputs(1, 256, 2, 4, 64, 64, "bf16", True, 308, gate=gate_mode, raw_qk=True)
    d = gpu(inp)
    o, s = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                             d["initial_state"], qk_l2norm=True)
    torch.cuda.synchronize()
    ref_o, ref_s = recurrent(**inp, qk_l2norm=True)
    assert_parity(to64(o), ref_o, torch.bfloat16, "o")
    assert_parity(to64(s), ref_s, torch.bfloat16, "state")


def _abi_fwd_null_workspace(d, o, s_out, dtype_code, chunk):
    """kda_chunk_fwd through the C ABI with a NULL workspace (the single fused kernel for
    bf16, the LDS-staged kernel for float32 and unaligned shapes)."""
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    B, T, H, K = d["q"].shape
    HV, V = d["v"].shape[2], d["v"].shape[3]
    rc = kda.library().kda_chunk_fwd(p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]),
                                     p(d["initial_state"]), p(s_out), p(o), B, T, H, HV, K, V,
                                     float(d["scale"]), chunk, dtype_code, None, 0, None)
    torch.cuda.synchronize()
    return rc


@pytest.mark.parametrize("case", [
    dict(B=1, T=1024, H=16, HV=16, K=128, V=128, dtype="bf16", chunk=64),  # fused kernel
    dict(B=2, T=200, H=2, HV=4, K=64, V=48, dtype="bf16", chunk=8),        # fused, ragged
    dict(B=1, T=136, H=1, HV=3, K=36, V=32, dtype="bf16", chunk=8),        # LDS-staged (K % 8 != 0)
    dict(B=2, T=16, H=2, HV=4, K=8, V=8, dtype="fp32", chunk=8),           # the tiny fp32 workload's shape
    dict(B=1, T=256, H=2, HV=4, K=64, V=64, dtype="fp32", chunk=64),       # fp32, K = 64
])
@pytest.mark.parametrize("gate_mode", ["const:-20", "mixed"])
def test_kernels_without_workspace_wide_decay(case, gate_mode):
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[case["dtype"]]
    shape = {k: case[k] for k in ("B", "T", "H", "HV", "K", "V")}
    log(f"prefill without workspace {shape} {case['dtype']} g={gate_mode}")
    inp = prefill_inputs(**shape, dtype=case["dtype"], init_state=True, seed=309, gate=gate_mode)
    d = gpu(inp)
    o = torch.full(d["v"].shape, float("nan"), dtype=dt, device="cuda")
    s = torch.full(d["initial_state"].shape, float("nan"), dtype=torch.float32, device="cuda")
    assert _abi_fwd_null_workspace(d, o, s, 1 if case["dtype"] == "bf16" else 0,
                                   case["chunk"]) == kda.KDA_OK
    ref_o, ref_s = recurrent(**inp)
    # the kernels without workspace round every operand once, as bf16 (no hi + lo pairs)
    assert_parity(to64(o), ref_o, dt, f"o ({gate_mode})", elem=False)
    assert_parity(to64(s), ref_s, dt, f"state ({gate_mode})", elem=False)


# ------------------------------------------------------------------ backward

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _bwd_case(inp, seed, chunk=64, what=""):
    from oracle import recurrent_bwd
    gen = torch.Generator().manual_seed(seed)
    B, T, HV, V = inp["v"].shape
    K = inp["q"].shape[-1]
    inp = dict(inp, do=torch.randn((B, T, HV, V), generator=gen).to(torch.bfloat16),
               dht=0.1 * torch.randn((B, HV, K, V), generator=gen))
    d = gpu(inp)
    got = kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["scale"],
                            d["initial_state"], d["dht"], chunk)
    torch.cuda.synchronize()
    ref = recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"],
                        inp["do"], inp["initial_state"], inp["dht"])
    for name, x, r in zip(GRADS, got, ref):
        # gradients: the RMS and row criteria (the per-element bound is for the forward)
        assert_parity(to64(x), r, torch.bfloat16, f"{what} {name}", elem=False)


@pytest.mark.parametrize("gate_mode", ["const:-8", "const:-20"])
def test_backward_constant_wide_decay(gate_mode):
    log(f"backward B1 T1024 H16 K128 g={gate_mode}")
    inp = prefill_inputs(1, 1024, 16, 16, 128, 128, "bf16", True, 310, gate=gate_mode)
    _bwd_case(inp, 311, what=gate_mode)


@pytest.mark.parametrize("shape", [
    dict(B=1, T=512, H=4, HV=4, K=128, V=128),
    dict(B=2, T=200, H=2, HV=4, K=64, V=48),   # GVA, ragged last chunk
    dict(B=1, T=128, H=1, HV=2, K=32, V=32),
])
def test_backward_mixed_decay(shape):
    log(f"backward {shape} g=mixed")
    inp = prefill_inputs(**shape, dtype="bf16", init_state=True, seed=312, gate="mixed")
    _bwd_case(inp, 313, chunk=64 if shape["T"] % 64 == 0 else 8, what="mixed")


def test_backward_standard_gate_values():
    """The backward on g made by the standard gate (no lower bound) from x ~ 3 N(0, 1)."""
    B, T, H, HV, K, V = 1, 1024, 16, 16, 128, 128
    log("backward on standard-gate g, B1 T1024 HV16 K128, x ~ 3 N(0, 1)")
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, seed=314)
    gi = gate_inputs(B, T, HV, K, "bf16", seed=315, x_std=3.0)
    g_ref = gate(gi["x"].double().numpy(), gi["A_log"].double().numpy(),
                 gi["dt_bias"].double().numpy(), None)
    inp["g"] = torch.from_numpy(g_ref).to(torch.bfloat16)
    _bwd_case(inp, 316, what="standard gate")
