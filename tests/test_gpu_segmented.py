"""GPU parity of the segmented prefill (kda_chunk_fwd_segmented, and kda_chunk_fwd when it picks
that route for few heads) against the fp64 oracle.

The segmented path composes per-segment affine state maps in a scan, so it differs from the
plain two-kernel path by rounding only; it is held to the same bf16 reading of the tolerance
(RMS(err) <= 2e-2 RMS(ref) with the per-row guard). Shapes cover one chunk per segment, a
segment count that is not a power of two, GVA, K < V and K > V, the scan's unrolled segment
counts (8, 16, 32) and its loop, an initial state updated in place, the input transforms, the
fused gate, and a 32,768-token sequence on four heads."""

import numpy as np
import pytest
import torch

import gated_delta_rule_67_amd as kda
from oracle import gate, recurrent
from synth import gate_inputs, prefill_inputs
from tests.helpers import assert_parity, gpu, log, to64

pytestmark = pytest.mark.gpu


def _check(o, s, inp, **kw):
    o_ref, s_ref = recurrent(**inp, **kw)
    assert_parity(to64(o), o_ref, torch.bfloat16, "o")
    assert_parity(to64(s), s_ref, torch.bfloat16, "state")


@pytest.mark.parametrize("case", [
    dict(B=1, T=1024, H=2, HV=2, K=128, V=128, segments=4),
    dict(B=2, T=512, H=2, HV=4, K=64, V=64, segments=8),     # one chunk per segment, GVA
    dict(B=1, T=768, H=1, HV=1, K=32, V=48, segments=3),     # 3 segments of 4 chunks, V > K
    dict(B=1, T=512, H=1, HV=2, K=128, V=64, segments=2),
    dict(B=1, T=256, H=1, HV=1, K=64, V=64, segments=1),     # the plain path
    dict(B=1, T=4096, H=1, HV=1, K=128, V=128, segments=32),  # the scan unrolled for 32
    dict(B=1, T=2048, H=1, HV=2, K=32, V=32, segments=16),    # ... for 16, at K = 32
])
def test_segmented_matches_oracle(case):
    seg = case.pop("segments")
    inp = prefill_inputs(**case, dtype="bf16", init_state=True, seed=sum(case.values()) + seg,
                         gate="slow")  # a slow gate carries state across segments
    log(f"segmented {case} segments={seg}")
    d = gpu(inp)
    o, s = kda.kda_chunk_fwd_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], seg,
                                       inp["scale"], d["initial_state"])
    torch.cuda.synchronize()
    _check(o, s, inp)


def test_segmented_in_place_state_and_transforms():
    inp = prefill_inputs(1, 1024, 2, 2, 128, 128, "bf16", True, seed=50, beta="logit",
                         raw_qk=True)
    d = gpu(inp)
    state = d["initial_state"].clone()
    ws_bytes = kda.library().kda_chunk_fwd_segmented_workspace_size(1, 1024, 2, 2, 128, 128, 4, 1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=state.device)
    o = torch.empty_like(d["v"])
    import ctypes
    rc = kda.library().kda_chunk_fwd_segmented(
        *(ctypes.c_void_p(d[n].data_ptr()) for n in ("q", "k", "v", "g", "beta")),
        ctypes.c_void_p(state.data_ptr()), ctypes.c_void_p(state.data_ptr()),
        ctypes.c_void_p(o.data_ptr()), 1, 1024, 2, 2, 128, 128, inp["scale"], 4, 1,
        ctypes.c_void_p(ws.data_ptr()), ws_bytes, kda.KDA_FLAG_QK_L2NORM | kda.KDA_FLAG_BETA_SIGMOID,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == kda.KDA_OK, kda.status_string(rc)
    _check(o, state, inp, qk_l2norm=True, beta_sigmoid=True)


def test_auto_selects_segments_for_few_heads():
    """B=1, T=4096, two heads: kda_chunk_fwd itself takes the segmented route (16 segments on
    a 256-CU device) and sizes its workspace for it."""
    B, T, H, HV, K, V = 1, 4096, 2, 2, 128, 128
    lib = kda.library()
    plain = lib.kda_chunk_fwd_segmented_workspace_size(B, T, H, HV, K, V, 1, 1)
    auto = lib.kda_chunk_fwd_workspace_size(B, T, H, HV, K, V, 64, 1)
    log(f"workspace plain {plain} auto {auto}")
    assert auto > plain  # the maps and entering states of the segments
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, seed=51, gate="slow")
    d = gpu(inp)
    o, s = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp["scale"],
                             d["initial_state"])
    o1, s1 = kda.kda_chunk_fwd_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], 1,
                                         inp["scale"], d["initial_state"])
    torch.cuda.synchronize()
    _check(o, s, inp)
    _check(o1, s1, inp)


def test_auto_selects_four_segments_for_sixteen_heads():
    """B=1, T=4096, 16 heads: the automatic route takes 4 segments (the largest count whose
    output pass fits a 256-CU chip in one round); its result is that of the explicit 4-segment
    call, bit for bit, and within the bf16 tolerance of the oracle."""
    B, T, H, HV, K, V = 1, 4096, 16, 16, 128, 128
    lib = kda.library()
    four = lib.kda_chunk_fwd_segmented_workspace_size(B, T, H, HV, K, V, 4, 1)
    auto = lib.kda_chunk_fwd_workspace_size(B, T, H, HV, K, V, 64, 1)
    log(f"workspace four segments {four} auto {auto}")
    assert auto == four
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, seed=57, gate="slow")
    d = gpu(inp)
    o, s = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp["scale"],
                             d["initial_state"])
    o4, s4 = kda.kda_chunk_fwd_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], 4,
                                         inp["scale"], d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o, o4) and torch.equal(s, s4)
    _check(o, s, inp)


def test_segmented_with_the_fused_gate():
    B, T, H, HV, K, V = 1, 2048, 2, 2, 64, 64
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, seed=52)
    gd = gate_inputs(B, T, HV, K, "bf16", 53)
    d = gpu(inp)
    dev = d["q"].device
    o, s = kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], gd["x"].to(dev), gd["A_log"].to(dev),
                                   gd["dt_bias"].to(dev), d["beta"], -5.0, inp["scale"],
                                   d["initial_state"])
    torch.cuda.synchronize()
    g_ref = gate(to64(gd["x"]), to64(gd["A_log"]), to64(gd["dt_bias"]), -5.0)
    _check(o, s, dict(inp, g=torch.from_numpy(g_ref).to(torch.bfloat16)))


def test_long_sequence_on_four_heads():
    """B=1, T=32768, H=HV=4, K=V=128 (the long-context layer's sequence on a four-head share):
    the default call runs 16 segments; the full outputs are checked."""
    B, T, H, HV, K, V = 1, 32768, 4, 4, 128, 128
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, seed=54, gate="slow")
    d = gpu(inp)
    log(f"long sequence B={B} T={T} HV={HV}")
    o, s = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp["scale"],
                             d["initial_state"])
    torch.cuda.synchronize()
    _check(o, s, inp)
