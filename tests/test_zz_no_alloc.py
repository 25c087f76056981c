"""The allocation-free prefill (kda_chunk_fwd_noalloc) through the C ABI against the
entry point it stands in for (kda_chunk_fwd_ex with a torch workspace): bit for bit, and
against the float64 oracle. Three calls in a row on one device share the library's scratch
array, each smaller than the one before (the first takes the segmented route for few heads,
the second the plain two-kernel path, the third a ragged last chunk)."""

import ctypes

import pytest
import torch

import gated_delta_rule_67_amd as kda
from oracle import recurrent
from synth import prefill_inputs
from tests.helpers import assert_parity, gpu, log, to64

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dims(d):
    B, T, H, K = d["q"].shape
    return B, T, H, d["v"].shape[2], K, d["v"].shape[3]


def _noalloc(d, o, s_out, chunk):
    lib = kda.library()
    B, T, H, HV, K, V = _dims(d)
    rc = lib.kda_chunk_fwd_noalloc(_p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["g"]), _p(d["beta"]),
                                   _p(d["initial_state"]), _p(s_out), _p(o), B, T, H, HV, K, V,
                                   float(d["scale"]), chunk, 1, 0, None)
    torch.cuda.synchronize()
    return rc


def _with_workspace(d, o, s_out, chunk):
    lib = kda.library()
    B, T, H, HV, K, V = _dims(d)
    n = lib.kda_chunk_fwd_workspace_size(B, T, H, HV, K, V, chunk, 1)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    rc = lib.kda_chunk_fwd_ex(_p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["g"]), _p(d["beta"]),
                              _p(d["initial_state"]), _p(s_out), _p(o), B, T, H, HV, K, V,
                              float(d["scale"]), chunk, 1, _p(ws), n, 0, None)
    torch.cuda.synchronize()
    return rc, n


CASES = [  # largest first: each later call leaves stale bytes of the earlier ones behind
    dict(B=1, T=8192, H=4, HV=4, K=128, V=128, seed=71, chunk=64),   # segmented, 44.6 MB
    dict(B=2, T=512, H=4, HV=8, K=64, V=64, seed=72, chunk=64),      # plain two-kernel path
    dict(B=1, T=200, H=1, HV=2, K=64, V=48, seed=73, chunk=8),       # ragged last chunk
]


def test_noalloc_matches_the_workspace_entry_point():
    lib = kda.library()
    for c in CASES:
        shape = {k: c[k] for k in ("B", "T", "H", "HV", "K", "V")}
        log(f"noalloc prefill {shape} chunk {c['chunk']}")
        inp = prefill_inputs(**shape, dtype="bf16", init_state=True, seed=c["seed"])
        d = gpu(inp)
        B, T, H, HV, K, V = _dims(d)
        need = lib.kda_chunk_fwd_workspace_size(B, T, H, HV, K, V, c["chunk"], 1)
        assert 0 < need <= kda.NOALLOC_SCRATCH_BYTES
        o_ref = torch.full_like(d["v"], float("nan"))
        s_ref = torch.full_like(d["initial_state"], float("nan"))
        rc, _ = _with_workspace(d, o_ref, s_ref, c["chunk"])
        assert rc == kda.KDA_OK
        o = torch.full_like(d["v"], float("nan"))
        s = torch.full_like(d["initial_state"], float("nan"))
        assert _noalloc(d, o, s, c["chunk"]) == kda.KDA_OK
        assert torch.equal(o, o_ref), "o differs from kda_chunk_fwd_ex"
        assert torch.equal(s, s_ref), "final state differs from kda_chunk_fwd_ex"
        ro, rs = recurrent(**inp)
        assert_parity(to64(o), ro, torch.bfloat16, "o")
        assert_parity(to64(s), rs, torch.bfloat16, "state")


def test_noalloc_binding_and_repeat():
    log("noalloc prefill through the binding, twice on one input")
    inp = prefill_inputs(2, 512, 4, 8, 64, 64, "bf16", True, seed=74)
    d = gpu(inp)
    o_ref, s_ref = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                                     d["initial_state"])
    for _ in range(2):
        o = torch.empty_like(d["v"])
        s = torch.empty_like(d["initial_state"])
        kda.kda_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], o, s, d["scale"],
                                  d["initial_state"])
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
