"""C-ABI checks that run without a GPU: the library loads, exports every function
that include/kda.h declares, and rejects invalid arguments before any launch
(validation returns before the first HIP call, so no device is touched)."""

import ctypes
import os
import re

import pytest

import gated_delta_rule_67_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.library_path):
        pytest.skip("libkda.so not built")
    return kda.library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("kda_chunk_fwd", "kda_chunk_fwd_ex", "kda_chunk_fwd_workspace_size",
                     "kda_chunk_fwd_varlen", "kda_chunk_fwd_varlen_workspace_size", "kda_chunk_bwd",
                     "kda_recurrent_step_slots", "kda_gate_fwd", "kda_gate_bwd",
                     "kda_gate_bwd_workspace_size",
                     "kda_recurrent_step", "kda_recurrent_step_ex", "kda_status_string",
                     "kda_version"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"libkda.so does not export {name}"


def test_status_strings(lib):
    for rc in (kda.KDA_OK, kda.KDA_ERR_INVALID, kda.KDA_ERR_UNSUPPORTED, kda.KDA_ERR_HIP, 7):
        s = kda.status_string(rc)
        assert isinstance(s, str) and s
    assert kda.status_string(kda.KDA_OK) == "KDA_OK"
    assert lib.kda_version().decode().startswith("kda-gfx950")


def test_workspace_size(lib):
    ws = lib.kda_chunk_fwd_workspace_size
    per = ws(1, 64, 1, 1, 128, 128, 64, 1)  # one (b, hv, 64-token chunk) block, K = 128
    # the block holds Q*Gam, K*Gam, (K*Gam_C/Gam)^T (64 x 128 bf16 each), the lower block
    # triangles of T and Aq (rows 0..31 x 32 and rows 32..63 x 64, bf16), Gam_C (128 fp32),
    # beta (64 fp32) and the residual of Aq's four diagonal 16 x 16 tiles (64 x 16 bf16), in
    # whole kilobytes
    need = 3 * 64 * 128 * 2 + 2 * (32 * 32 + 32 * 64) * 2 + 128 * 4 + 64 * 4 + 64 * 16 * 2
    assert need <= per < need + 1024 and per % 1024 == 0
    assert ws(4, 8192, 16, 16, 128, 128, 64, 1) == 4 * 16 * 128 * per
    assert ws(2, 65, 4, 8, 128, 64, 1, 1) == 2 * 8 * 2 * per     # a partial last chunk counts
    assert ws(1, 64, 1, 1, 64, 64, 64, 1) < per                   # K = 64 blocks are smaller
    assert ws(4, 8192, 16, 16, 64, 64, 64, 0) == 0                # fp32: fused, no workspace
    assert ws(4, 8192, 16, 16, 124, 128, 64, 1) == 0              # K % 8 != 0: generic kernel
    assert ws(4, 8192, 16, 16, 128, 36, 64, 1) == 0               # V % 8 != 0: fused kernel
    assert ws(0, 64, 1, 1, 128, 128, 64, 1) == 0                  # invalid shapes ask for none


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def _chunk(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, sT=None, o=FAKE, B=2, T=64, H=2,
             HV=4, K=64, V=64, scale=0.125, chunk=64, dtype=1)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["sT"], a["o"],
                             a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"], a["scale"],
                             a["chunk"], a["dtype"], a.get("ws"), a.get("ws_bytes", 0), None)


@pytest.mark.parametrize("bad,rc", [
    (dict(q=None), kda.KDA_ERR_INVALID),
    (dict(o=None), kda.KDA_ERR_INVALID),
    (dict(beta=None), kda.KDA_ERR_INVALID),
    (dict(B=0), kda.KDA_ERR_INVALID),
    (dict(T=-1), kda.KDA_ERR_INVALID),
    (dict(HV=3), kda.KDA_ERR_INVALID),            # HV % H != 0
    (dict(T=72), kda.KDA_ERR_INVALID),            # T % chunk != 0
    (dict(chunk=48), kda.KDA_ERR_INVALID),        # not a supported chunk size
    (dict(chunk=256, T=256), kda.KDA_ERR_INVALID),       # larger than the pages' 128
    (dict(scale=float("nan")), kda.KDA_ERR_INVALID),
    (dict(scale=float("inf")), kda.KDA_ERR_INVALID),
    (dict(dtype=2), kda.KDA_ERR_INVALID),         # no fp16
    (dict(K=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(V=160), kda.KDA_ERR_UNSUPPORTED),
    (dict(K=128, dtype=0), kda.KDA_ERR_UNSUPPORTED),  # fp32 needs K <= 64
    (dict(ws=FAKE, ws_bytes=1024), kda.KDA_ERR_INVALID),          # workspace too small
    (dict(ws=ctypes.c_void_p(0x1010), ws_bytes=1 << 30), kda.KDA_ERR_INVALID),  # misaligned
])
def test_chunk_fwd_rejects_invalid_arguments(lib, bad, rc):
    assert _chunk(lib, **bad) == rc


def _step(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, o=FAKE, B=2, H=2, HV=4, K=64,
             V=64, scale=0.125, dtype=1)
    a.update(kw)
    return lib.kda_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], a["o"],
                                  a["B"], a["H"], a["HV"], a["K"], a["V"], a["scale"], a["dtype"],
                                  None)


@pytest.mark.parametrize("bad,rc", [
    (dict(state=None), kda.KDA_ERR_INVALID),
    (dict(q=None), kda.KDA_ERR_INVALID),
    (dict(H=0), kda.KDA_ERR_INVALID),
    (dict(HV=6, H=4), kda.KDA_ERR_INVALID),
    (dict(scale=float("nan")), kda.KDA_ERR_INVALID),
    (dict(dtype=5), kda.KDA_ERR_INVALID),
    (dict(state=ctypes.c_void_p(0x1004)), kda.KDA_ERR_INVALID),  # state not 16-byte aligned
    (dict(V=62), kda.KDA_ERR_UNSUPPORTED),
    (dict(K=129), kda.KDA_ERR_UNSUPPORTED),
])
def test_recurrent_step_rejects_invalid_arguments(lib, bad, rc):
    assert _step(lib, **bad) == rc


def test_binding_fails_loudly_without_a_gpu_tensor():
    import torch
    x = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kda.kda_chunk_fwd(x, x, x, x, torch.zeros(1, 64, 1, dtype=torch.bfloat16))


def _chunk_ex(lib, flags, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, sT=None, o=FAKE, B=2, T=64, H=2,
             HV=4, K=64, V=64, scale=0.125, chunk=64, dtype=1)
    a.update(kw)
    return lib.kda_chunk_fwd_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["sT"],
                                a["o"], a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"],
                                a["scale"], a["chunk"], a["dtype"], a.get("ws"),
                                a.get("ws_bytes", 0), flags, None)


def test_flag_constants_match_header():
    text = open(HEADER).read()
    assert re.search(r"KDA_FLAG_QK_L2NORM\s*=\s*%d" % kda.KDA_FLAG_QK_L2NORM, text)
    assert re.search(r"KDA_FLAG_BETA_SIGMOID\s*=\s*%d" % kda.KDA_FLAG_BETA_SIGMOID, text)


@pytest.mark.parametrize("flags,kw,rc", [
    (4, {}, kda.KDA_ERR_INVALID),                         # unknown flag bit
    (0x80000000, {}, kda.KDA_ERR_INVALID),
    (1, dict(dtype=0), kda.KDA_ERR_UNSUPPORTED),          # fp32 has no transform path
    (2, {}, kda.KDA_ERR_UNSUPPORTED),                     # bf16 without a workspace
    (3, dict(V=36), kda.KDA_ERR_UNSUPPORTED),             # V % 8 != 0: fused kernel only
    (1, dict(q=None), kda.KDA_ERR_INVALID),               # validation order: pointers first
])
def test_chunk_fwd_ex_rejects_unsupported_flags(lib, flags, kw, rc):
    assert _chunk_ex(lib, flags, **kw) == rc


@pytest.mark.parametrize("flags,kw,rc", [
    (4, {}, kda.KDA_ERR_INVALID),
    (8, dict(dtype=0), kda.KDA_ERR_INVALID),
    (3, dict(V=62), kda.KDA_ERR_UNSUPPORTED),
    (1, dict(state=None), kda.KDA_ERR_INVALID),
])
def test_recurrent_step_ex_rejects_invalid_arguments(lib, flags, kw, rc):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, o=FAKE, B=2, H=2, HV=4, K=64,
             V=64, scale=0.125, dtype=1)
    a.update(kw)
    assert lib.kda_recurrent_step_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"],
                                     a["o"], a["B"], a["H"], a["HV"], a["K"], a["V"], a["scale"],
                                     a["dtype"], flags, None) == rc


def _bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, do=FAKE, dht=None, dq=FAKE,
             dk=FAKE, dv=FAKE, dg=FAKE, dbeta=FAKE, dh0=None, B=2, T=64, H=2, HV=4, K=64, V=64,
             scale=0.125, chunk=64, dtype=1, ws=ctypes.c_void_p(0x100000), ws_bytes=1 << 40)
    a.update(kw)
    return lib.kda_chunk_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["do"],
                             a["dht"], a["dq"], a["dk"], a["dv"], a["dg"], a["dbeta"], a["dh0"],
                             a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"], a["scale"],
                             a["chunk"], a["dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("bad,rc", [
    (dict(q=None), kda.KDA_ERR_INVALID),
    (dict(do=None), kda.KDA_ERR_INVALID),
    (dict(dbeta=None), kda.KDA_ERR_INVALID),
    (dict(T=72), kda.KDA_ERR_INVALID),                 # T % chunk != 0
    (dict(HV=3), kda.KDA_ERR_INVALID),
    (dict(scale=float("nan")), kda.KDA_ERR_INVALID),
    (dict(ws=None), kda.KDA_ERR_INVALID),              # the backward always needs a workspace
    (dict(ws_bytes=4096), kda.KDA_ERR_INVALID),
    (dict(ws=ctypes.c_void_p(0x100010)), kda.KDA_ERR_INVALID),
    (dict(dtype=0), kda.KDA_ERR_UNSUPPORTED),           # bf16 only
    (dict(K=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(V=40), kda.KDA_ERR_UNSUPPORTED),
    (dict(V=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(q=ctypes.c_void_p(0x1008)), kda.KDA_ERR_UNSUPPORTED),  # not 16-byte aligned
    (dict(dq=ctypes.c_void_p(0x1008)), kda.KDA_ERR_UNSUPPORTED),  # dq, dk: 16-byte row stores
    (dict(dk=ctypes.c_void_p(0x1002)), kda.KDA_ERR_UNSUPPORTED),
    (dict(dg=ctypes.c_void_p(0x1004)), kda.KDA_ERR_UNSUPPORTED),
])
def test_chunk_bwd_rejects_invalid_arguments(lib, bad, rc):
    assert _bwd(lib, **bad) == rc


def test_bwd_workspace_size(lib):
    ws = lib.kda_chunk_bwd_workspace_size
    small = ws(1, 64, 1, 1, 64, 64, 64, 1)
    assert small > 0 and small % 256 == 0
    assert ws(2, 64, 1, 1, 64, 64, 64, 1) > small
    assert ws(1, 72, 1, 1, 64, 64, 8, 1) > small     # a partial second 64-token chunk
    assert ws(1, 64, 1, 2, 64, 64, 64, 1) > 2 * small  # GVA adds fp32 dq / dk buffers
    assert ws(1, 64, 1, 1, 64, 64, 64, 0) == 0        # fp32: no backward
    assert ws(1, 64, 1, 1, 48, 64, 64, 1) == 0
    assert ws(1, 72, 1, 1, 64, 64, 64, 1) == 0        # T % chunk != 0


def _varlen(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, N=2, s0=None, sT=None, o=FAKE,
             T=128, H=2, HV=4, K=64, V=64, scale=0.125, dtype=1, ws=ctypes.c_void_p(0x100000),
             ws_bytes=1 << 40, flags=0)
    a.update(kw)
    return lib.kda_chunk_fwd_varlen(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"],
                                    a["s0"], a["sT"], a["o"], a["T"], a["H"], a["HV"], a["K"],
                                    a["V"], a["scale"], a["dtype"], a["ws"], a["ws_bytes"],
                                    a["flags"], None)


@pytest.mark.parametrize("bad,rc", [
    (dict(cu=None), kda.KDA_ERR_INVALID),
    (dict(o=None), kda.KDA_ERR_INVALID),
    (dict(N=0), kda.KDA_ERR_INVALID),
    (dict(T=0), kda.KDA_ERR_INVALID),
    (dict(HV=3), kda.KDA_ERR_INVALID),
    (dict(flags=4), kda.KDA_ERR_INVALID),
    (dict(ws=None), kda.KDA_ERR_INVALID),
    (dict(ws_bytes=1024), kda.KDA_ERR_INVALID),
    (dict(ws=ctypes.c_void_p(0x100080)), kda.KDA_ERR_INVALID),
    (dict(dtype=0), kda.KDA_ERR_UNSUPPORTED),           # the two-kernel bf16 path only
    (dict(K=60), kda.KDA_ERR_UNSUPPORTED),
    (dict(V=36), kda.KDA_ERR_UNSUPPORTED),
    (dict(K=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(g=ctypes.c_void_p(0x1004)), kda.KDA_ERR_UNSUPPORTED),
])
def test_chunk_fwd_varlen_rejects_invalid_arguments(lib, bad, rc):
    assert _varlen(lib, **bad) == rc


def test_varlen_workspace_size(lib):
    ws = lib.kda_chunk_fwd_varlen_workspace_size
    one = ws(1, 64, 1, 1, 64, 64, 1)
    assert one > 0 and one % 256 == 0
    assert ws(2, 64, 1, 1, 64, 64, 1) > one        # one more possible partial chunk
    assert ws(1, 128, 1, 1, 64, 64, 1) > one
    assert ws(1, 64, 1, 1, 64, 64, 0) == 0         # fp32: no varlen path
    assert ws(1, 64, 1, 1, 60, 64, 1) == 0


@pytest.mark.parametrize("bad,rc", [
    (dict(slots=None), kda.KDA_ERR_INVALID),
    (dict(num_slots=0), kda.KDA_ERR_INVALID),
    (dict(state=None), kda.KDA_ERR_INVALID),
    (dict(flags=8), kda.KDA_ERR_INVALID),
    (dict(V=62), kda.KDA_ERR_UNSUPPORTED),
])
def test_recurrent_step_slots_rejects_invalid_arguments(lib, bad, rc):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, slots=FAKE, num_slots=4,
             o=FAKE, B=2, H=2, HV=4, K=64, V=64, scale=0.125, dtype=1, flags=0)
    a.update(bad)
    assert lib.kda_recurrent_step_slots(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"],
                                        a["slots"], a["num_slots"], a["o"], a["B"], a["H"],
                                        a["HV"], a["K"], a["V"], a["scale"], a["dtype"],
                                        a["flags"], None) == rc


def test_chunk_bwd_ex_rejects_unknown_flags(lib):
    assert lib.kda_chunk_bwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
                                FAKE, FAKE, None, 2, 64, 2, 4, 64, 64, 0.125, 64, 1,
                                ctypes.c_void_p(0x100000), 1 << 40, 4, None) == kda.KDA_ERR_INVALID
    assert lib.kda_chunk_bwd_workspace_size_ex(2, 64, 2, 4, 64, 64, 64, 1, 4) == 0
    # the q/k normalisation needs fp32 per-value-head dq / dk even without GVA
    assert (lib.kda_chunk_bwd_workspace_size_ex(1, 64, 1, 1, 64, 64, 64, 1, 1)
            > lib.kda_chunk_bwd_workspace_size_ex(1, 64, 1, 1, 64, 64, 64, 1, 0))


def _gate(lib, bwd=False, **kw):
    a = dict(x=FAKE, A_log=FAKE, dt_bias=None, g=FAKE, dg=FAKE, dx=FAKE, B=2, T=64, HV=4, K=64,
             lb=-5.0, dtype=1, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    if not bwd:
        return lib.kda_gate_fwd(a["x"], a["A_log"], a["dt_bias"], a["g"], a["B"], a["T"], a["HV"],
                                a["K"], a["lb"], a["dtype"], None)
    return lib.kda_gate_bwd(a["x"], a["A_log"], a["dt_bias"], a["dg"], a["dx"], None, None,
                            a["B"], a["T"], a["HV"], a["K"], a["lb"], a["dtype"], a["ws"],
                            a["ws_bytes"], None)


@pytest.mark.parametrize("bwd", [False, True])
@pytest.mark.parametrize("bad,rc", [
    (dict(x=None), kda.KDA_ERR_INVALID),
    (dict(A_log=None), kda.KDA_ERR_INVALID),
    (dict(B=-1), kda.KDA_ERR_INVALID),
    (dict(HV=0), kda.KDA_ERR_INVALID),
    (dict(K=0), kda.KDA_ERR_INVALID),
    (dict(lb=float("nan")), kda.KDA_ERR_INVALID),
    (dict(lb=0.5), kda.KDA_ERR_INVALID),          # a positive bound would make g grow the state
    (dict(dtype=2), kda.KDA_ERR_INVALID),
    (dict(K=12), kda.KDA_ERR_UNSUPPORTED),        # bf16 needs K % 8 == 0
    (dict(K=6, dtype=0), kda.KDA_ERR_UNSUPPORTED),  # float32 needs K % 4 == 0
    (dict(x=ctypes.c_void_p(0x1008)), kda.KDA_ERR_UNSUPPORTED),  # not 16-byte aligned
])
def test_gate_rejects_invalid_arguments(lib, bwd, bad, rc):
    assert _gate(lib, bwd, **bad) == rc


@pytest.mark.parametrize("bad,rc", [
    (dict(g=None), kda.KDA_ERR_INVALID),
])
def test_gate_fwd_rejects_missing_output(lib, bad, rc):
    assert _gate(lib, False, **bad) == rc


@pytest.mark.parametrize("bad,rc", [
    (dict(dg=None), kda.KDA_ERR_INVALID),
    (dict(dx=None), kda.KDA_ERR_INVALID),
    (dict(ws=None), kda.KDA_ERR_INVALID),
    (dict(ws_bytes=1024), kda.KDA_ERR_INVALID),            # workspace too small
    (dict(ws=ctypes.c_void_p(0x1010)), kda.KDA_ERR_INVALID),  # misaligned
    (dict(dx=ctypes.c_void_p(0x1008)), kda.KDA_ERR_UNSUPPORTED),
])
def test_gate_bwd_rejects_invalid_arguments(lib, bad, rc):
    assert _gate(lib, True, **bad) == rc


def test_gate_empty_input_needs_no_launch(lib):
    assert _gate(lib, False, B=0) == kda.KDA_OK
    assert _gate(lib, False, T=0) == kda.KDA_OK


def test_gate_bwd_workspace_size(lib):
    ws = lib.kda_gate_bwd_workspace_size
    assert ws(0, 64, 4, 64, 1) == 0
    assert ws(2, 64, 0, 64, 1) == 0          # invalid arguments
    assert ws(2, 64, 4, 12, 1) == 0          # unsupported K
    big = ws(4, 8192, 16, 128, 1)
    assert big % 256 == 0 and 0 < big <= 16 << 20   # partial sums stay small next to the tensors
    assert ws(4, 8192, 16, 128, 0) > 0


def test_gate_empty_input_accepts_null_token_tensors(lib):
    assert _gate(lib, False, B=0, x=None, g=None) == kda.KDA_OK
    assert _gate(lib, False, B=0, A_log=None) == kda.KDA_ERR_INVALID


def _gated_chunk(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, x=FAKE, A_log=FAKE, dt_bias=None, lb=-5.0, beta=FAKE,
             s0=None, sT=None, o=FAKE, B=2, T=128, H=2, HV=4, K=64, V=64, scale=0.125, chunk=64,
             dtype=1, ws=FAKE, ws_bytes=1 << 30, flags=0)
    a.update(kw)
    return lib.kda_chunk_fwd_gated(a["q"], a["k"], a["v"], a["x"], a["A_log"], a["dt_bias"],
                                   a["lb"], a["beta"], a["s0"], a["sT"], a["o"], a["B"], a["T"],
                                   a["H"], a["HV"], a["K"], a["V"], a["scale"], a["chunk"],
                                   a["dtype"], a["ws"], a["ws_bytes"], a["flags"], None)


def _gated_step(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, x=FAKE, A_log=FAKE, dt_bias=None, lb=-5.0, beta=FAKE,
             state=FAKE, o=FAKE, B=2, H=2, HV=4, K=64, V=64, scale=0.125, dtype=1, flags=0)
    a.update(kw)
    return lib.kda_recurrent_step_gated(a["q"], a["k"], a["v"], a["x"], a["A_log"], a["dt_bias"],
                                        a["lb"], a["beta"], a["state"], a["o"], a["B"], a["H"],
                                        a["HV"], a["K"], a["V"], a["scale"], a["dtype"],
                                        a["flags"], None)


@pytest.mark.parametrize("call", [_gated_chunk, _gated_step])
@pytest.mark.parametrize("bad,rc", [
    (dict(A_log=None), kda.KDA_ERR_INVALID),
    (dict(x=None), kda.KDA_ERR_INVALID),
    (dict(lb=float("nan")), kda.KDA_ERR_INVALID),
    (dict(lb=1.0), kda.KDA_ERR_INVALID),
    (dict(flags=4), kda.KDA_ERR_INVALID),                       # not a caller flag
    (dict(dt_bias=ctypes.c_void_p(0x1004)), kda.KDA_ERR_UNSUPPORTED),  # misaligned bias
    (dict(scale=float("nan")), kda.KDA_ERR_INVALID),
])
def test_gated_entry_points_reject_invalid_arguments(lib, call, bad, rc):
    assert call(lib, **bad) == rc


@pytest.mark.parametrize("bad,rc", [
    (dict(ws=None), kda.KDA_ERR_UNSUPPORTED),      # the gate needs the two-kernel path
    (dict(dtype=0, K=32, V=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(K=60), kda.KDA_ERR_UNSUPPORTED),
    (dict(T=100), kda.KDA_ERR_INVALID),            # T % chunk_size != 0
])
def test_gated_chunk_needs_the_two_kernel_path(lib, bad, rc):
    assert _gated_chunk(lib, **bad) == rc


def test_ex_entry_points_reject_the_internal_gate_flag(lib):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, o=FAKE)
    assert lib.kda_recurrent_step_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"],
                                     a["o"], 2, 2, 4, 64, 64, 0.125, 1, 4, None) == kda.KDA_ERR_INVALID
    assert lib.kda_chunk_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 2, 128, 2, 4, 64,
                                64, 0.125, 64, 1, FAKE, 1 << 30, 4, None) == kda.KDA_ERR_INVALID


def _segmented(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, sT=None, o=FAKE, B=1, T=1024,
             H=2, HV=2, K=128, V=128, scale=0.125, segments=4, dtype=1, ws=FAKE, ws_bytes=1 << 30,
             flags=0)
    a.update(kw)
    return lib.kda_chunk_fwd_segmented(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["sT"],
                                       a["o"], a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"],
                                       a["scale"], a["segments"], a["dtype"], a["ws"],
                                       a["ws_bytes"], a["flags"], None)


@pytest.mark.parametrize("bad,rc", [
    (dict(q=None), kda.KDA_ERR_INVALID),
    (dict(segments=0), kda.KDA_ERR_INVALID),
    (dict(segments=3), kda.KDA_ERR_INVALID),       # 1024 is not a multiple of 64 * 3
    (dict(T=1000), kda.KDA_ERR_INVALID),
    (dict(ws=None), kda.KDA_ERR_INVALID),
    (dict(ws_bytes=4096), kda.KDA_ERR_INVALID),
    (dict(ws=ctypes.c_void_p(0x1010)), kda.KDA_ERR_INVALID),
    (dict(flags=4), kda.KDA_ERR_INVALID),
    (dict(dtype=0, K=64, V=64), kda.KDA_ERR_UNSUPPORTED),
    (dict(K=60), kda.KDA_ERR_UNSUPPORTED),
    (dict(g=ctypes.c_void_p(0x1008)), kda.KDA_ERR_UNSUPPORTED),
])
def test_segmented_rejects_invalid_arguments(lib, bad, rc):
    assert _segmented(lib, **bad) == rc


def test_segmented_workspace_sizes(lib):
    ws = lib.kda_chunk_fwd_segmented_workspace_size
    plain = ws(1, 4096, 2, 2, 128, 128, 1, 1)
    assert plain == 1 * 2 * (4096 // 64) * lib.kda_chunk_fwd_workspace_size(1, 64, 1, 1, 128, 128, 64, 1)
    seg = ws(1, 4096, 2, 2, 128, 128, 16, 1)
    # the same factor blocks plus, per segment and head, the maps [Bm | A] (K x (V + K)) and
    # S_in (K x V) in fp32
    assert seg == plain + 16 * 2 * 128 * (2 * 128 + 128) * 4
    plain64 = ws(1, 4096, 2, 2, 64, 128, 1, 1)
    assert ws(1, 4096, 2, 2, 64, 128, 8, 1) == plain64 + 8 * 2 * 64 * (2 * 128 + 64) * 4
    assert ws(1, 4096, 2, 2, 128, 128, 3, 1) == 0     # 4096 is not a multiple of 64 * 3
    assert ws(1, 4096, 2, 2, 128, 128, 16, 0) == 0    # bf16 only


@pytest.mark.parametrize("HV,segments", [(2, 16), (4, 16), (8, 8), (16, 4), (32, 1), (64, 1)])
def test_automatic_segment_count(lib, HV, segments):
    # B = 1, T = 4096 (64 chunks), K = V = 128: the largest power of two P with
    # P * HV * ceil(V / 32) <= 256, at least 4 chunks per segment, taken from P = 4 on
    auto = lib.kda_chunk_fwd_workspace_size(1, 4096, HV, HV, 128, 128, 64, 1)
    assert auto == lib.kda_chunk_fwd_segmented_workspace_size(1, 4096, HV, HV, 128, 128, segments, 1)


def _noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, sT=None, o=FAKE, B=2, T=64, H=2,
             HV=4, K=64, V=64, scale=0.125, chunk=64, dtype=1, flags=0)
    a.update(kw)
    return lib.kda_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["sT"],
                                     a["o"], a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"],
                                     a["scale"], a["chunk"], a["dtype"], a["flags"], None)


def test_noalloc_scratch_constant_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define KDA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == kda.NOALLOC_SCRATCH_BYTES
    assert re.search(r"KDA_ERR_SCRATCH = (-\d+)", text).group(1) == str(kda.KDA_ERR_SCRATCH)


@pytest.mark.parametrize("bad,rc", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(T=0), -1), (dict(chunk=48), -1),
    (dict(T=100), -1), (dict(HV=3), -1), (dict(scale=float("nan")), -1), (dict(flags=4), -1),
    (dict(K=256), -2),
    # B4 T8192 H16 K=V=128 needs 512 MB of workspace: more than the fixed array, rejected
    # before any HIP call
    (dict(B=4, T=8192, H=16, HV=16, K=128, V=128), -4),
    # B1 T32768 H4 would take the segmented route (140 MB) and its plain path needs 128 MB
    (dict(B=1, T=32768, H=4, HV=4, K=128, V=128), -4),
])
def test_noalloc_rejects_before_any_launch(lib, bad, rc):
    assert _noalloc(lib, **bad) == rc
    assert "scratch" in kda.status_string(kda.KDA_ERR_SCRATCH)


@pytest.mark.parametrize("src,dst,nbytes", [
    (None, ctypes.c_void_p(0x2000), 64),                     # null source
    (ctypes.c_void_p(0x1000), None, 64),                     # null destination
    (ctypes.c_void_p(0x1000), ctypes.c_void_p(0x100000), 24),  # not a multiple of 16 bytes
    (ctypes.c_void_p(0x1008), ctypes.c_void_p(0x100000), 64),  # misaligned source
    (ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1020), 64),    # overlapping ranges
])
def test_stream_copy_rejects_invalid_arguments(lib, src, dst, nbytes):
    # every call fails validation before anything is enqueued (the pointers are never touched)
    assert lib.kda_stream_copy(src, dst, nbytes, None) == kda.KDA_ERR_INVALID


def test_stream_copy_of_nothing_is_ok(lib):
    assert lib.kda_stream_copy(None, None, 0, None) == kda.KDA_OK
