"""MI355X-native Kimi Delta Attention (KDA) forward: Python binding of libkda.so.

The binding only marshals arguments: it checks devices, dtypes, shapes and
contiguity, allocates outputs with torch (device memory and streams are all
torch is used for) and calls the C ABI declared in ``include/kda.h``. Every step
of the computation runs in the HIP kernels. There is no CPU or PyTorch fallback:
if ``libkda.so`` is missing or a call fails, an error is raised.

Entry points (same names as the C ABI):

* ``kda_chunk_fwd(q, k, v, g, beta, scale=None, initial_state=None,
  output_final_state=True, chunk_size=64, qk_l2norm=False, beta_sigmoid=False)
  -> (o, final_state)``
* ``kda_recurrent_step(q, k, v, g, beta, state, scale=None, qk_l2norm=False,
  beta_sigmoid=False) -> o`` (updates ``state`` in place)
* ``kda_gate_fwd(x, A_log, dt_bias=None, lower_bound=None) -> g`` and
  ``kda_gate_bwd(x, A_log, dt_bias, dg, lower_bound=None) -> (dx, dA_log, ddt_bias)``:
  the decay gate that produces g, and its backward
* ``kda_chunk_fwd_gated`` / ``kda_recurrent_step_gated``: the prefill and the decode step
  with that gate applied inside the kernels (the gate's input in place of g)
* ``kda_chunk_fwd_segmented(q, k, v, g, beta, segments, ...)``: the prefill over segments
  of each sequence composed by a scan (for few heads)
* ``kda_chunk_fwd_noalloc(q, k, v, g, beta, o, final_state=None, ...)``: the prefill into
  caller-provided outputs, with the workspace taken from the library's fixed per-device
  scratch array (no device allocation anywhere in the call)

``qk_l2norm`` / ``beta_sigmoid`` ask the kernels to L2-normalise q and k and to
apply the sigmoid to beta (``kda_chunk_fwd_ex`` / ``kda_recurrent_step_ex``).
"""

import ctypes
import math
import os

import torch

__all__ = ["kda_chunk_fwd", "kda_chunk_fwd_varlen", "kda_chunk_bwd",
           "kda_chunk_bwd_varlen", "kda_recurrent_step",
           "kda_recurrent_step_slots", "kda_gate_fwd", "kda_gate_bwd",
           "kda_chunk_fwd_gated", "kda_recurrent_step_gated", "kda_chunk_fwd_segmented",
           "kda_chunk_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "library", "library_path", "status_string",
           "KDA_OK", "KDA_ERR_INVALID", "KDA_ERR_UNSUPPORTED", "KDA_ERR_HIP", "KDA_ERR_SCRATCH",
           "KDA_FLAG_QK_L2NORM", "KDA_FLAG_BETA_SIGMOID"]

KDA_OK, KDA_ERR_INVALID, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP, KDA_ERR_SCRATCH = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 64 << 20  # KDA_NOALLOC_SCRATCH_BYTES
KDA_FLAG_QK_L2NORM, KDA_FLAG_BETA_SIGMOID = 1, 2
_DTYPE = {torch.float32: 0, torch.bfloat16: 1}

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")
_lib = None


def library():
    """Load libkda.so (once) and declare its C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is not built; run `python -m gated_delta_rule_67_amd.build`")
    lib = ctypes.CDLL(library_path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.kda_chunk_fwd.argtypes = [vp] * 8 + [i] * 6 + [f, i, i, vp, sz, vp]
    lib.kda_chunk_fwd.restype = i
    lib.kda_chunk_fwd_ex.argtypes = [vp] * 8 + [i] * 6 + [f, i, i, vp, sz, ctypes.c_uint, vp]
    lib.kda_chunk_fwd_ex.restype = i
    lib.kda_chunk_fwd_workspace_size.argtypes = [i] * 8
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd_varlen.argtypes = [vp] * 6 + [i] + [vp] * 3 + [i] * 5 + [f, i, vp, sz,
                                                                            ctypes.c_uint, vp]
    lib.kda_chunk_fwd_varlen.restype = i
    lib.kda_chunk_fwd_varlen_workspace_size.argtypes = [i] * 7
    lib.kda_chunk_fwd_varlen_workspace_size.restype = sz
    u = ctypes.c_uint
    lib.kda_chunk_bwd.argtypes = [vp] * 14 + [i] * 6 + [f, i, i, vp, sz, vp]
    lib.kda_chunk_bwd_ex.argtypes = [vp] * 14 + [i] * 6 + [f, i, i, vp, sz, u, vp]
    lib.kda_chunk_bwd_ex.restype = i
    lib.kda_chunk_bwd_workspace_size_ex.argtypes = [i] * 8 + [u]
    lib.kda_chunk_bwd_workspace_size_ex.restype = sz
    lib.kda_chunk_bwd_varlen.argtypes = [vp] * 6 + [i] + [vp] * 9 + [i] * 5 + [f, i, vp, sz, u, vp]
    lib.kda_chunk_bwd_varlen.restype = i
    lib.kda_chunk_bwd_varlen_workspace_size.argtypes = [i] * 7 + [u]
    lib.kda_chunk_bwd_varlen_workspace_size.restype = sz
    lib.kda_chunk_bwd.restype = i
    lib.kda_chunk_bwd_workspace_size.argtypes = [i] * 8
    lib.kda_chunk_bwd_workspace_size.restype = sz
    lib.kda_recurrent_step.argtypes = [vp] * 7 + [i] * 5 + [f, i, vp]
    lib.kda_recurrent_step.restype = i
    lib.kda_recurrent_step_ex.argtypes = [vp] * 7 + [i] * 5 + [f, i, ctypes.c_uint, vp]
    lib.kda_recurrent_step_ex.restype = i
    lib.kda_recurrent_step_slots.argtypes = [vp] * 7 + [i, vp] + [i] * 5 + [f, i, ctypes.c_uint, vp]
    lib.kda_recurrent_step_slots.restype = i
    lib.kda_gate_fwd.argtypes = [vp] * 4 + [i] * 4 + [f, i, vp]
    lib.kda_gate_fwd.restype = i
    lib.kda_gate_bwd_workspace_size.argtypes = [i] * 5
    lib.kda_gate_bwd_workspace_size.restype = sz
    lib.kda_gate_bwd.argtypes = [vp] * 7 + [i] * 4 + [f, i, vp, sz, vp]
    lib.kda_gate_bwd.restype = i
    lib.kda_chunk_fwd_gated.argtypes = [vp] * 6 + [f] + [vp] * 4 + [i] * 6 + [f, i, i, vp, sz,
                                                                            ctypes.c_uint, vp]
    lib.kda_chunk_fwd_gated.restype = i
    lib.kda_recurrent_step_gated.argtypes = [vp] * 6 + [f] + [vp] * 3 + [i] * 5 + [f, i,
                                                                                 ctypes.c_uint, vp]
    lib.kda_recurrent_step_gated.restype = i
    lib.kda_chunk_fwd_segmented.argtypes = [vp] * 8 + [i] * 6 + [f, i, i, vp, sz, ctypes.c_uint, vp]
    lib.kda_chunk_fwd_segmented.restype = i
    lib.kda_chunk_fwd_segmented_workspace_size.argtypes = [i] * 8
    lib.kda_chunk_fwd_segmented_workspace_size.restype = sz
    lib.kda_chunk_fwd_noalloc.argtypes = [vp] * 8 + [i] * 6 + [f, i, i, ctypes.c_uint, vp]
    lib.kda_chunk_fwd_noalloc.restype = i
    lib.kda_stream_copy.argtypes = [vp, vp, sz, vp]
    lib.kda_stream_copy.restype = i
    lib.kda_status_string.argtypes = [i]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(rc):
    return library().kda_status_string(int(rc)).decode()


def _check(rc):
    if rc != KDA_OK:
        raise RuntimeError(status_string(rc))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_tensors(named, dtype, device):
    for name, t in named:
        _require(t.device == device, f"{name} is on {t.device}, expected {device}")
        _require(t.dtype == dtype, f"{name} has dtype {t.dtype}, expected {dtype}")
        _require(t.is_contiguous(), f"{name} must be contiguous")


def _flags(qk_l2norm, beta_sigmoid):
    return (KDA_FLAG_QK_L2NORM if qk_l2norm else 0) | (KDA_FLAG_BETA_SIGMOID if beta_sigmoid else 0)


def kda_chunk_fwd(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=True,
                  chunk_size=64, qk_l2norm=False, beta_sigmoid=False):
    """Chunked KDA prefill. q, k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV,K]; beta [B,T,HV];
    initial_state [B,HV,K,V] float32 or None. Returns (o [B,T,HV,V], final_state or None).
    qk_l2norm / beta_sigmoid: apply those input transforms in the kernels."""
    _require(q.is_cuda, "inputs must be on a GPU")
    dev, dt = q.device, q.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    _require(k.shape == q.shape, "k must match q")
    _require(tuple(v.shape[:2]) == (B, T), "v must be [B, T, HV, V]")
    _require(tuple(g.shape) == (B, T, HV, K), "g must be [B, T, HV, K]")
    _require(tuple(beta.shape) == (B, T, HV), "beta must be [B, T, HV]")
    _check_tensors([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)], dt, dev)
    if initial_state is not None:
        _require(tuple(initial_state.shape) == (B, HV, K, V), "initial_state must be [B, HV, K, V]")
        _check_tensors([("initial_state", initial_state)], torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    lib = library()
    o = torch.empty((B, T, HV, V), dtype=dt, device=dev)
    final = torch.empty((B, HV, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    ws_bytes = lib.kda_chunk_fwd_workspace_size(B, T, H, HV, K, V, chunk_size, _DTYPE[dt])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(initial_state), _ptr(final), _ptr(o), B, T, H, HV, K, V,
                                  float(scale), int(chunk_size), _DTYPE[dt], _ptr(ws), ws_bytes,
                                  _flags(qk_l2norm, beta_sigmoid), ctypes.c_void_p(stream))
    _check(rc)
    return o, final


def kda_chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, scale=None, initial_state=None,
                         output_final_state=True, qk_l2norm=False, beta_sigmoid=False):
    """Packed variable-length prefill (bf16). q, k [1,T,H,K] (or [T,H,K]); v [1,T,HV,V];
    g [1,T,HV,K]; beta [1,T,HV]; cu_seqlens int32 [N+1] on the same device; initial_state
    [N,HV,K,V] float32 or None. Returns (o shaped like v, final_state [N,HV,K,V] or None)."""
    _require(q.is_cuda, "inputs must be on a GPU")
    dev, dt = q.device, q.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    squeeze = q.dim() == 3
    if not squeeze:
        _require(q.shape[0] == 1, "packed inputs have batch size 1")
        q, k, v, g, beta = q[0], k[0], v[0], g[0], beta[0]
    T, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    _require(k.shape == q.shape, "k must match q")
    _require(v.shape[0] == T, "v must be [T, HV, V]")
    _require(tuple(g.shape) == (T, HV, K), "g must be [T, HV, K]")
    _require(tuple(beta.shape) == (T, HV), "beta must be [T, HV]")
    _check_tensors([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)], dt, dev)
    _require(cu_seqlens.is_cuda and cu_seqlens.device == dev, "cu_seqlens must be on the same GPU")
    _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1 and cu_seqlens.is_contiguous(),
             "cu_seqlens must be a contiguous int32 vector")
    N = cu_seqlens.numel() - 1
    _require(N >= 1, "cu_seqlens needs at least two offsets")
    if initial_state is not None:
        _require(tuple(initial_state.shape) == (N, HV, K, V), "initial_state must be [N, HV, K, V]")
        _check_tensors([("initial_state", initial_state)], torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    lib = library()
    o = torch.empty((T, HV, V), dtype=dt, device=dev)
    final = torch.empty((N, HV, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    ws_bytes = lib.kda_chunk_fwd_varlen_workspace_size(N, T, H, HV, K, V, _DTYPE[dt])
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(cu_seqlens), N, _ptr(initial_state), _ptr(final),
                                      _ptr(o), T, H, HV, K, V, float(scale), _DTYPE[dt], _ptr(ws),
                                      ws_bytes, _flags(qk_l2norm, beta_sigmoid),
                                      ctypes.c_void_p(stream))
    _check(rc)
    return (o if squeeze else o.unsqueeze(0)), final


def kda_chunk_bwd(q, k, v, g, beta, do, scale=None, initial_state=None, dht=None, chunk_size=64,
                  need_dh0=True, qk_l2norm=False, beta_sigmoid=False):
    """Gradients of <o, do> + <final_state, dht> for kda_chunk_fwd's inputs (bf16).
    Shapes as kda_chunk_fwd; do [B,T,HV,V]; dht [B,HV,K,V] float32 or None.
    Returns (dq, dk, dv, dg, dbeta, dh0 or None); dh0 is float32 [B,HV,K,V].
    qk_l2norm / beta_sigmoid: the forward applied those transforms; gradients are for the
    raw inputs."""
    _require(q.is_cuda, "inputs must be on a GPU")
    dev, dt = q.device, q.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    _require(k.shape == q.shape, "k must match q")
    _require(tuple(v.shape[:2]) == (B, T), "v must be [B, T, HV, V]")
    _require(tuple(g.shape) == (B, T, HV, K), "g must be [B, T, HV, K]")
    _require(tuple(beta.shape) == (B, T, HV), "beta must be [B, T, HV]")
    _require(tuple(do.shape) == (B, T, HV, V), "do must be [B, T, HV, V]")
    _check_tensors([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("do", do)], dt, dev)
    for name, t in (("initial_state", initial_state), ("dht", dht)):
        if t is not None:
            _require(tuple(t.shape) == (B, HV, K, V), f"{name} must be [B, HV, K, V]")
            _check_tensors([(name, t)], torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    lib = library()
    dq = torch.empty((B, T, H, K), dtype=dt, device=dev)
    dk = torch.empty((B, T, H, K), dtype=dt, device=dev)
    dv = torch.empty((B, T, HV, V), dtype=dt, device=dev)
    dg = torch.empty((B, T, HV, K), dtype=dt, device=dev)
    dbeta = torch.empty((B, T, HV), dtype=dt, device=dev)
    dh0 = torch.empty((B, HV, K, V), dtype=torch.float32, device=dev) if need_dh0 else None
    flags = _flags(qk_l2norm, beta_sigmoid)
    ws_bytes = lib.kda_chunk_bwd_workspace_size_ex(B, T, H, HV, K, V, chunk_size, _DTYPE[dt], flags)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_chunk_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(initial_state), _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), B, T, H, HV, K, V,
                                  float(scale), int(chunk_size), _DTYPE[dt], _ptr(ws), ws_bytes,
                                  flags, ctypes.c_void_p(stream))
    _check(rc)
    return dq, dk, dv, dg, dbeta, dh0


def kda_chunk_bwd_varlen(q, k, v, g, beta, do, cu_seqlens, scale=None, initial_state=None,
                         dht=None, need_dh0=True, qk_l2norm=False, beta_sigmoid=False):
    """Gradients for kda_chunk_fwd_varlen's inputs (bf16, packed sequences). Token tensors
    [1,T,...] (or [T,...]); cu_seqlens int32 [N+1]; initial_state, dht [N,HV,K,V] float32 or
    None. Returns (dq, dk, dv, dg, dbeta shaped like their inputs, dh0 [N,HV,K,V] or None)."""
    _require(q.is_cuda, "inputs must be on a GPU")
    dev, dt = q.device, q.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    squeeze = q.dim() == 3
    if not squeeze:
        _require(q.shape[0] == 1, "packed inputs have batch size 1")
        q, k, v, g, beta, do = q[0], k[0], v[0], g[0], beta[0], do[0]
    T, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    _require(k.shape == q.shape, "k must match q")
    _require(tuple(v.shape) == (T, HV, V) and tuple(do.shape) == (T, HV, V), "v, do must be [T, HV, V]")
    _require(tuple(g.shape) == (T, HV, K), "g must be [T, HV, K]")
    _require(tuple(beta.shape) == (T, HV), "beta must be [T, HV]")
    _check_tensors([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("do", do)], dt, dev)
    _require(cu_seqlens.is_cuda and cu_seqlens.device == dev and cu_seqlens.dtype == torch.int32
             and cu_seqlens.dim() == 1 and cu_seqlens.is_contiguous(), "cu_seqlens must be int32 on the GPU")
    N = cu_seqlens.numel() - 1
    _require(N >= 1, "cu_seqlens needs at least two offsets")
    for name, t in (("initial_state", initial_state), ("dht", dht)):
        if t is not None:
            _require(tuple(t.shape) == (N, HV, K, V), f"{name} must be [N, HV, K, V]")
            _check_tensors([(name, t)], torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    lib = library()
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    dv, dg, dbeta = torch.empty_like(v), torch.empty_like(g), torch.empty_like(beta)
    dh0 = torch.empty((N, HV, K, V), dtype=torch.float32, device=dev) if need_dh0 else None
    flags = _flags(qk_l2norm, beta_sigmoid)
    ws_bytes = lib.kda_chunk_bwd_varlen_workspace_size(N, T, H, HV, K, V, _DTYPE[dt], flags)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_chunk_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(cu_seqlens), N, _ptr(initial_state), _ptr(do),
                                      _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                      _ptr(dbeta), _ptr(dh0), T, H, HV, K, V, float(scale),
                                      _DTYPE[dt], _ptr(ws), ws_bytes, flags, ctypes.c_void_p(stream))
    _check(rc)
    outs = (dq, dk, dv, dg, dbeta)
    if not squeeze:
        outs = tuple(x.unsqueeze(0) for x in outs)
    return outs + (dh0,)


def kda_recurrent_step(q, k, v, g, beta, state, scale=None, qk_l2norm=False, beta_sigmoid=False):
    """One decode token. q, k [B,H,K] (or [B,1,H,K]); v [B,HV,V]; g [B,HV,K]; beta [B,HV];
    state [B,HV,K,V] float32, updated in place. Returns o [B,HV,V].
    qk_l2norm / beta_sigmoid: apply those input transforms in the kernel."""
    _require(q.is_cuda, "inputs must be on a GPU")
    dev, dt = q.device, q.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    if q.dim() == 4:
        q, k, v, g, beta = q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0]
    B, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    _require(k.shape == q.shape, "k must match q")
    _require(tuple(g.shape) == (B, HV, K), "g must be [B, HV, K]")
    _require(tuple(beta.shape) == (B, HV), "beta must be [B, HV]")
    _require(tuple(state.shape) == (B, HV, K, V), "state must be [B, HV, K, V]")
    _check_tensors([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)], dt, dev)
    _check_tensors([("state", state)], torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    lib = library()
    o = torch.empty((B, HV, V), dtype=dt, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_recurrent_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(state), _ptr(o), B, H, HV, K, V, float(scale),
                                       _DTYPE[dt], _flags(qk_l2norm, beta_sigmoid),
                                       ctypes.c_void_p(stream))
    _check(rc)
    return o


def kda_recurrent_step_slots(q, k, v, g, beta, state_pool, slots, scale=None, qk_l2norm=False,
                             beta_sigmoid=False):
    """One decode token per request against a slot-indexed state pool. q, k [B,H,K];
    v [B,HV,V]; g [B,HV,K]; beta [B,HV]; state_pool [num_slots,HV,K,V] float32 (updated in
    place); slots int32 [B] (a slot outside [0, num_slots) gives o = 0 and no update).
    Returns o [B,HV,V]."""
    _require(q.is_cuda, "inputs must be on a GPU")
    dev, dt = q.device, q.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    if q.dim() == 4:
        q, k, v, g, beta = q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0]
    B, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    _require(k.shape == q.shape, "k must match q")
    _require(tuple(g.shape) == (B, HV, K), "g must be [B, HV, K]")
    _require(tuple(beta.shape) == (B, HV), "beta must be [B, HV]")
    _require(state_pool.dim() == 4 and tuple(state_pool.shape[1:]) == (HV, K, V),
             "state_pool must be [num_slots, HV, K, V]")
    _check_tensors([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)], dt, dev)
    _check_tensors([("state_pool", state_pool)], torch.float32, dev)
    _require(slots.is_cuda and slots.device == dev and slots.dtype == torch.int32
             and tuple(slots.shape) == (B,) and slots.is_contiguous(), "slots must be int32 [B] on the GPU")
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    lib = library()
    o = torch.empty((B, HV, V), dtype=dt, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_recurrent_step_slots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                          _ptr(state_pool), _ptr(slots), state_pool.shape[0],
                                          _ptr(o), B, H, HV, K, V, float(scale), _DTYPE[dt],
                                          _flags(qk_l2norm, beta_sigmoid), ctypes.c_void_p(stream))
    _check(rc)
    return o


def _gate_args(x, A_log, dt_bias, lower_bound):
    _require(x.is_cuda, "inputs must be on a GPU")
    dev, dt = x.device, x.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    _require(x.dim() == 4, "x must be [B, T, HV, K]")
    B, T, HV, K = x.shape
    _check_tensors([("x", x)], dt, dev)
    _require(tuple(A_log.shape) == (HV,), "A_log must be [HV]")
    _check_tensors([("A_log", A_log)], torch.float32, dev)
    if dt_bias is not None:
        _require(dt_bias.numel() == HV * K, "dt_bias must be [HV, K]")
        _check_tensors([("dt_bias", dt_bias)], torch.float32, dev)
    lb = float("-inf") if lower_bound is None else float(lower_bound)
    return dev, dt, B, T, HV, K, lb


def kda_gate_fwd(x, A_log, dt_bias=None, lower_bound=None):
    """The KDA decay gate: g = max(lower_bound, -exp(A_log[hv]) * softplus(x + dt_bias[hv]))
    for x [B,T,HV,K] (bf16 or float32), A_log [HV] and dt_bias [HV,K] float32 (or None).
    lower_bound None is the standard gate; a number <= 0 (the pages use -5) the safe gate.
    Returns g shaped and typed like x."""
    dev, dt, B, T, HV, K, lb = _gate_args(x, A_log, dt_bias, lower_bound)
    lib = library()
    g = torch.empty_like(x)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_gate_fwd(_ptr(x), _ptr(A_log), _ptr(dt_bias), _ptr(g), B, T, HV, K, lb,
                              _DTYPE[dt], ctypes.c_void_p(stream))
    _check(rc)
    return g


def kda_gate_bwd(x, A_log, dt_bias, dg, lower_bound=None):
    """Backward of kda_gate_fwd for the gradient dg reaching g. Returns (dx like x,
    dA_log [HV] float32, ddt_bias [HV,K] float32)."""
    dev, dt, B, T, HV, K, lb = _gate_args(x, A_log, dt_bias, lower_bound)
    _require(dg.shape == x.shape, "dg must match x")
    _check_tensors([("dg", dg)], dt, dev)
    lib = library()
    dx = torch.empty_like(x)
    dA_log = torch.empty((HV,), dtype=torch.float32, device=dev)
    ddt_bias = torch.empty((HV, K), dtype=torch.float32, device=dev)
    ws_bytes = lib.kda_gate_bwd_workspace_size(B, T, HV, K, _DTYPE[dt])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_gate_bwd(_ptr(x), _ptr(A_log), _ptr(dt_bias), _ptr(dg), _ptr(dx),
                              _ptr(dA_log), _ptr(ddt_bias), B, T, HV, K, lb, _DTYPE[dt],
                              _ptr(ws), ws_bytes, ctypes.c_void_p(stream))
    _check(rc)
    return dx, dA_log, ddt_bias


def _gate_params(A_log, dt_bias, lower_bound, HV, K, dev):
    _require(tuple(A_log.shape) == (HV,), "A_log must be [HV]")
    _check_tensors([("A_log", A_log)], torch.float32, dev)
    if dt_bias is not None:
        _require(dt_bias.numel() == HV * K, "dt_bias must be [HV, K]")
        _check_tensors([("dt_bias", dt_bias)], torch.float32, dev)
    return float("-inf") if lower_bound is None else float(lower_bound)


def kda_chunk_fwd_gated(q, k, v, gate_x, A_log, dt_bias, beta, lower_bound=-5.0, scale=None,
                        initial_state=None, output_final_state=True, chunk_size=64,
                        qk_l2norm=False, beta_sigmoid=False):
    """kda_chunk_fwd with the decay gate applied in the kernels: gate_x [B,T,HV,K] (bf16) is
    the gate's input; g = max(lower_bound, -exp(A_log) softplus(gate_x + dt_bias)), rounded
    to bf16 as kda_gate_fwd stores it. lower_bound None: the standard gate.
    Returns (o, final_state)."""
    _require(q.is_cuda, "inputs must be on a GPU")
    dev, dt = q.device, q.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    _require(k.shape == q.shape, "k must match q")
    _require(tuple(v.shape[:2]) == (B, T), "v must be [B, T, HV, V]")
    _require(tuple(gate_x.shape) == (B, T, HV, K), "gate_x must be [B, T, HV, K]")
    _require(tuple(beta.shape) == (B, T, HV), "beta must be [B, T, HV]")
    _check_tensors([("q", q), ("k", k), ("v", v), ("gate_x", gate_x), ("beta", beta)], dt, dev)
    lb = _gate_params(A_log, dt_bias, lower_bound, HV, K, dev)
    if initial_state is not None:
        _require(tuple(initial_state.shape) == (B, HV, K, V), "initial_state must be [B, HV, K, V]")
        _check_tensors([("initial_state", initial_state)], torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    lib = library()
    o = torch.empty((B, T, HV, V), dtype=dt, device=dev)
    final = torch.empty((B, HV, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    ws_bytes = lib.kda_chunk_fwd_workspace_size(B, T, H, HV, K, V, chunk_size, _DTYPE[dt])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(gate_x), _ptr(A_log),
                                     _ptr(dt_bias), lb, _ptr(beta), _ptr(initial_state),
                                     _ptr(final), _ptr(o), B, T, H, HV, K, V, float(scale),
                                     int(chunk_size), _DTYPE[dt], _ptr(ws), ws_bytes,
                                     _flags(qk_l2norm, beta_sigmoid), ctypes.c_void_p(stream))
    _check(rc)
    return o, final


def kda_recurrent_step_gated(q, k, v, gate_x, A_log, dt_bias, beta, state, lower_bound=-5.0,
                             scale=None, qk_l2norm=False, beta_sigmoid=False):
    """kda_recurrent_step with the decay gate applied in the kernel: gate_x [B,HV,K] is the
    gate's input (as kda_chunk_fwd_gated). Updates state in place; returns o [B,HV,V]."""
    _require(q.is_cuda, "inputs must be on a GPU")
    dev, dt = q.device, q.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    if q.dim() == 4:
        q, k, v, gate_x, beta = q[:, 0], k[:, 0], v[:, 0], gate_x[:, 0], beta[:, 0]
    B, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    _require(k.shape == q.shape, "k must match q")
    _require(tuple(gate_x.shape) == (B, HV, K), "gate_x must be [B, HV, K]")
    _require(tuple(beta.shape) == (B, HV), "beta must be [B, HV]")
    _require(tuple(state.shape) == (B, HV, K, V), "state must be [B, HV, K, V]")
    _check_tensors([("q", q), ("k", k), ("v", v), ("gate_x", gate_x), ("beta", beta)], dt, dev)
    _check_tensors([("state", state)], torch.float32, dev)
    lb = _gate_params(A_log, dt_bias, lower_bound, HV, K, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    lib = library()
    o = torch.empty((B, HV, V), dtype=dt, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_recurrent_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(gate_x), _ptr(A_log),
                                          _ptr(dt_bias), lb, _ptr(beta), _ptr(state), _ptr(o), B,
                                          H, HV, K, V, float(scale), _DTYPE[dt],
                                          _flags(qk_l2norm, beta_sigmoid), ctypes.c_void_p(stream))
    _check(rc)
    return o


def kda_chunk_fwd_segmented(q, k, v, g, beta, segments, scale=None, initial_state=None,
                            output_final_state=True, qk_l2norm=False, beta_sigmoid=False):
    """kda_chunk_fwd over `segments` equal segments of each sequence, composed by a scan of the
    segments' affine state maps (bf16; T % (64 * segments) == 0). kda_chunk_fwd takes this
    route by itself when it pays; this entry point chooses the segment count explicitly.
    Returns (o, final_state)."""
    _require(q.is_cuda, "inputs must be on a GPU")
    dev, dt = q.device, q.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    _require(k.shape == q.shape, "k must match q")
    _require(tuple(v.shape[:2]) == (B, T), "v must be [B, T, HV, V]")
    _require(tuple(g.shape) == (B, T, HV, K), "g must be [B, T, HV, K]")
    _require(tuple(beta.shape) == (B, T, HV), "beta must be [B, T, HV]")
    _check_tensors([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)], dt, dev)
    if initial_state is not None:
        _require(tuple(initial_state.shape) == (B, HV, K, V), "initial_state must be [B, HV, K, V]")
        _check_tensors([("initial_state", initial_state)], torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    lib = library()
    o = torch.empty((B, T, HV, V), dtype=dt, device=dev)
    final = torch.empty((B, HV, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    ws_bytes = lib.kda_chunk_fwd_segmented_workspace_size(B, T, H, HV, K, V, int(segments), _DTYPE[dt])
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_chunk_fwd_segmented(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         _ptr(initial_state), _ptr(final), _ptr(o), B, T, H, HV,
                                         K, V, float(scale), int(segments), _DTYPE[dt], _ptr(ws),
                                         ws_bytes, _flags(qk_l2norm, beta_sigmoid),
                                         ctypes.c_void_p(stream))
    _check(rc)
    return o, final


def kda_chunk_fwd_noalloc(q, k, v, g, beta, o, final_state=None, scale=None, initial_state=None,
                          chunk_size=64, qk_l2norm=False, beta_sigmoid=False):
    """kda_chunk_fwd writing into the caller's o [B,T,HV,V] (and final_state [B,HV,K,V]
    float32, or None), with no device allocation: the library's fixed per-device scratch
    array serves as the workspace (calls overlapping on one GPU race on it). Raises on
    KDA_ERR_SCRATCH when the shape needs more than NOALLOC_SCRATCH_BYTES. Returns o."""
    _require(q.is_cuda, "inputs must be on a GPU")
    dev, dt = q.device, q.dtype
    _require(dt in _DTYPE, f"unsupported dtype {dt}")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    _require(k.shape == q.shape, "k must match q")
    _require(tuple(v.shape[:2]) == (B, T), "v must be [B, T, HV, V]")
    _require(tuple(g.shape) == (B, T, HV, K), "g must be [B, T, HV, K]")
    _require(tuple(beta.shape) == (B, T, HV), "beta must be [B, T, HV]")
    _require(tuple(o.shape) == (B, T, HV, V), "o must be [B, T, HV, V]")
    _check_tensors([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("o", o)], dt, dev)
    for name, st in (("initial_state", initial_state), ("final_state", final_state)):
        if st is not None:
            _require(tuple(st.shape) == (B, HV, K, V), f"{name} must be [B, HV, K, V]")
            _check_tensors([(name, st)], torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    lib = library()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(initial_state), _ptr(final_state), _ptr(o), B, T, H,
                                       HV, K, V, float(scale), int(chunk_size), _DTYPE[dt],
                                       _flags(qk_l2norm, beta_sigmoid), ctypes.c_void_p(stream))
    _check(rc)
    return o


def stream_copy(src, dst):
    """kda_stream_copy: copy the bytes of contiguous device tensor src into dst (same byte
    size, 16-byte aligned, not overlapping) with the library's streaming copy kernel. A
    measuring stick for HBM figures, not part of the operator."""
    _require(src.is_cuda and dst.is_cuda, "tensors must be on a GPU")
    _require(src.is_contiguous() and dst.is_contiguous(), "tensors must be contiguous")
    nbytes = src.numel() * src.element_size()
    _require(dst.numel() * dst.element_size() == nbytes, "src and dst must have the same byte size")
    with torch.cuda.device(src.device):
        stream = torch.cuda.current_stream(src.device).cuda_stream
        _check(library().kda_stream_copy(_ptr(src), _ptr(dst), nbytes, ctypes.c_void_p(stream)))
