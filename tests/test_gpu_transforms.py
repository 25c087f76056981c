"""GPU parity of the in-kernel input transforms (q/k L2 normalisation, beta sigmoid)
against the fp64 oracle applying the same transforms (``oracle.transforms``).

Inputs are the raw values a model's projections would hand over: q and k standard
normal (norms near sqrt(K), scaled by powers of two so that the normalisation has
work to do), beta as logits spread over [-8, 8]. Tolerances as for the other parity
tests: float32 decode 1e-5 max-abs, bf16 2e-2 x RMS with the per-row guard."""

import numpy as np
import pytest
import torch

import gated_delta_rule_67_amd as kda
from oracle import decode_step, recurrent
from synth import decode_inputs, prefill_inputs
from tests.helpers import assert_parity, gpu, head_slice, log, to64

pytestmark = pytest.mark.gpu


def _raw_prefill(B, T, H, HV, K, V, seed, qk_l2norm, beta_sigmoid):
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, seed, raw_qk=qk_l2norm,
                         beta="logit" if beta_sigmoid else "default")
    if qk_l2norm:  # powers of two are exact in bf16
        inp["q"] = inp["q"] * 8.0
        inp["k"] = inp["k"] * 0.25
    if beta_sigmoid:
        inp["beta"] = inp["beta"] * 4.0
    return inp


def _prefill_gpu(inp, chunk, **flags):
    d = gpu(inp)
    o, s = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                             d["initial_state"], True, chunk, **flags)
    torch.cuda.synchronize()
    return o, s


@pytest.mark.parametrize("flags", [dict(qk_l2norm=True, beta_sigmoid=True),
                                   dict(qk_l2norm=True, beta_sigmoid=False),
                                   dict(qk_l2norm=False, beta_sigmoid=True)])
@pytest.mark.parametrize("shape,chunk", [
    (dict(B=2, T=256, H=2, HV=4, K=64, V=64), 64),
    (dict(B=1, T=320, H=1, HV=2, K=128, V=128), 64),
    (dict(B=1, T=256, H=2, HV=2, K=128, V=40), 32),
])
def test_prefill_transforms(shape, chunk, flags):
    log(f"prefill transforms {flags} {shape} chunk {chunk}")
    inp = _raw_prefill(**shape, seed=sum(shape.values()) + 3, **flags)
    o, s = _prefill_gpu(inp, chunk, **flags)
    o_ref, s_ref = recurrent(**inp, **flags)
    assert_parity(to64(o), o_ref, torch.bfloat16, "o")
    assert_parity(to64(s), s_ref, torch.bfloat16, "state")


def test_prefill_transforms_bench_shape_sampled():
    """B4 T8192 H16 K=V=128 with both transforms, sampled heads against the oracle."""
    log("prefill transforms B4 T8192 H16 K=V=128 (sampled heads)")
    flags = dict(qk_l2norm=True, beta_sigmoid=True)
    inp = _raw_prefill(4, 8192, 16, 16, 128, 128, 91, **flags)
    o, s = _prefill_gpu(inp, 64, **flags)
    for b, hv in ((0, 0), (3, 15)):
        ref_o, ref_s = recurrent(**head_slice(inp, b, hv, 1), **flags)
        assert_parity(to64(o[b:b + 1, :, hv:hv + 1]), ref_o, torch.bfloat16, f"o ({b},{hv})")
        assert_parity(to64(s[b:b + 1, hv:hv + 1]), ref_s, torch.bfloat16, f"state ({b},{hv})")


def test_prefill_transforms_unsupported_paths_raise():
    """The transforms live in the two-kernel bf16 path only: fp32 inputs and V % 8 != 0
    report KDA_ERR_UNSUPPORTED instead of silently skipping them."""
    inp = prefill_inputs(1, 64, 1, 1, 32, 32, "fp32", True, 5)
    d = gpu(inp)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                          d["initial_state"], True, 64, qk_l2norm=True)
    inp = prefill_inputs(1, 64, 1, 1, 32, 20, "bf16", True, 6)
    d = gpu(inp)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                          d["initial_state"], True, 64, beta_sigmoid=True)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 4, 8, 64, 64), (2, 1, 3, 128, 128), (1, 2, 2, 20, 12)])
def test_decode_transforms(dtype, shape):
    B, H, HV, K, V = shape
    steps = 5
    log(f"decode transforms dtype={dtype} B={B} H={H} HV={HV} K={K} V={V}")
    inp = decode_inputs(steps, B, H, HV, K, V, dtype, True, 300 + K, beta="logit", raw_qk=True)
    inp["q"] = inp["q"] * 4.0
    inp["beta"] = inp["beta"] * 4.0
    dev = "cuda"
    state = inp["state"].to(dev).clone()
    q, k, v, g, beta = (inp[n].to(dev) for n in ("q", "k", "v", "g", "beta"))
    outs = [kda.kda_recurrent_step(q[t], k[t], v[t], g[t], beta[t], state, inp["scale"],
                                   qk_l2norm=True, beta_sigmoid=True) for t in range(steps)]
    torch.cuda.synchronize()
    s_ref = to64(inp["state"])
    for t in range(steps):
        o_ref, s_ref = decode_step(to64(inp["q"][t]), to64(inp["k"][t]), to64(inp["v"][t]),
                                   to64(inp["g"][t]), to64(inp["beta"][t]), s_ref, inp["scale"],
                                   qk_l2norm=True, beta_sigmoid=True)
        og = to64(outs[t])
        if dtype == "fp32":
            assert np.max(np.abs(og - o_ref)) <= 1e-5, f"step {t}"
        else:
            assert_parity(og, o_ref, torch.bfloat16, f"o step {t}")
    if dtype == "fp32":
        assert np.max(np.abs(to64(state) - s_ref)) <= 1e-5
    else:
        assert_parity(to64(state), s_ref, torch.bfloat16, "state")
