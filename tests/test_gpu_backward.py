"""GPU parity of kda_chunk_bwd against the fp64 oracle (oracle.recurrent_bwd, pinned to
finite differences of the forward oracle).

Inputs are bf16 (q, k unit-norm, gates in [-5, 0], beta in (0, 1)); do is standard
normal, dht and the initial state N(0, 0.1^2)-ish. Each gradient is held to the bf16
reading of the tolerance the forward uses: RMS(err) <= 2e-2 RMS(ref) with the per-row
guard (tests/helpers.py). Shapes span several 64-token chunks, a ragged last chunk,
GVA (HV > H), K in {32, 64, 128} and V < K; the full-size case is B4 T8192 H16 K=V=128
with sampled heads."""

import numpy as np
import pytest
import torch

import gated_delta_rule_67_amd as kda
from oracle import recurrent_bwd
from synth import prefill_inputs
from tests.helpers import assert_parity, log, to64

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _grad_inputs(B, T, H, HV, K, V, seed, gate="default", beta="default"):
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, seed, gate=gate, beta=beta)
    gen = torch.Generator().manual_seed(seed + 7)
    inp["do"] = torch.randn((B, T, HV, V), generator=gen).to(torch.bfloat16)
    inp["dht"] = 0.1 * torch.randn((B, HV, K, V), generator=gen)
    return inp


def _gpu_bwd(inp, chunk=64):
    d = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
    out = kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["scale"],
                            d["initial_state"], d["dht"], chunk)
    torch.cuda.synchronize()
    return out


def _ref(inp):
    return recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"],
                         inp["do"], inp["initial_state"], inp["dht"])


def _check(got, ref, what=""):
    for name, x, r in zip(NAMES, got, ref):
        # gradients: the RMS and row criteria (the per-element bound is for the forward)
        assert_parity(to64(x), r, torch.bfloat16, f"{what} {name}", elem=False)


@pytest.mark.parametrize("shape", [
    dict(B=1, T=64, H=1, HV=1, K=32, V=32),
    dict(B=2, T=128, H=2, HV=4, K=64, V=64),      # GVA, two chunks
    dict(B=1, T=200, H=1, HV=2, K=64, V=48),      # ragged last chunk, V < K
    dict(B=1, T=256, H=2, HV=2, K=128, V=128),
    dict(B=2, T=96, H=1, HV=3, K=128, V=16),      # G = 3, one 16-column tile
])
def test_small_shapes(shape):
    log(f"backward {shape}")
    inp = _grad_inputs(**shape, seed=sum(shape.values()))
    chunk = 64 if shape["T"] % 64 == 0 else 8  # kernels tile by 64 and mask the ragged tail
    _check(_gpu_bwd(inp, chunk), _ref(inp), str(shape))


@pytest.mark.parametrize("gate,beta", [("bound", "default"), ("zero", "large"), ("slow", "small")])
def test_stress_gates(gate, beta):
    log(f"backward stress gate={gate} beta={beta} (B1 T512 H=HV=2 K=V=128)")
    inp = _grad_inputs(1, 512, 2, 2, 128, 128, 61, gate=gate, beta=beta)
    _check(_gpu_bwd(inp), _ref(inp), f"{gate}/{beta}")


def test_chunk_size_does_not_change_the_result():
    inp = _grad_inputs(1, 256, 1, 2, 64, 64, 5)
    a = _gpu_bwd(inp, 64)
    for chunk in (16, 128):
        b = _gpu_bwd(inp, chunk)
        for name, x, y in zip(NAMES, a, b):
            assert torch.equal(x, y), f"{name} differs at chunk {chunk}"


def test_full_size_sampled_heads():
    """B4 T8192 H16 K=V=128 (the prefill workload), two heads against the oracle."""
    log("backward B4 T8192 H16 K=V=128 (sampled heads)")
    inp = _grad_inputs(4, 8192, 16, 16, 128, 128, 1236)
    got = _gpu_bwd(inp)
    for b, hv in ((0, 0), (3, 11)):
        one = {n: (t[b:b + 1, :, hv:hv + 1] if t.dim() >= 3 and n != "initial_state" and n != "dht"
                   else t) for n, t in inp.items() if isinstance(t, torch.Tensor)}
        one["initial_state"] = inp["initial_state"][b:b + 1, hv:hv + 1]
        one["dht"] = inp["dht"][b:b + 1, hv:hv + 1]
        one["scale"] = inp["scale"]
        ref = _ref(one)
        sub = [got[0][b:b + 1, :, hv:hv + 1], got[1][b:b + 1, :, hv:hv + 1],
               got[2][b:b + 1, :, hv:hv + 1], got[3][b:b + 1, :, hv:hv + 1],
               got[4][b:b + 1, :, hv:hv + 1], got[5][b:b + 1, hv:hv + 1]]
        _check(sub, ref, f"({b},{hv})")


def test_unsupported_shapes_raise():
    inp = prefill_inputs(1, 64, 1, 1, 48, 32, "bf16", True, 3)
    d = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
    do = torch.zeros_like(d["v"])
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, d["scale"])


def _packed_grad_inputs(lengths, H, HV, K, V, seed):
    T = int(sum(lengths))
    inp = _grad_inputs(1, T, H, HV, K, V, seed)
    gen = torch.Generator().manual_seed(seed + 3)
    N = len(lengths)
    inp["initial_state"] = 0.1 * torch.randn((N, HV, K, V), generator=gen)
    inp["dht"] = 0.1 * torch.randn((N, HV, K, V), generator=gen)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return inp, cu


def _gpu_bwd_varlen(inp, cu):
    d = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
    out = kda.kda_chunk_bwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], cu.cuda(),
                                   d["scale"], d["initial_state"], d["dht"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("lengths,H,HV,K,V", [
    ([1, 63, 64, 65, 150, 0, 130], 1, 2, 64, 64),
    ([200, 17], 2, 4, 128, 48),              # GVA
])
def test_packed_sequences(lengths, H, HV, K, V):
    log(f"backward packed lengths={lengths} H={H} HV={HV} K={K} V={V}")
    inp, cu = _packed_grad_inputs(lengths, H, HV, K, V, seed=len(lengths) * 7 + K)
    got = _gpu_bwd_varlen(inp, cu)
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:  # empty: the state gradient passes through
            assert torch.equal(got[5][s].cpu(), inp["dht"][s]), f"sequence {s}"
            continue
        one = {n: inp[n][:, a:b] for n in ("q", "k", "v", "g", "beta", "do")}
        one.update(scale=inp["scale"], initial_state=inp["initial_state"][s:s + 1],
                   dht=inp["dht"][s:s + 1])
        ref = _ref(one)
        sub = [x[:, a:b] for x in got[:5]] + [got[5][s:s + 1]]
        _check(sub, ref, f"sequence {s} ({b - a} tokens)")


def test_packed_equal_lengths_match_the_batched_backward():
    log("backward packed 3 x 192 tokens vs kda_chunk_bwd with B = 3 (GVA)")
    B, T, H, HV, K, V = 3, 192, 2, 4, 64, 64
    inp = _grad_inputs(B, T, H, HV, K, V, 88)
    a = _gpu_bwd(inp)
    packed = {n: inp[n].reshape((1, B * T) + tuple(inp[n].shape[2:]))
              for n in ("q", "k", "v", "g", "beta", "do")}
    packed.update(scale=inp["scale"], initial_state=inp["initial_state"], dht=inp["dht"])
    cu = torch.arange(0, (B + 1) * T, T, dtype=torch.int32)
    b = _gpu_bwd_varlen(packed, cu)
    for name, x, y in zip(NAMES, a, b):
        assert torch.equal(x, y.reshape(x.shape)), f"{name} differs"


@pytest.mark.parametrize("flags", [dict(qk_l2norm=True, beta_sigmoid=True),
                                   dict(qk_l2norm=True, beta_sigmoid=False),
                                   dict(qk_l2norm=False, beta_sigmoid=True)])
@pytest.mark.parametrize("shape", [dict(B=1, T=192, H=1, HV=1, K=128, V=128),
                                   dict(B=2, T=128, H=2, HV=4, K=64, V=32)])
def test_through_input_transforms(shape, flags):
    """Raw q, k (norms far from 1) and beta logits; gradients for the raw inputs against the
    oracle's chain rule through the same transforms."""
    log(f"backward through transforms {flags} {shape}")
    B, T, H, HV, K, V = (shape[n] for n in ("B", "T", "H", "HV", "K", "V"))
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, 71 + K, raw_qk=flags["qk_l2norm"],
                         beta="logit" if flags["beta_sigmoid"] else "default")
    if flags["qk_l2norm"]:
        inp["q"] = inp["q"] * 4.0
    if flags["beta_sigmoid"]:
        inp["beta"] = inp["beta"] * 3.0
    gen = torch.Generator().manual_seed(72)
    inp["do"] = torch.randn((B, T, HV, V), generator=gen).to(torch.bfloat16)
    inp["dht"] = 0.1 * torch.randn((B, HV, K, V), generator=gen)
    d = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
    got = kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["scale"],
                            d["initial_state"], d["dht"], 64, **flags)
    torch.cuda.synchronize()
    ref = recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"],
                        inp["do"], inp["initial_state"], inp["dht"], **flags)
    _check(got, ref, str(flags))


def test_packed_sequences_through_input_transforms():
    log("backward packed, q/k L2 norm and beta sigmoid")
    flags = dict(qk_l2norm=True, beta_sigmoid=True)
    lengths = [70, 1, 128]
    T = sum(lengths)
    inp = prefill_inputs(1, T, 1, 2, 64, 64, "bf16", True, 75, raw_qk=True, beta="logit")
    gen = torch.Generator().manual_seed(76)
    inp["do"] = torch.randn((1, T, 2, 64), generator=gen).to(torch.bfloat16)
    inp["initial_state"] = 0.1 * torch.randn((3, 2, 64, 64), generator=gen)
    inp["dht"] = 0.1 * torch.randn((3, 2, 64, 64), generator=gen)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    d = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
    got = kda.kda_chunk_bwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], cu.cuda(),
                                   d["scale"], d["initial_state"], d["dht"], **flags)
    torch.cuda.synchronize()
    for s in range(3):
        a, b = int(cu[s]), int(cu[s + 1])
        one = {n: inp[n][:, a:b] for n in ("q", "k", "v", "g", "beta", "do")}
        ref = recurrent_bwd(one["q"], one["k"], one["v"], one["g"], one["beta"], inp["scale"],
                            one["do"], inp["initial_state"][s:s + 1], inp["dht"][s:s + 1], **flags)
        sub = [x[:, a:b] for x in got[:5]] + [got[5][s:s + 1]]
        _check(sub, ref, f"sequence {s}")


@pytest.mark.parametrize("shape", [dict(B=1, T=256, H=2, HV=4, K=64, V=64),
                                   dict(B=1, T=200, H=1, HV=1, K=128, V=128),
                                   dict(B=1, T=200, H=1, HV=2, K=64, V=48)])
def test_backward_is_reproducible(shape):
    """Every sum in the backward runs in a fixed order (the row sums of dS * h by lane shuffles,
    or from per-piece partials in LDS when V / 8 is not a power of two; the dbeta partial sums
    take exactly two terms, and a sum of two terms does not depend on their order), so two
    calls on the same inputs agree bit for bit."""
    inp = _grad_inputs(**shape, seed=91)
    log(f"backward twice {shape}")
    chunk = 64 if shape["T"] % 64 == 0 else 8  # chunk_size must divide T; kernels tile by 64
    first = _gpu_bwd(inp, chunk)
    second = _gpu_bwd(inp, chunk)
    for name, a, b in zip(NAMES, first, second):
        assert torch.equal(a, b), f"{name} differs between two calls"
