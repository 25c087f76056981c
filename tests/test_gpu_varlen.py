"""GPU parity of kda_chunk_fwd_varlen (packed variable-length sequences, each with its own
state) against the fp64 oracle run on every sequence separately, and against the
fixed-length kda_chunk_fwd when all lengths are equal (bit-exact: the same per-chunk
arithmetic). Lengths cover 1, 63, 64, 65, an empty sequence and multi-chunk sequences.
Tolerance: bf16 2e-2 x RMS with the per-row guard (tests/helpers.py)."""

import numpy as np
import pytest
import torch

import gated_delta_rule_67_amd as kda
from oracle import recurrent
from synth import prefill_inputs
from tests.helpers import assert_parity, log, to64

pytestmark = pytest.mark.gpu


def _packed(lengths, H, HV, K, V, seed, raw=False):
    """One packed batch row of sum(lengths) tokens plus per-sequence initial states."""
    T = int(sum(lengths))
    inp = prefill_inputs(1, T, H, HV, K, V, "bf16", True, seed, raw_qk=raw,
                         beta="logit" if raw else "default")
    gen = torch.Generator().manual_seed(seed + 1)
    s0 = 0.1 * torch.randn((len(lengths), HV, K, V), generator=gen)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return inp, s0, cu


def _run(inp, s0, cu, **flags):
    d = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
    o, sT = kda.kda_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu.cuda(),
                                     d["scale"], s0.cuda(), True, **flags)
    torch.cuda.synchronize()
    return o, sT


def _check_each(inp, s0, cu, o, sT, sample=None, **flags):
    seqs = range(len(cu) - 1) if sample is None else sample
    for s in seqs:
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:  # empty: the state passes through
            assert torch.equal(sT[s].cpu(), s0[s]), f"sequence {s}: empty sequence changed the state"
            continue
        one = {n: inp[n][:, a:b] for n in ("q", "k", "v", "g", "beta")}
        ref_o, ref_s = recurrent(**one, scale=inp["scale"], initial_state=s0[s:s + 1], **flags)
        assert_parity(to64(o[:, a:b]), ref_o, torch.bfloat16, f"o of sequence {s} ({b - a} tokens)")
        assert_parity(to64(sT[s:s + 1]), ref_s, torch.bfloat16, f"state of sequence {s}")


@pytest.mark.parametrize("lengths,K,V", [
    ([1, 63, 64, 65, 200, 0, 130], 64, 64),
    ([300, 17, 128], 128, 128),
    ([5, 0, 0, 70], 32, 24),
])
def test_mixed_lengths(lengths, K, V):
    log(f"varlen lengths={lengths} K={K} V={V}")
    inp, s0, cu = _packed(lengths, 2, 4, K, V, seed=len(lengths) + K)
    o, sT = _run(inp, s0, cu)
    _check_each(inp, s0, cu, o, sT)


def test_equal_lengths_match_the_batched_forward_bit_exactly():
    log("varlen 3 x 256 tokens vs kda_chunk_fwd with B = 3")
    B, T, H, HV, K, V = 3, 256, 2, 4, 128, 128
    inp = prefill_inputs(B, T, H, HV, K, V, "bf16", True, 17)
    d = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
    o_b, s_b = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                                 d["initial_state"], True, 64)
    packed = {n: d[n].reshape((1, B * T) + tuple(d[n].shape[2:])) for n in ("q", "k", "v", "g", "beta")}
    cu = torch.arange(0, (B + 1) * T, T, dtype=torch.int32, device="cuda")
    o_v, s_v = kda.kda_chunk_fwd_varlen(packed["q"], packed["k"], packed["v"], packed["g"],
                                        packed["beta"], cu, d["scale"], d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o_v.reshape(o_b.shape), o_b)
    assert torch.equal(s_v, s_b)


def test_transforms_on_packed_sequences():
    log("varlen with q/k L2 normalisation and beta sigmoid")
    flags = dict(qk_l2norm=True, beta_sigmoid=True)
    inp, s0, cu = _packed([90, 1, 64], 1, 2, 64, 64, seed=29, raw=True)
    inp["q"] = inp["q"] * 8.0
    inp["beta"] = inp["beta"] * 4.0
    o, sT = _run(inp, s0, cu, **flags)
    _check_each(inp, s0, cu, o, sT, **flags)


def test_long_packed_batch_sampled():
    """Eight sequences of 128 .. 4000 tokens at H=HV=16, K=V=128; two sequences checked."""
    lengths = [4000, 128, 1500, 777, 2048, 333, 3001, 999]
    log(f"varlen H=16 K=V=128 lengths={lengths} (sampled)")
    inp, s0, cu = _packed(lengths, 16, 16, 128, 128, seed=4242)
    o, sT = _run(inp, s0, cu)
    for s in (0, 5):
        a, b = int(cu[s]), int(cu[s + 1])
        for hv in (0, 13):
            one = {n: inp[n][:, a:b, hv:hv + 1] for n in ("q", "k", "v", "g", "beta")}
            ref_o, ref_s = recurrent(**one, scale=inp["scale"], initial_state=s0[s:s + 1, hv:hv + 1])
            assert_parity(to64(o[:, a:b, hv:hv + 1]), ref_o, torch.bfloat16, f"o seq {s} head {hv}")
            assert_parity(to64(sT[s:s + 1, hv:hv + 1]), ref_s, torch.bfloat16, f"state seq {s} head {hv}")


def test_offsets_need_not_start_at_zero():
    log("varlen with cu_seqlens covering tokens 10 .. 150 of 200")
    inp, s0, _ = _packed([200], 1, 1, 64, 64, seed=3)
    cu = torch.tensor([10, 80, 150], dtype=torch.int32)
    s0 = torch.cat([s0, s0])
    o, sT = _run(inp, s0, cu)
    _check_each(inp, s0, cu, o, sT)


def test_unsupported_inputs_raise():
    inp, s0, cu = _packed([64, 64], 1, 1, 60, 64, seed=2)
    d = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        kda.kda_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu.cuda(), d["scale"])
