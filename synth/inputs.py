"""Seeded CPU synthesis of KDA inputs.

Value distributions (the layer shapes and distributions of the five workloads):

* q, k ``[B, T, H, K]``: standard normal, then divided by their L2 norm over K
  (in float32, no epsilon), then cast to the workload dtype;
* v ``[B, T, HV, V]``: standard normal;
* g ``[B, T, HV, K]``: ``max(-5, -softplus(N(0, 1)))`` (natural-log decay,
  the "safe gate" lower bound of -5);
* beta ``[B, T, HV]``: ``sigmoid(N(0, 1))``;
* initial state ``[B, HV, K, V]`` float32: ``0.1 * N(0, 1)`` or absent (zeros).

``gate_inputs`` draws the decay gate's inputs (its docstring gives the recipe).

Draw order is q, k, v, g, beta, state from one ``torch.Generator('cpu')``
seeded with ``seed``; everything is computed in float32 and rounded to the
workload dtype (round to nearest even for bfloat16). The gate and beta modes
are stress variants used for parity only; "const:<v>" and "mixed" reach decays far
below the safe gate's -5 (the standard gate has no lower bound).
"""

import math

import torch
import torch.nn.functional as F

# The five workloads, by name. 'prefill' entries run kda_chunk_fwd; 'decode' runs
# kda_recurrent_step `steps` times on one in-place state. Each has its own seed.
WORKLOADS = {
    "tiny-B2-T16-H2-HV4-K8-fp32": dict(
        kind="prefill", B=2, T=16, H=2, HV=4, K=8, V=8, dtype="fp32", chunk=8,
        init_state=False, seed=1234),
    "gva-B2-T512-H4-HV8-K64-bf16": dict(
        kind="prefill", B=2, T=512, H=4, HV=8, K=64, V=64, dtype="bf16", chunk=64,
        init_state=True, seed=1235),
    "prefill-B4-T8192-H16-K128": dict(
        kind="prefill", B=4, T=8192, H=16, HV=16, K=128, V=128, dtype="bf16", chunk=64,
        init_state=False, seed=1236),
    "decode-B256-H16-K128-64steps": dict(
        kind="decode", steps=64, B=256, H=16, HV=16, K=128, V=128, dtype="bf16",
        init_state=True, seed=1237),
    "prefill-B1-T32768-H96-K128": dict(
        kind="prefill", B=1, T=32768, H=96, HV=96, K=128, V=128, dtype="bf16", chunk=64,
        init_state=True, seed=1238),
}

DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


def _gate(shape, gen, mode):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if mode == "default":
        return torch.clamp(-F.softplus(x), min=-5.0)
    if mode == "slow":
        return -0.01 * F.softplus(x)
    if mode == "zero":
        return torch.zeros(shape)
    if mode == "bound":
        return torch.full(shape, -5.0)
    if mode.startswith("const:"):  # every g equal to one value, e.g. "const:-20"
        return torch.full(shape, float(mode[6:]))
    if mode == "mixed":
        # the default gate, except that about one token in 64 (per value head, all channels)
        # decays 40 times faster: chunks then mix blocks of both kinds of decay span
        fast = torch.rand(shape[:-1] + (1,), generator=gen) < 1.0 / 64.0
        return torch.where(fast, -40.0 * F.softplus(x), torch.clamp(-F.softplus(x), min=-5.0))
    raise ValueError(mode)


def _beta(shape, gen, mode):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if mode == "logit":  # for callers that apply the sigmoid themselves
        return x
    if mode == "default":
        return torch.sigmoid(x)
    if mode == "small":
        return torch.sigmoid(x - 7.0)
    if mode == "large":
        return torch.sigmoid(x + 7.0)
    raise ValueError(mode)


def _unit(shape, gen, raw=False):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x if raw else x / x.norm(dim=-1, keepdim=True)


def prefill_inputs(B, T, H, HV, K, V, dtype="bf16", init_state=True, seed=0,
                   gate="default", beta="default", raw_qk=False):
    """Inputs for one chunked forward. Returns a dict of CPU tensors plus 'scale'.
    raw_qk: q and k stay standard normal (not normalised), for callers that normalise."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = DTYPES[dtype]
    q = _unit((B, T, H, K), gen, raw_qk).to(dt)
    k = _unit((B, T, H, K), gen, raw_qk).to(dt)
    v = torch.randn((B, T, HV, V), generator=gen, dtype=torch.float32).to(dt)
    g = _gate((B, T, HV, K), gen, gate).to(dt)
    b = _beta((B, T, HV), gen, beta).to(dt)
    s0 = None
    if init_state:
        s0 = 0.1 * torch.randn((B, HV, K, V), generator=gen, dtype=torch.float32)
    return dict(q=q, k=k, v=v, g=g, beta=b, initial_state=s0, scale=1.0 / math.sqrt(K))


def decode_inputs(steps, B, H, HV, K, V, dtype="bf16", init_state=True, seed=0,
                  gate="default", beta="default", raw_qk=False):
    """Inputs for `steps` single-token decode steps on one state.

    q, k [steps, B, H, K]; v [steps, B, HV, V]; g [steps, B, HV, K];
    beta [steps, B, HV]; state [B, HV, K, V] float32."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = DTYPES[dtype]
    q = _unit((steps, B, H, K), gen, raw_qk).to(dt)
    k = _unit((steps, B, H, K), gen, raw_qk).to(dt)
    v = torch.randn((steps, B, HV, V), generator=gen, dtype=torch.float32).to(dt)
    g = _gate((steps, B, HV, K), gen, gate).to(dt)
    b = _beta((steps, B, HV), gen, beta).to(dt)
    if init_state:
        s0 = 0.1 * torch.randn((B, HV, K, V), generator=gen, dtype=torch.float32)
    else:
        s0 = torch.zeros((B, HV, K, V), dtype=torch.float32)
    return dict(q=q, k=k, v=v, g=g, beta=b, state=s0, scale=1.0 / math.sqrt(K))


def gate_inputs(B, T, HV, K, dtype="bf16", seed=0, x_std=1.0):
    """Inputs of the decay gate and its backward, drawn in this order:

    * x ``[B, T, HV, K]``: ``x_std * N(0, 1)`` (the gate projection), rounded to dtype;
    * A_log ``[HV]`` float32: ``log(U(1, 16))`` per head;
    * dt_bias ``[HV, K]`` float32: ``log(expm1(dt))`` with dt log-uniform in
      [1e-3, 1e-1] (softplus(dt_bias) = dt), per channel;
    * dg ``[B, T, HV, K]``: ``N(0, 1)``, rounded to dtype (the gradient reaching g).

    The pages give no initialisation for A_log and dt_bias; these are the usual ranges of
    per-head rates and per-channel time steps of decay gates."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = DTYPES[dtype]
    x = (x_std * torch.randn((B, T, HV, K), generator=gen, dtype=torch.float32)).to(dt)
    a = 1.0 + 15.0 * torch.rand((HV,), generator=gen, dtype=torch.float64)
    A_log = torch.log(a).float()
    u = torch.rand((HV, K), generator=gen, dtype=torch.float64)
    step = torch.exp(math.log(1e-3) + u * (math.log(1e-1) - math.log(1e-3)))
    dt_bias = torch.log(torch.expm1(step)).float()
    dg = torch.randn((B, T, HV, K), generator=gen, dtype=torch.float32).to(dt)
    return dict(x=x, A_log=A_log, dt_bias=dt_bias, dg=dg)


def workload_inputs(name, **overrides):
    """Inputs for the named workload with its own seed."""
    c = dict(WORKLOADS[name])
    c.update(overrides)
    seed = c.pop("seed")
    if c["kind"] == "decode":
        return decode_inputs(c["steps"], c["B"], c["H"], c["HV"], c["K"], c["V"],
                             c["dtype"], c["init_state"], seed)
    return prefill_inputs(c["B"], c["T"], c["H"], c["HV"], c["K"], c["V"], c["dtype"],
                          c["init_state"], seed)
