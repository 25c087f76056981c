"""Benchmark of the KDA forward on one MI355X.

A step is one chunked prefill (kda_chunk_fwd) over the prefill workload
B=4, T=8192, H=HV=16, K=V=128, bf16 inputs, fp32 state, chunk 64 (synthetic,
seeded; the 16 x 128 head layout and 8,192-token context of the pages' KDA
layers). `value` is prefill tokens/s (B*T per step). Timed in the same run, each
reported under its own key:
* "prefill_long": the long-context wide-head prefill, B=1, T=32768, H=HV=96,
  K=V=128, initial state N(0, 0.1), on the default path;
* "decode": kda_recurrent_step, 64 consecutive steps on a B=256, H=HV=16, K=V=128
  fp32 state cache, and the same steps over 4 distinct caches in turn (1.07 GB, more
  than the last-level cache, as the layers of a model would be);
* "backward": kda_chunk_bwd (dq, dk, dv, dg, dbeta, dh0) of the prefill workload for a
  seeded dO;
* "few_heads": the prefill at B=1, T=32768 on 4, 8 and 16 heads (segmented when it pays);
* "gate": kda_gate_fwd / kda_gate_bwd on the prefill layer's [B, T, HV, K] gate input,
  and the gate fused into the prefill.

Timing uses HIP events recorded on the stream the kernels are launched on,
bracketed by device synchronisation. One prefill call is three kernels on that
stream (factors_kernel: the state-independent per-chunk factors for all chunks;
factors_exact_kernel: the chunks whose decay span is too wide for them, which exits at
once when there are none; state_kernel: the sequential state pass), timed together. The
roofline object prices the call's algorithmic bytes (q, k, v, g, beta read once, o and
the final state written once) against MI355X's 8 TB/s HBM3E peak; the decode object
prices its algorithmic bytes (state read + write, plus the token vectors) the same way.
A 1 GiB device copy by the library's streaming copy kernel, timed right before the prefill
steps (after their inputs are on the device and their first call is checked), gives the
measured HBM ceiling (the runtime's copy is reported beside it) and brings the clocks up.
The decode steps and the gate calls, whose kernels take 50-90 us, are issued through the
C ABI with their outputs allocated up front (checked bit for bit against the Python
binding first), so that the host's per-call work in the binding does not leave gaps
between the timed kernels.

The CPU leg runs first, before the GPU is touched: the fp64 oracle over the whole prefill
workload on one worker process per host core (up to 16, one numpy thread each) is the
"cpu_baseline"; the same leg computes the oracle's results for sampled heads of every
other timed configuration. Each timed configuration's first call (the one checked before
its timing loop) is compared with those results: "cpu_baseline.parity_of_timed_calls".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2516.6     # MI355X dense bf16 MFMA, published (no sparsity)
METRIC = "KDA prefill tokens/s + MFMA util (H=16,K=V=128,T=8192); decode state HBM GB/s"
PREFILL_KERNELS = ["kda::wy::factors_kernel<128, false, false, false>",
                   "kda::wy::factors_exact_kernel<128, false, false, false>",
                   "kda::wy::state_kernel<128, 2, false, true>"]
LONG_KERNELS = ["kda::wy::factors_kernel<128, false, false, false>",
                "kda::wy::factors_exact_kernel<128, false, false, false>",
                "kda::wy::state_kernel<128, 4, false, true>"]
PREFILL_WORKLOAD = "prefill-B4-T8192-H16-K128"
LONG_WORKLOAD = "prefill-B1-T32768-H96-K128"
DECODE_WORKLOAD = "decode-B256-H16-K128-64steps"
BACKWARD_DO_SEED = 4321
# committed rocprofv3 counter records, each valid while the sources it names are unchanged
COUNTER_RECORDS = {
    "prefill": ("prefill_traffic.json", ["kda_chunk_wy.hip", "kda_device.h"]),
    "decode": ("decode_traffic.json", ["kda_decode.hip", "kda_device.h"]),
    "backward": ("backward_traffic.json", ["kda_chunk_bwd.hip", "kda_device.h"]),
}
BF16_REL, BF16_UNIT = 2e-2, 2.0 ** -8


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_algorithmic(B, T, H, HV, K, V, ib, state_in, state_out):
    """Bytes and flops the operator must move / do, per launch.

    Bytes: q, k read once per q/k head; v, g, beta read once; o written once;
    the K x V fp32 state read (if given) and written once per value head.
    Flops per token-head (chunk C, triangle-aware): C(3K + 2V) + 6KV + C^2/3."""
    C = 64
    tok = B * T
    byts = tok * (H * 2 * K * ib + HV * (V + K + 1 + V) * ib)
    byts += B * HV * K * V * 4 * (int(state_in) + int(state_out))
    flops = tok * HV * (C * (3 * K + 2 * V) + 6 * K * V + C * C / 3.0)
    return byts, flops


def backward_algorithmic(B, T, H, HV, K, V, ib):
    """Bytes of one backward call: q, k, v, g, beta, dO and the initial state read once;
    dq, dk, dv, dg, dbeta and dh0 written once."""
    qk = 2 * B * T * H * K * ib
    per_v = B * T * HV * (V + K + 1 + V) * ib      # v, g, beta, dO
    state = B * HV * K * V * 4
    reads = qk + per_v + state
    writes = qk + B * T * HV * (V + K + 1) * ib + state
    return reads + writes


def gate_algorithmic(n, HV, K, ib=2):
    """Bytes of the gate's calls over n elements: forward reads x and writes g; backward
    reads x and dg and writes dx, plus the fp32 parameters and their gradients."""
    params = HV * 4 + HV * K * 4
    return 2 * n * ib + params, 3 * n * ib + 2 * params


def decode_algorithmic(B, H, HV, K, V, ib):
    """Bytes per decode step: fp32 state read + write, q/k per q/k head, v/g/beta/o per value head."""
    return B * HV * 2 * K * V * 4 + B * (H * 2 * K + HV * (V + K + 1 + V)) * ib


def source_hash(names):
    """Hash of kernel sources (a counter record goes stale when they change)."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "gated_delta_rule_67_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_record(which):
    """The committed rocprofv3 --pmc record of a path, if its sources have not changed since
    the counters were taken; else None."""
    fname, sources = COUNTER_RECORDS[which]
    try:
        with open(os.path.join(ROOT, "profiles", fname)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("source_sha256_16") == source_hash(sources) else None


def measured_traffic(which):
    """HBM bytes per launch from the counter record, or None."""
    rec = counter_record(which)
    return rec.get("bytes_per_launch") if rec else None


def time_launches(fn, steps, warmup, torch, settle=None):
    """Average launch duration in ms over `steps` back-to-back launches, timed by two events on
    the launch stream around all of them; then, in a second pass of `steps` launches with an
    event after each, the per-launch median and minimum. `settle` (if given) runs first, right
    before the warm-up launches."""
    if settle is not None:
        settle()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return avg, per[len(per) // 2], per[0]


def gate_abi_calls(kda, x, A_log, dt_bias, dg, lower_bound, torch):
    """kda_gate_fwd and kda_gate_bwd called through the C ABI with their outputs and workspace
    allocated once. The kernels take about 50 and 90 us; the Python binding's per-call checks
    and allocations take about as long, so timing back-to-back calls through it would measure
    the host. Each caller returns the status; the first calls are checked here, and their
    outputs are compared with the binding's, bit for bit."""
    import ctypes
    lib = kda.library()
    B, T, HV, K = x.shape
    dt = kda._DTYPE[x.dtype]
    g = torch.empty_like(x)
    dx = torch.empty_like(x)
    dA = torch.empty((HV,), dtype=torch.float32, device=x.device)
    db = torch.empty((HV, K), dtype=torch.float32, device=x.device)
    ws_bytes = lib.kda_gate_bwd_workspace_size(B, T, HV, K, dt)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    fwd_args = (p(x), p(A_log), p(dt_bias), p(g), B, T, HV, K, float(lower_bound), dt, stream)
    bwd_args = (p(x), p(A_log), p(dt_bias), p(dg), p(dx), p(dA), p(db), B, T, HV, K,
                float(lower_bound), dt, p(ws), ws_bytes, stream)
    fwd = lambda: lib.kda_gate_fwd(*fwd_args)
    bwd = lambda: lib.kda_gate_bwd(*bwd_args)
    assert fwd() == kda.KDA_OK and bwd() == kda.KDA_OK, "gate entry points failed"
    ref_g = kda.kda_gate_fwd(x, A_log, dt_bias, lower_bound)
    ref_dx, ref_dA, ref_db = kda.kda_gate_bwd(x, A_log, dt_bias, dg, lower_bound)
    torch.cuda.synchronize()
    assert torch.equal(g, ref_g) and torch.equal(dx, ref_dx), "C ABI and binding differ"
    assert torch.equal(dA, ref_dA) and torch.equal(db, ref_db), "C ABI and binding differ"
    return fwd, bwd


def clock_settler(torch, kda, nbytes=1 << 30, reps=110):
    """About 40 ms of streaming copies (kda_stream_copy, 1 GiB each way), run right before a
    leg's warm-up: the chip lowers its clock for some tens of milliseconds after a heavy load
    starts on an idle GPU (as it is after a leg's inputs go to the device and its first call's
    outputs come back), and this way that happens during the copies, not the timed calls."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def settle():
        for _ in range(reps):
            kda.stream_copy(src, dst)
        torch.cuda.synchronize()
    return settle


def copy_ceiling(torch, kda, nbytes=1 << 30, reps=20):
    """Measured HBM ceiling: GB/s (read + write bytes) of a 1 GiB device-to-device copy by the
    library's streaming copy (kda_stream_copy: non-temporal 16-byte accesses), and of the
    runtime's copy (torch copy_) for reference. Run first, it also brings the clocks up
    before the prefill is timed."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(50):  # about 20 ms of copies: the clocks' ramp on a fresh box
        dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(5):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return 2 * nbytes / (ev[0].elapsed_time(ev[1]) / reps * 1e-3) / 1e9

    runtime = timed(lambda: dst.copy_(src))
    dst.zero_()
    kernel = timed(lambda: kda.stream_copy(src, dst))
    assert torch.equal(dst[:4096], src[:4096]) and torch.equal(dst[-4096:], src[-4096:]), \
        "kda_stream_copy did not copy"
    del src, dst
    return kernel, runtime


def sample_heads(c, n):
    """n distinct (b, hv) heads of a workload, drawn from its seed."""
    rng = np.random.default_rng(c["seed"])
    heads = []
    while len(heads) < n:
        h = (int(rng.integers(c["B"])), int(rng.integers(c["HV"])))
        if h not in heads:
            heads.append(h)
    return heads


# ================================================================ CPU leg: the oracle
# Everything below this line up to `compare` calls the oracle; it runs in worker processes
# forked before the GPU is touched, one numpy thread each.

_SHARED = {}  # inputs the workers read (set before the fork, shared copy-on-write)


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def _np(t):
    """A CPU tensor (bf16 / fp32) as a float32 numpy array (exact for bf16), or None."""
    return None if t is None else t.float().numpy()


def host_inputs(inputs, samples):
    """The inputs the oracle needs, as numpy arrays (the workers run no torch op): the whole
    prefill workload, and the sampled heads of the other configurations."""
    def arrays(inp):
        return {n: (_np(v) if n != "scale" else v) for n, v in inp.items()}
    host = {"prefill": arrays(inputs["prefill"])}
    if "long" in samples:
        host["long"] = {h: arrays(_head(inputs["long"], *h)) for h in samples["long"]}
    if "backward" in samples:
        host["dout"] = {h: _np(inputs["dout"][h[0]:h[0] + 1, :, h[1]:h[1] + 1].contiguous())
                        for h in samples["backward"]}
    if "decode" in samples:
        host["decode"] = arrays(inputs["decode"])
    return host


def _head(inp, b, hv, tokens=None, hv_end=None):
    """Value heads hv .. hv_end - 1 (default: hv alone) of batch b of a prefill input as a
    B = 1 problem; hv and hv_end are multiples of G (GVA: q/k head hv / G)."""
    G = inp["v"].shape[2] // inp["q"].shape[2]
    hv_end = hv + 1 if hv_end is None else hv_end
    h, h_end = hv // G, (hv_end + G - 1) // G
    t = slice(None) if tokens is None else slice(0, tokens)
    out = dict(q=inp["q"][b:b + 1, t, h:h_end], k=inp["k"][b:b + 1, t, h:h_end],
               v=inp["v"][b:b + 1, t, hv:hv_end], g=inp["g"][b:b + 1, t, hv:hv_end],
               beta=inp["beta"][b:b + 1, t, hv:hv_end], scale=inp["scale"])
    s0 = inp.get("initial_state")
    out["initial_state"] = None if s0 is None else s0[b:b + 1, hv:hv_end]
    return out


def _oracle_prefill(task):
    """The oracle on value heads hv .. hv_end - 1 of batch b (one call: the heads side by side)."""
    from oracle import recurrent
    key, b, hv, hv_end, tokens = task
    one = _head(_SHARED["prefill"], b, hv, tokens, hv_end) if key == "prefill" else _SHARED["long"][(b, hv)]
    o, s = recurrent(**one)
    return key, b, hv, o[0], s[0]


def _oracle_backward(task):
    from oracle import recurrent_bwd
    _, b, hv = task
    one = _head(_SHARED["prefill"], b, hv)
    g = recurrent_bwd(one["q"], one["k"], one["v"], one["g"], one["beta"], one["scale"],
                      _SHARED["dout"][(b, hv)], one["initial_state"], None)
    return "backward", b, hv, [x[0, :, 0] for x in g[:5]] + [g[5][0, 0]]


def _oracle_decode(task):
    from oracle import decode_step
    _, bs, hs = task
    inp = _SHARED["decode"]
    G = inp["v"].shape[2] // inp["q"].shape[2]
    s = inp["state"][np.ix_(bs, hs)]
    outs = []
    for t in range(inp["q"].shape[0]):
        o, s = decode_step(inp["q"][t][bs][:, [h // G for h in hs]],
                           inp["k"][t][bs][:, [h // G for h in hs]],
                           inp["v"][t][np.ix_(bs, hs)], inp["g"][t][np.ix_(bs, hs)],
                           inp["beta"][t][np.ix_(bs, hs)], s, inp["scale"])
        outs.append(o)
    return "decode", bs, hs, np.stack(outs), s


def _run(fn_task):
    fn, task = fn_task
    return fn(task)


def cpu_leg(host, samples, tokens, workers):
    """The oracle on the host, on numpy inputs (host_inputs). Times the whole prefill workload
    (its first `tokens` tokens) over `workers` processes; then the sampled heads of the other
    configurations."""
    import multiprocessing as mp
    _SHARED.update(host)
    pre = host["prefill"]
    B, T, HV = pre["q"].shape[0], pre["q"].shape[1], pre["v"].shape[2]
    G = HV // pre["q"].shape[2]
    # tasks: batches, each split into head groups (whole q/k heads) so that there are about
    # as many tasks as workers; a task's heads run side by side in one oracle call
    groups = max(1, min(HV // G, -(-workers // B)))
    bounds = [G * (i * (HV // G) // groups) for i in range(groups + 1)]
    base_tasks = [(_oracle_prefill, ("prefill", b, bounds[i], bounds[i + 1], tokens))
                  for b in range(B) for i in range(groups)]
    other = [(_oracle_prefill, ("long", b, hv, hv + 1, None)) for b, hv in samples.get("long", [])]
    other += [(_oracle_backward, ("backward", b, hv)) for b, hv in samples.get("backward", [])]
    if "decode" in samples:
        other.append((_oracle_decode, ("decode",) + samples["decode"]))
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_one_thread) as pool:
        t0 = time.perf_counter()
        base = pool.map(_run, base_tasks, chunksize=1)
        dt = time.perf_counter() - t0
        rest = pool.map(_run, other, chunksize=1) if other else []
    ref = {"prefill": {}}
    for _, b, hv, o, s in base:  # o [T, n, V], s [n, K, V] for heads hv .. hv + n - 1
        for j in range(s.shape[0]):
            ref["prefill"][(b, hv + j)] = (o[:, j], s[j])
    for r in rest:
        if r[0] == "long":
            ref.setdefault("long", {})[(r[1], r[2])] = (r[3][:, 0], r[4][0])
        elif r[0] == "backward":
            ref.setdefault("backward", {})[(r[1], r[2])] = r[3]
        else:
            ref["decode"] = r
    baseline = dict(value=B * tokens / dt, unit="tokens/s", cores=workers, kind="oracle",
                    sample=f"first {tokens} of the {T} tokens of the prefill workload, all B={B} x "
                           f"{HV} heads ({B * tokens} tokens, {dt:.1f} s wall), numpy float64, "
                           f"{workers} worker processes of one thread, {len(base_tasks)} tasks of "
                           f"{bounds[1] - bounds[0]} heads side by side")
    return baseline, ref


def compare(got, ref, elem=True):
    """Parity of one tensor pair at the bf16 reading: RMS(err) <= 2e-2 RMS(ref), every row
    (last axis) within 2e-2 (row RMS + RMS), and, if elem, every element within
    2e-2 RMS + 2^-8 |ref| (bf16's unit roundoff)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = got - ref
    rms = float(np.sqrt(np.mean(ref ** 2)))
    rel = float(np.sqrt(np.mean(err ** 2))) / rms
    row = float(np.max(np.sqrt(np.mean(err ** 2, axis=-1)) / (np.sqrt(np.mean(ref ** 2, axis=-1)) + rms)))
    ratio = float(np.max(np.abs(err) / (BF16_REL * rms + BF16_UNIT * np.abs(ref))))
    ok = bool(np.all(np.isfinite(got)) and rel <= BF16_REL and row <= BF16_REL and (ratio <= 1.0 or not elem))
    return {"rms_err_over_rms": rel, "worst_row": row, "elem_bound_ratio": ratio,
            "elem_bound_asserted": elem, "pass": ok}


# ================================================================ GPU legs

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-reps", type=int, default=3)
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--cpu-workers", type=int, default=0, help="0: one per host core, at most 16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-gate", action="store_true")
    ap.add_argument("--no-segmented", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=20)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU code: it would shard by (batch, value head) with no "
              "communication).", file=sys.stderr)
        sys.exit(2)

    import torch

    from synth import WORKLOADS, workload_inputs

    c = WORKLOADS[PREFILL_WORKLOAD]
    cl = WORKLOADS[LONG_WORKLOAD]
    c3 = WORKLOADS[DECODE_WORKLOAD]
    log(f"bench: generating {PREFILL_WORKLOAD}")
    inputs = {"prefill": workload_inputs(PREFILL_WORKLOAD)}
    gen = torch.Generator().manual_seed(BACKWARD_DO_SEED)
    inputs["dout"] = torch.randn(inputs["prefill"]["v"].shape, generator=gen).to(torch.bfloat16)
    if not args.no_long:
        log(f"bench: generating {LONG_WORKLOAD}")
        inputs["long"] = workload_inputs(LONG_WORKLOAD)
    if not args.no_decode:
        inputs["decode"] = workload_inputs(DECODE_WORKLOAD)

    # ---------------- the CPU leg, before anything touches the GPU
    samples = {}
    if not args.no_long:
        samples["long"] = sample_heads(cl, 2)
    if not args.no_backward:
        samples["backward"] = sample_heads(c, 2)
    if not args.no_decode:
        rng = np.random.default_rng(c3["seed"])
        samples["decode"] = (np.sort(rng.choice(c3["B"], 8, replace=False)),
                             np.sort(rng.choice(c3["HV"], 4, replace=False)))
    baseline = ref = None
    if not args.no_cpu_baseline:
        try:
            avail = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            avail = os.cpu_count() or 1
        workers = args.cpu_workers or max(1, min(16, avail))
        tokens = min(args.cpu_tokens, c["T"])
        log(f"bench: the oracle on the host ({workers} workers, {tokens} tokens of the prefill "
            f"workload, then the sampled heads)")
        baseline, ref = cpu_leg(host_inputs(inputs, samples), samples, tokens, workers)

    import gated_delta_rule_67_amd as kda

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    checked = {}  # outputs of each configuration's first call, on the host

    # ---------------- prefill workload (the step)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inputs["prefill"].items()}

    def prefill():
        return kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                                 d["initial_state"], True, c["chunk"])

    o, s = prefill()
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all(), "non-finite prefill output"
    checked["prefill"] = (o.cpu(), s.cpu())
    del o, s
    # The copy ceiling runs right before the timed calls, with the inputs already on the device:
    # the chip lowers its clock for some tens of milliseconds after a heavy load starts on an
    # idle GPU, and without a gap between the copies and the prefill calls that happens during
    # the copies.
    ceiling, runtime_copy = copy_ceiling(torch, kda)
    settle = clock_settler(torch, kda)  # for the later legs, which follow uploads and checks
    log(f"bench: timing {args.steps} prefill steps after {args.warmup} warmup")
    avg_ms, med_ms, min_ms = time_launches(prefill, args.steps, args.warmup, torch)
    tokens = c["B"] * c["T"]
    byts, flops = prefill_algorithmic(c["B"], c["T"], c["H"], c["HV"], c["K"], c["V"], 2,
                                      c["init_state"], True)
    achieved = byts / (avg_ms * 1e-3) / 1e9
    tflops = flops / (avg_ms * 1e-3) / 1e12
    t_bound = max(flops / (MFMA_BF16_PEAK_TFS * 1e12), byts / (HBM_PEAK_GBS * 1e9))

    result = {
        "metric": METRIC,
        "value": tokens / (avg_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": avg_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "KDA chunked prefill B=4 T=8192 H=HV=16 K=V=128 bf16 in, fp32 state, "
                               "chunk 64, zero initial state",
                   "B": c["B"], "T": c["T"], "H": c["H"], "HV": c["HV"], "K": c["K"], "V": c["V"],
                   "chunk_size": c["chunk"], "seed": c["seed"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("prefill"),
                     "kernel": " + ".join(PREFILL_KERNELS) + " (one kda_chunk_fwd call)",
                     "algorithmic_bytes_per_launch": byts,
                     "avg_launch_ms": avg_ms, "median_launch_ms": med_ms, "min_launch_ms": min_ms,
                     "roofline_frac": t_bound * 1e3 / avg_ms,
                     "measured_copy_ceiling_gbs": ceiling, "frac_of_copy_ceiling": achieved / ceiling,
                     "runtime_copy_gbs": runtime_copy},
        "mfma": {"algorithmic_tflops": tflops, "peak_tflops": MFMA_BF16_PEAK_TFS,
                 "frac": tflops / MFMA_BF16_PEAK_TFS, "algorithmic_flops_per_launch": flops},
    }
    rec = counter_record("prefill")
    if rec and "issued_bf16_flops_per_launch" in rec:
        # issued MFMA work (full tiles, V-tile duplication) from the counter record, priced at
        # this run's call time; and the counters' own MFMA-busy fraction
        issued = rec["issued_bf16_flops_per_launch"]
        result["mfma"].update({"issued_tflops_counters": issued / (avg_ms * 1e-3) / 1e12,
                               "issued_frac_counters": issued / (avg_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
                               "issued_bf16_flops_per_launch": issued,
                               "mfma_busy_frac_counters": rec.get("mfma_busy_frac")})

    # ---------------- long-context wide-head prefill
    if not args.no_long:
        log(f"bench: {LONG_WORKLOAD}")
        dl = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inputs["long"].items()}

        def prefill_long():
            return kda.kda_chunk_fwd(dl["q"], dl["k"], dl["v"], dl["g"], dl["beta"], dl["scale"],
                                     dl["initial_state"], True, cl["chunk"])

        o, s = prefill_long()
        torch.cuda.synchronize()
        checked["long"] = {h: (o[h[0], :, h[1]].cpu(), s[h[0], h[1]].cpu()) for h in samples["long"]}
        del o, s
        l_avg, l_med, l_min = time_launches(prefill_long, args.steps, min(args.warmup, 10), torch,
                                            settle)
        lbytes, lflops = prefill_algorithmic(cl["B"], cl["T"], cl["H"], cl["HV"], cl["K"], cl["V"], 2,
                                             True, True)
        lgbs = lbytes / (l_avg * 1e-3) / 1e9
        result["prefill_long"] = {
            "workload": "KDA chunked prefill B=1 T=32768 H=HV=96 K=V=128 bf16 in, fp32 state, "
                        "chunk 64, initial state N(0, 0.1)",
            "ms_per_call": l_avg, "median_ms": l_med, "min_ms": l_min,
            "tokens_per_s": cl["B"] * cl["T"] / (l_avg * 1e-3),
            "roofline": {"bound": "hbm", "achieved": lgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": lgbs / HBM_PEAK_GBS,
                         "hbm_bound_ms": lbytes / (HBM_PEAK_GBS * 1e9) * 1e3,
                         "kernel": " + ".join(LONG_KERNELS) + " (one kda_chunk_fwd call)",
                         "algorithmic_bytes_per_launch": lbytes},
            "mfma": {"algorithmic_tflops": lflops / (l_avg * 1e-3) / 1e12,
                     "frac": lflops / (l_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS},
        }
        del dl

    # ---------------- decode workload
    if not args.no_decode:
        import ctypes
        log(f"bench: {DECODE_WORKLOAD}")
        dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inputs["decode"].items()}
        steps = c3["steps"]
        views = [[dd[n][t] for n in ("q", "k", "v", "g", "beta")] for t in range(steps)]
        # the steps go through the C ABI with every o allocated up front: a step's kernel
        # takes about 80 us, close to what the binding's per-call checks and allocation cost
        # the host, so calls through the binding would leave gaps between the kernels
        lib = kda.library()
        outs = [torch.empty_like(dd["v"][t]) for t in range(steps)]
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        stream = torch.cuda.current_stream()
        sp = ctypes.c_void_p(stream.cuda_stream)
        B3, H3, K3 = dd["q"][0].shape
        HV3, V3 = dd["v"][0].shape[1], dd["v"][0].shape[2]
        caches = [dd["state"].clone() for _ in range(4)]  # caches[0]: the single-cache runs
        step_args = [[tuple(p(x) for x in views[t]) + (p(cache), p(outs[t]), B3, H3, HV3, K3, V3,
                                                         float(dd["scale"]), kda._DTYPE[dd["q"].dtype], sp)
                      for t in range(steps)] for cache in caches]

        def one(t, cache=0):
            return lib.kda_recurrent_step(*step_args[cache][t])

        # warm-up on a scratch copy of the state; the C ABI's first step matches the binding's
        state = caches[0]
        assert one(0) == kda.KDA_OK, "kda_recurrent_step failed"
        state.copy_(dd["state"])
        one(0)
        s_abi, o_abi = state.clone(), outs[0].clone()
        state.copy_(dd["state"])
        o_ref = kda.kda_recurrent_step(*views[0], state, dd["scale"])
        torch.cuda.synchronize()
        assert torch.equal(o_abi, o_ref) and torch.equal(s_abi, state), "C ABI and binding differ"
        del s_abi, o_abi, o_ref

        def run_steps(rotate):
            for cc in caches if rotate else caches[:1]:
                cc.copy_(dd["state"])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for t in range(steps):
                one(t, t % 4 if rotate else 0)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        settle()
        for rotate in (False, True):
            run_steps(rotate)  # warm
        single = [run_steps(False) for _ in range(args.decode_reps)]
        # the last single-cache pass leaves every step's o and the final state: checked below
        bs, hs = samples["decode"]
        checked["decode"] = (np.stack([outs[t].double().cpu().numpy()[np.ix_(bs, hs)] for t in range(steps)]),
                             caches[0].double().cpu().numpy()[np.ix_(bs, hs)])
        rot = [run_steps(True) for _ in range(args.decode_reps)]
        caches[0].copy_(dd["state"])  # per-step durations: one more pass, an event after each step
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for t in range(steps):
            one(t)
            ev[t + 1].record(stream)
        torch.cuda.synchronize()
        per_step = sorted(ev[t].elapsed_time(ev[t + 1]) for t in range(steps))
        step_ms, rot_ms = min(single) / steps, min(rot) / steps
        dbytes = decode_algorithmic(c3["B"], c3["H"], c3["HV"], c3["K"], c3["V"], 2)
        gbs, rgbs = dbytes / (step_ms * 1e-3) / 1e9, dbytes / (rot_ms * 1e-3) / 1e9
        result["decode"] = {
            "workload": "KDA decode, 64 consecutive steps, B=256 H=HV=16 K=V=128, bf16 vectors, "
                        "fp32 state [256,16,128,128] updated in place",
            "value": gbs, "unit": "GB/s", "ms_per_step": step_ms,
            "tokens_per_s": c3["B"] / (step_ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "frac_of_copy_ceiling": gbs / ceiling,
                         "traffic": measured_traffic("decode"),
                         "kernel": "decode_step_kernel",
                         "algorithmic_bytes_per_launch": dbytes,
                         "median_launch_ms": per_step[len(per_step) // 2]},
            "rotating_4_caches": {
                "workload": "the same 64 steps, step t on cache t % 4 of 4 distinct "
                            "[256,16,128,128] fp32 caches (1.07 GB, above the last-level cache)",
                "value": rgbs, "unit": "GB/s", "ms_per_step": rot_ms,
                "tokens_per_s": c3["B"] / (rot_ms * 1e-3),
                "roofline": {"bound": "hbm", "achieved": rgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": rgbs / HBM_PEAK_GBS, "frac_of_copy_ceiling": rgbs / ceiling,
                             "algorithmic_bytes_per_launch": dbytes}},
        }
        rec = counter_record("decode")
        if rec:
            result["decode"]["counters"] = {k: rec[k] for k in ("single_cache", "rotating_4_caches")
                                            if k in rec}
        del dd, caches, views, outs, step_args, state

    # ---------------- chunked backward on the prefill workload
    if not args.no_backward:
        log(f"bench: timing {args.backward_steps} backward calls on {PREFILL_WORKLOAD}")
        dout = inputs["dout"].to(dev)

        def backward():
            return kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dout, d["scale"],
                                     d["initial_state"], None, c["chunk"])

        grads = backward()
        torch.cuda.synchronize()
        assert all(torch.isfinite(x.float()).all() for x in grads), "non-finite gradient"
        checked["backward"] = {
            h: [grads[i][h[0], :, h[1]].cpu() for i in range(5)] + [grads[5][h[0], h[1]].cpu()]
            for h in samples["backward"]}
        del grads
        b_avg, b_med, b_min = time_launches(backward, args.backward_steps, 10, torch, settle)
        bbytes = backward_algorithmic(c["B"], c["T"], c["H"], c["HV"], c["K"], c["V"], 2)
        bgbs = bbytes / (b_avg * 1e-3) / 1e9
        result["backward"] = {
            "workload": PREFILL_WORKLOAD + ", seeded dO, gradients of every input and of the "
                        "initial state",
            "ms_per_call": b_avg, "median_ms": b_med, "min_ms": b_min,
            "tokens_per_s": tokens / (b_avg * 1e-3),
            "roofline": {"bound": "hbm", "achieved": bgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bgbs / HBM_PEAK_GBS, "traffic": measured_traffic("backward"),
                         "kernel": "kda::bwd prep_kernel + fwd_sweep_kernel + rev_sweep_kernel + "
                                   "local_kernel (one kda_chunk_bwd call)",
                         "algorithmic_bytes_per_launch": bbytes},
        }
        rec = counter_record("backward")
        if rec:
            result["backward"]["counters"] = rec.get("kernels")
        del dout

    # ---------------- few heads, long sequence: the segmented prefill against the plain path
    if not args.no_segmented:
        from synth import prefill_inputs
        result["few_heads"] = []
        for (fb, ft, fh) in ((1, 32768, 4), (1, 32768, 8), (1, 32768, 16)):
            log(f"bench: few heads B={fb} T={ft} H=HV={fh}")
            fi = prefill_inputs(fb, ft, fh, fh, 128, 128, "bf16", True, seed=4323)
            fd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in fi.items()}
            del fi
            segs = kda.library().kda_chunk_fwd_workspace_size(fb, ft, fh, fh, 128, 128, 64, 1)
            nseg = next(P for P in (1, 2, 4, 8, 16, 32, 64) if segs ==
                        kda.library().kda_chunk_fwd_segmented_workspace_size(fb, ft, fh, fh, 128,
                                                                             128, P, 1))
            auto = lambda: kda.kda_chunk_fwd(fd["q"], fd["k"], fd["v"], fd["g"], fd["beta"],
                                             fd["scale"], fd["initial_state"])
            plain = lambda: kda.kda_chunk_fwd_segmented(fd["q"], fd["k"], fd["v"], fd["g"],
                                                        fd["beta"], 1, fd["scale"],
                                                        fd["initial_state"])
            a_avg, a_med, _ = time_launches(auto, args.steps, args.warmup, torch, settle)
            p_avg, p_med, _ = time_launches(plain, args.steps, args.warmup, torch, settle)
            fbytes, _ = prefill_algorithmic(fb, ft, fh, fh, 128, 128, 2, True, True)
            result["few_heads"].append({
                "workload": f"KDA chunked prefill B={fb} T={ft} H=HV={fh} K=V=128 bf16, "
                            "initial state N(0, 0.1)",
                "default_ms": a_avg, "default_median_ms": a_med,
                "default_tokens_per_s": fb * ft / (a_avg * 1e-3),
                "default_roofline_frac": fbytes / (a_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "plain_two_kernel_ms": p_avg, "plain_two_kernel_median_ms": p_med,
                "workspace_bytes": segs, "segments": nseg,
                "kernel": "kda_chunk_fwd (segmented when few heads) against "
                          "kda_chunk_fwd_segmented(segments=1)"})
            del fd

    # ---------------- decay gate (forward and backward) on the prefill layer's g shape
    if not args.no_gate:
        from synth import gate_inputs
        log(f"bench: timing the decay gate on the {PREFILL_WORKLOAD} gate shape")
        gi = gate_inputs(c["B"], c["T"], c["HV"], c["K"], "bf16", seed=4322)
        gx, gA, gb, gdg = (gi[n].to(dev) for n in ("x", "A_log", "dt_bias", "dg"))
        del gi
        gate_fwd, gate_bwd = gate_abi_calls(kda, gx, gA, gb, gdg, -5.0, torch)
        f_avg, f_med, f_min = time_launches(gate_fwd, args.steps, args.warmup, torch, settle)
        r_avg, r_med, r_min = time_launches(gate_bwd, args.steps, args.warmup, torch, settle)
        # the gate fused into the prefill, against the gate then the prefill
        fused = lambda: kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], gx, gA, gb, d["beta"], -5.0,
                                                d["scale"], d["initial_state"])
        unfused = lambda: kda.kda_chunk_fwd(d["q"], d["k"], d["v"], kda.kda_gate_fwd(gx, gA, gb, -5.0),
                                            d["beta"], d["scale"], d["initial_state"])
        u_avg, u_med, _ = time_launches(unfused, args.steps, args.warmup, torch, settle)
        z_avg, z_med, _ = time_launches(fused, args.steps, args.warmup, torch, settle)
        n = gx.numel()
        fbytes, rbytes = gate_algorithmic(n, c["HV"], c["K"])
        result["gate"] = {
            "workload": f"safe gate (lower bound -5) on x [B={c['B']}, T={c['T']}, "
                        f"HV={c['HV']}, K={c['K']}] bf16, A_log [HV] and dt_bias [HV, K] fp32",
            "fwd": {"ms_per_call": f_avg, "median_ms": f_med, "min_ms": f_min,
                    "roofline": {"bound": "hbm", "achieved": fbytes / (f_avg * 1e-3) / 1e9,
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": fbytes / (f_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                 "kernel": "kda::gate::fwd_kernel<bf16>",
                                 "algorithmic_bytes_per_launch": fbytes}},
            "bwd": {"ms_per_call": r_avg, "median_ms": r_med, "min_ms": r_min,
                    "roofline": {"bound": "hbm", "achieved": rbytes / (r_avg * 1e-3) / 1e9,
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": rbytes / (r_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                 "kernel": "kda::gate::bwd_kernel<bf16> + reduce_kernel "
                                           "(one kda_gate_bwd call)",
                                 "algorithmic_bytes_per_launch": rbytes}},
            "prefill_gated": {
                "workload": PREFILL_WORKLOAD + " with g made by the safe gate from x",
                "fused_ms": z_avg, "fused_median_ms": z_med,
                "fused_tokens_per_s": tokens / (z_avg * 1e-3),
                "gate_then_prefill_ms": u_avg, "gate_then_prefill_median_ms": u_med,
                "kernel": "kda_chunk_fwd_gated (factors_kernel with the gate + state_kernel) "
                          "against kda_gate_fwd + kda_chunk_fwd"},
        }
        del gx, gA, gb, gdg
    del d

    # ---------------- the timed calls against the oracle (the CPU leg's results)
    if baseline is not None:
        par = {}
        if args.cpu_tokens >= c["T"]:
            o, s = checked["prefill"]
            B, HV = c["B"], c["HV"]
            o_ref = np.stack([np.stack([ref["prefill"][(b, hv)][0] for hv in range(HV)], 1) for b in range(B)])
            s_ref = np.stack([np.stack([ref["prefill"][(b, hv)][1] for hv in range(HV)]) for b in range(B)])
            par["prefill"] = {"heads": "all", "o": compare(o.double().numpy(), o_ref),
                              "final_state": compare(s.double().numpy(), s_ref)}
        if "long" in checked:
            par["prefill_long"] = {f"b={b} hv={hv}": {
                "o": compare(checked["long"][(b, hv)][0].double().numpy(), ref["long"][(b, hv)][0]),
                "final_state": compare(checked["long"][(b, hv)][1].double().numpy(), ref["long"][(b, hv)][1])}
                for b, hv in samples["long"]}
        if "decode" in checked:
            _, bs, hs, o_ref, s_ref = ref["decode"]
            par["decode"] = {"heads": f"b in {bs.tolist()}, hv in {hs.tolist()}, all 64 steps",
                             "o": compare(checked["decode"][0], o_ref),
                             "final_state": compare(checked["decode"][1], s_ref)}
        if "backward" in checked:
            names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
            # gradients: RMS and row criteria; the per-element figure is reported, not asserted
            par["backward"] = {f"b={b} hv={hv}": {
                n: compare(x.double().numpy(), r, elem=False)
                for n, x, r in zip(names, checked["backward"][(b, hv)], ref["backward"][(b, hv)])}
                for b, hv in samples["backward"]}

        def passes(x):
            return x["pass"] if "pass" in x else all(passes(v) for v in x.values() if isinstance(v, dict))

        par["all_pass"] = passes(par)
        if not par["all_pass"]:
            log("bench: PARITY FAILURE in a timed configuration (see cpu_baseline.parity_of_timed_calls)")
        baseline["parity_of_timed_calls"] = par
        result["cpu_baseline"] = baseline

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
