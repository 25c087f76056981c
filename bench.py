"""Benchmark of the KDA forward on one MI355X.

A step is one chunked prefill (kda_chunk_fwd) over the prefill workload
B=4, T=8192, H=HV=16, K=V=128, bf16 inputs, fp32 state, chunk 64 (synthetic,
seeded; the 16 x 128 head layout and 8,192-token context of the pages' KDA
layers). `value` is prefill tokens/s (B*T per step). The decode step
(kda_recurrent_step, 64 consecutive steps on a B=256, H=HV=16, K=V=128 fp32
state cache) is timed in the same run and reported under "decode", and the chunked
backward (kda_chunk_bwd: dq, dk, dv, dg, dbeta, dh0 of the prefill workload for a
seeded dO) under "backward", and the decay gate (kda_gate_fwd / kda_gate_bwd on the
same layer's [B, T, HV, K] gate input) under "gate".

Timing uses HIP events recorded on the stream the kernels are launched on,
bracketed by device synchronisation. One prefill call is two kernels on that
stream (factors_kernel: the state-independent per-chunk factors for all chunks;
state_kernel: the sequential state pass), timed together. The roofline object
prices the call's algorithmic bytes (q, k, v, g, beta read once, o and the final
state written once) against MI355X's 8 TB/s HBM3E peak; the decode object prices
its algorithmic bytes (state read + write, plus the token vectors) the same way.
A 1 GiB device copy is timed in the same run as the measured HBM ceiling.
The decode steps and the gate calls, whose kernels take 50-90 us, are issued
through the C ABI with their outputs allocated up front (checked bit for bit
against the Python binding first), so that the host's per-call work in the
binding does not leave gaps between the timed kernels.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2516.6     # MI355X dense bf16 MFMA, published (no sparsity)
METRIC = "KDA prefill tokens/s + MFMA util (H=16,K=V=128,T=8192); decode state HBM GB/s"
PREFILL_KERNELS = ["kda::wy::factors_kernel<128, false, false, false>", "kda::wy::state_kernel<128, 2, false>"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_traffic.json")
MEASURED_SOURCES = ["kda_chunk_wy.hip", "kda_device.h"]
PREFILL_WORKLOAD = "prefill-B4-T8192-H16-K128"
DECODE_WORKLOAD = "decode-B256-H16-K128-64steps"


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


def source_hash():
    """Hash of the sources of the measured prefill kernels (traffic counters go stale when
    they change)."""
    h = hashlib.sha256()
    for name in MEASURED_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_67_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_record():
    """The committed rocprofv3 --pmc record for the prefill kernels, if the kernel source has
    not changed since the counters were taken; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("source_sha256_16") == source_hash() else None


def measured_traffic():
    """HBM bytes per prefill launch from the counter record, or None."""
    rec = counter_record()
    return rec.get("bytes_per_launch") if rec else None


def time_launches(fn, steps, warmup, torch):
    """Average launch duration in ms over `steps` back-to-back launches, timed by two events on
    the launch stream around all of them; then, in a second pass of `steps` launches with an
    event after each, the per-launch median and minimum."""
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


def copy_ceiling(torch, nbytes=1 << 30, reps=5):
    """Measured HBM ceiling: GB/s of a 1 GiB device-to-device copy (read + write bytes)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(tokens, gpu_out=None):
    """The fp64 oracle on the first `tokens` tokens of the prefill workload (all batches and
    heads), single-threaded, on this host. With gpu_out = (o, final_state) of the timed GPU
    call on the whole workload (CPU tensors) and the whole workload timed, the oracle's result
    also checks that call: RMS(err) <= 2e-2 RMS(ref) over each tensor and every row within
    2e-2 (RMS_row(ref) + RMS(ref)), the bf16 reading the parity tests use."""
    import numpy as np
    from oracle import recurrent
    from synth import workload_inputs

    inp = workload_inputs(PREFILL_WORKLOAD)
    sl = {k: (v[:, :tokens] if k in ("q", "k", "v", "g", "beta") else v) for k, v in inp.items()}
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except ImportError:  # pragma: no cover
        limiter = None
    t0 = time.perf_counter()
    o_ref, s_ref = recurrent(**sl)
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    B = inp["q"].shape[0]
    out = dict(value=B * tokens / dt, unit="tokens/s", cores=1, kind="oracle",
               sample=f"first {tokens} of the 8192 tokens of the prefill workload, all B=4 x 16 heads "
                      f"({B * tokens} tokens, {dt:.1f} s, numpy float64, one thread)")
    if gpu_out is not None and tokens == inp["q"].shape[1]:
        checks = {}
        for name, got, ref in (("o", gpu_out[0], o_ref), ("final_state", gpu_out[1], s_ref)):
            got = got.double().numpy()
            err = got - ref
            rms = float(np.sqrt(np.mean(ref ** 2)))
            rel = float(np.sqrt(np.mean(err ** 2))) / rms
            row = float(np.max(np.sqrt(np.mean(err ** 2, axis=-1)) /
                               (np.sqrt(np.mean(ref ** 2, axis=-1)) + rms)))
            checks[name] = {"rms_err_over_rms": rel, "worst_row": row,
                            "pass": bool(rel <= 2e-2 and row <= 2e-2)}
        out["parity_of_timed_call"] = checks
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-reps", type=int, default=3)
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-gate", action="store_true")
    ap.add_argument("--no-segmented", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=5)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU code: it would shard by (batch, value head) with no "
              "communication).", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_67_amd as kda
    from synth import WORKLOADS, workload_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------- prefill workload
    c = WORKLOADS[PREFILL_WORKLOAD]
    log(f"bench: generating prefill workload {PREFILL_WORKLOAD}")
    inp = workload_inputs(PREFILL_WORKLOAD)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    del inp

    def prefill():
        return kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                                 d["initial_state"], True, c["chunk"])

    o, s = prefill()
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all(), "non-finite prefill output"
    checked = (o.cpu(), s.cpu()) if not args.no_cpu_baseline else None  # checked by the oracle leg
    log(f"bench: timing {args.steps} prefill steps after {args.warmup} warmup")
    avg_ms, med_ms, min_ms = time_launches(prefill, args.steps, args.warmup, torch)
    tokens = c["B"] * c["T"]
    byts, flops = prefill_algorithmic(c["B"], c["T"], c["H"], c["HV"], c["K"], c["V"], 2,
                                      c["init_state"], True)
    achieved = byts / (avg_ms * 1e-3) / 1e9
    tflops = flops / (avg_ms * 1e-3) / 1e12
    traffic = measured_traffic()
    del o, s
    ceiling = copy_ceiling(torch)
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
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": " + ".join(PREFILL_KERNELS) + " (one kda_chunk_fwd call)",
                     "algorithmic_bytes_per_launch": byts,
                     "avg_launch_ms": avg_ms, "median_launch_ms": med_ms, "min_launch_ms": min_ms,
                     "roofline_frac": t_bound * 1e3 / avg_ms,
                     "measured_copy_ceiling_gbs": ceiling, "frac_of_copy_ceiling": achieved / ceiling},
        "mfma": {"algorithmic_tflops": tflops, "peak_tflops": MFMA_BF16_PEAK_TFS,
                 "frac": tflops / MFMA_BF16_PEAK_TFS, "algorithmic_flops_per_launch": flops},
    }
    rec = counter_record()
    if rec and "issued_bf16_flops_per_launch" in rec:
        # issued MFMA work (full tiles, V-tile duplication) from the counter record, priced at
        # this run's call time; and the counters' own MFMA-busy fraction
        issued = rec["issued_bf16_flops_per_launch"]
        result["mfma"].update({"issued_tflops_counters": issued / (avg_ms * 1e-3) / 1e12,
                               "issued_frac_counters": issued / (avg_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
                               "issued_bf16_flops_per_launch": issued,
                               "mfma_busy_frac_counters": rec.get("mfma_busy_frac")})

    # ---------------- decode workload
    if not args.no_decode:
        c3 = WORKLOADS[DECODE_WORKLOAD]
        log(f"bench: generating decode workload {DECODE_WORKLOAD}")
        dinp = workload_inputs(DECODE_WORKLOAD)
        dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in dinp.items()}
        del dinp
        state = dd["state"].clone()
        steps = c3["steps"]
        views = [[dd[n][t] for n in ("q", "k", "v", "g", "beta")] for t in range(steps)]
        # the steps go through the C ABI with every o allocated up front: a step's kernel
        # takes about 80 us, close to what the binding's per-call checks and allocation cost
        # the host, so calls through the binding would leave gaps between the kernels
        import ctypes
        lib = kda.library()
        outs = [torch.empty_like(dd["v"][t]) for t in range(steps)]
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        stream = torch.cuda.current_stream()
        sp = ctypes.c_void_p(stream.cuda_stream)
        B3, H3, K3 = dd["q"][0].shape
        HV3, V3 = dd["v"][0].shape[1], dd["v"][0].shape[2]
        step_args = [tuple(p(x) for x in views[t]) + (p(state), p(outs[t]), B3, H3, HV3, K3, V3,
                                                      float(dd["scale"]), kda._DTYPE[dd["q"].dtype], sp)
                     for t in range(steps)]

        def one(t):
            return lib.kda_recurrent_step(*step_args[t])

        # warm-up on a scratch copy of the state; the C ABI's first step matches the binding's
        assert one(0) == kda.KDA_OK, "kda_recurrent_step failed"
        state.copy_(dd["state"])
        one(0)
        s_abi, o_abi = state.clone(), outs[0].clone()
        state.copy_(dd["state"])
        o_ref = kda.kda_recurrent_step(*views[0], state, dd["scale"])
        torch.cuda.synchronize()
        assert torch.equal(o_abi, o_ref) and torch.equal(s_abi, state), "C ABI and binding differ"
        del s_abi, o_abi, o_ref
        for t in range(3):
            one(t)
        per_step = []
        totals = []
        for _ in range(args.decode_reps):  # 64 steps between two events
            state.copy_(dd["state"])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for t in range(steps):
                one(t)
            e1.record(stream)
            torch.cuda.synchronize()
            totals.append(e0.elapsed_time(e1))
        state.copy_(dd["state"])  # per-step durations: one more pass, an event after each step
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for t in range(steps):
            one(t)
            ev[t + 1].record(stream)
        torch.cuda.synchronize()
        per_step = [ev[t].elapsed_time(ev[t + 1]) for t in range(steps)]
        step_ms = min(totals) / steps
        dbytes = decode_algorithmic(c3["B"], c3["H"], c3["HV"], c3["K"], c3["V"], 2)
        gbs = dbytes / (step_ms * 1e-3) / 1e9
        per_step.sort()
        result["decode"] = {
            "workload": "KDA decode, 64 consecutive steps, B=256 H=HV=16 K=V=128, bf16 vectors, "
                        "fp32 state [256,16,128,128] updated in place",
            "value": gbs, "unit": "GB/s", "ms_per_step": step_ms,
            "tokens_per_s": c3["B"] / (step_ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "frac_of_copy_ceiling": gbs / ceiling,
                         "kernel": "decode_step_kernel",
                         "algorithmic_bytes_per_launch": dbytes,
                         "median_launch_ms": per_step[len(per_step) // 2]},
        }
        del dd, state, views, outs, step_args

    # ---------------- chunked backward on the prefill workload
    if not args.no_backward:
        log(f"bench: timing {args.backward_steps} backward calls on {PREFILL_WORKLOAD}")
        gen = torch.Generator(device=dev).manual_seed(4321)
        dout = torch.randn(d["v"].shape, generator=gen, device=dev).to(torch.bfloat16)

        def backward():
            return kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dout, d["scale"],
                                     d["initial_state"], None, c["chunk"])

        grads = backward()
        torch.cuda.synchronize()
        assert all(torch.isfinite(x.float()).all() for x in grads), "non-finite gradient"
        del grads
        b_avg, b_med, b_min = time_launches(backward, args.backward_steps, 1, torch)
        bbytes = backward_algorithmic(c["B"], c["T"], c["H"], c["HV"], c["K"], c["V"], 2)
        bgbs = bbytes / (b_avg * 1e-3) / 1e9
        result["backward"] = {
            "workload": PREFILL_WORKLOAD + ", seeded dO, gradients of every input and of the "
                        "initial state",
            "ms_per_call": b_avg, "median_ms": b_med, "min_ms": b_min,
            "tokens_per_s": tokens / (b_avg * 1e-3),
            "roofline": {"bound": "hbm", "achieved": bgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bgbs / HBM_PEAK_GBS,
                         "kernel": "kda::bwd prep_kernel + fwd_sweep_kernel + rev_sweep_kernel + "
                                   "local_kernel (one kda_chunk_bwd call)",
                         "algorithmic_bytes_per_launch": bbytes},
        }
        del dout

    # ---------------- few heads, long sequence: the segmented prefill against the plain path
    if not args.no_segmented:
        from synth import prefill_inputs
        result["few_heads"] = []
        for (fb, ft, fh) in ((1, 32768, 4), (1, 32768, 8)):
            log(f"bench: few heads B={fb} T={ft} H=HV={fh}")
            fi = prefill_inputs(fb, ft, fh, fh, 128, 128, "bf16", True, seed=4323)
            fd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in fi.items()}
            del fi
            segs = kda.library().kda_chunk_fwd_workspace_size(fb, ft, fh, fh, 128, 128, 64, 1)
            auto = lambda: kda.kda_chunk_fwd(fd["q"], fd["k"], fd["v"], fd["g"], fd["beta"],
                                             fd["scale"], fd["initial_state"])
            plain = lambda: kda.kda_chunk_fwd_segmented(fd["q"], fd["k"], fd["v"], fd["g"],
                                                        fd["beta"], 1, fd["scale"],
                                                        fd["initial_state"])
            a_avg, a_med, _ = time_launches(auto, args.steps, args.warmup, torch)
            p_avg, p_med, _ = time_launches(plain, args.steps, args.warmup, torch)
            fbytes, _ = prefill_algorithmic(fb, ft, fh, fh, 128, 128, 2, True, True)
            result["few_heads"].append({
                "workload": f"KDA chunked prefill B={fb} T={ft} H=HV={fh} K=V=128 bf16, "
                            "initial state N(0, 0.1)",
                "default_ms": a_avg, "default_median_ms": a_med,
                "default_tokens_per_s": fb * ft / (a_avg * 1e-3),
                "default_roofline_frac": fbytes / (a_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "plain_two_kernel_ms": p_avg, "plain_two_kernel_median_ms": p_med,
                "workspace_bytes": segs,
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
        f_avg, f_med, f_min = time_launches(gate_fwd, args.steps, args.warmup, torch)
        r_avg, r_med, r_min = time_launches(gate_bwd, args.steps, args.warmup, torch)
        # the gate fused into the prefill, against the gate then the prefill
        fused = lambda: kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], gx, gA, gb, d["beta"], -5.0,
                                                d["scale"], d["initial_state"])
        unfused = lambda: kda.kda_chunk_fwd(d["q"], d["k"], d["v"], kda.kda_gate_fwd(gx, gA, gb, -5.0),
                                            d["beta"], d["scale"], d["initial_state"])
        u_avg, u_med, _ = time_launches(unfused, args.steps, args.warmup, torch)
        z_avg, z_med, _ = time_launches(fused, args.steps, args.warmup, torch)
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

    # ---------------- oracle on the host
    if not args.no_cpu_baseline:
        log(f"bench: timing the CPU oracle on {args.cpu_tokens} tokens")
        result["cpu_baseline"] = cpu_baseline(args.cpu_tokens, checked)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
