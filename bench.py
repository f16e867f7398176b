"""Benchmark of the ParaRNN hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of seeded synthetic input, with the
inputs already resident in HBM.  Default workload: the long-context diagonal GRU (bf16 storage,
fp32 arithmetic, B=1, T=131072, D=1024): a Newton solve from the zero guess until the max
residual is below 1e-5 (at most 8 iterations), then the reverse-scan VJP for an upstream gradient
dL/dh ~ N(0, 1).  Other workloads (--workload 0..3) time one Newton solve or one linear scan.

--variants times the same workload with the options built on the method (warm start, the measured
budget K*(T), packed sequences) and prints one JSON line per variant instead; --kstar times the
automatic budget over a grid of sequence lengths; --slstm and --head time the diagonal sLSTM and the
head-wise block GRU.  None of them is the benchmark line.

Prints ONE JSON line.  value = channel-tokens/s = B*T*D*K / (seconds per step), K the Newton
iterations the solve ran (a linear scan counts K = 1).  The timed solves use the library's own launch
length (fuse_iters = 0: in tolerance mode a speculative fused launch of K*(T) + 1 iterations, its
re-run launch, then one launch per further iteration).  fuse_prev times the same step with the launch
length set to the iteration count of the solve before it (a loop of solves can pass that; the result is
the same bit for bit), for context only.

roofline: HBM, as the method's bytes: a Newton iteration reads the gate inputs and H^k and writes
H^{k+1} (GRU bf16: 6 + 4 + 4 = 14 B per element; iteration 0 of a zero start reads no H^k: 10 B;
LSTM fp32: 16 + 8 + 8 = 32, 24), the linear scan reads a, b and writes h (12 B).  achieved = those
bytes for the iterations the solve ran x elements / the duration of the solve's launches (HIP events on
the launch stream around every solve of the timed region).  The fused launch keeps the trajectory on
chip between iterations, so its effective rate can exceed what it moves: its real HBM bytes are
roofline.traffic (rocprofv3 counters, when taken on this source), and roofline.alu rates the same time
in algorithmic flops (fma = 2, add / mul / exp2 / rcp = 1) against the 78.6 TFLOP/s vector fp32 peak
that code without packed-fp32 instructions can reach.  roofline.copy_gbs is a device-to-device copy's
bandwidth on the same GPU, for context; per_iteration_kernel is the one-launch-per-iteration kernel's
HBM figure, timed after the timed region.  cpu_baseline: the fp64 CPU oracle on a bounded sample of
channels of the same workload on every core this process may use (value: its Newton solve + VJP;
unroll_value: its sequential unroll, the exact solution; nproc: the host's core count).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "channel-tokens/s per Newton solve (B*T*D*K/s) + achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
VALU_FP32_PEAK_TFLOPS = 157.3   # MI355X vector fp32 (256 CUs, 2.4 GHz; the packed-fp32 figure)
# 256 CUs x 4 SIMDs x 16 lanes x 2 flops (fma) x 2.4 GHz: what code without packed-fp32 instructions can reach
VALU_FP32_NONPACKED_TFLOPS = 78.6


def iteration_bytes(cell: str, dtype: str, first: bool) -> int:
    """HBM bytes per element of one Newton iteration: the gate inputs, H^k (not for iteration 0 of a zero
    start) and H^{k+1}."""
    esz = 2 if dtype == "bf16" else 4
    G, S = (3, 1) if cell == "gru" else (4, 2)
    return G * esz + (0 if first else 4 * S) + 4 * S


def solve_bytes(cell: str, dtype: str, iters: int) -> int:
    """HBM bytes per element of a zero-start solve of `iters` iterations, iteration by iteration."""
    return iteration_bytes(cell, dtype, True) + (iters - 1) * iteration_bytes(cell, dtype, False)

# algorithmic flops of one element-iteration of a Newton solve (fma = 2, add / mul / exp2 / rcp = 1):
#   GRU: cell value and Jacobian 44, scan element (residual, b = f - J h) 3, composition 3, update 2
#   LSTM: cell 64, elements 10, 2x2 composition 20, update 8
FLOPS_PER_ELEM_ITER = {"gru": 52, "lstm": 102}


# algorithmic HBM bytes per element of one launch of the dominant kernel
#   GRU steady iteration: read U (3 planes) + read H^k + write H^{k+1}
#   LSTM steady iteration: read U (4 planes) + read (c, h)^k + write (c, h)^{k+1}
#   linear scan: read a, b + write h
def algo_bytes(cell: str, dtype: str) -> int:
    esz = 2 if dtype == "bf16" else 4
    if cell == "gru":
        return 3 * esz + 4 + 4
    if cell == "lstm":
        return 4 * esz + 8 + 8
    return 2 * esz + 4


def vjp_bytes(cell: str, dtype: str) -> int:
    """VJP kernel: read U, H, g; write dU (fp32, G planes)."""
    esz = 2 if dtype == "bf16" else 4
    G, S = {"gru": (3, 1), "lstm": (4, 2), "linear": (2, 1)}[cell]
    return G * esz + 4 * S + 4 + 4 * G


def source_hash() -> str:
    """sha256 of the kernel source's code: comments, trailing blanks and empty lines removed, so that a
    comment edit leaves a counter record valid and any code edit invalidates it."""
    import hashlib
    import re
    with open(os.path.join(ROOT, "nonlinear_rnn_solve_amd", "csrc", "pararnn.hip")) as f:
        txt = f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    lines = [re.sub(r"//.*$", "", line).rstrip() for line in txt.splitlines()]
    return hashlib.sha256("\n".join(line for line in lines if line).encode()).hexdigest()


def measured_record(key: str):
    """The committed counter summary of a workload's dominant kernel (profiles/traffic.json), or None when
    that summary was taken on other source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash():
        return None
    return rec.get("kernels", {}).get(key)


def measured_traffic(key: str):
    """HBM bytes per launch of the dominant kernel from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE per dispatch, each scaled by what the same counter reads for a copy of known size), or None
    when that summary was taken on other source."""
    k = measured_record(key)
    return None if k is None else float(k["bytes_per_launch"])


def cpu_threads() -> int:
    """Every core this process may run on (its CPU affinity), for the oracle's worker threads."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        return max(1, os.cpu_count() or 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-channels", type=int, default=0, help="channels in the CPU-baseline sample (0: auto)")
    ap.add_argument("--variants", action="store_true", help="time warm start / K* budget / packed variants")
    ap.add_argument("--kstar", action="store_true", help="time the automatic budget over a grid of lengths")
    ap.add_argument("--slstm", action="store_true", help="time the diagonal sLSTM solve and VJP over a grid of lengths")
    ap.add_argument("--head", action="store_true", help="time the head-wise block GRU solve and VJP")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the hot path, time a plain device-to-device copy of this many MiB "
                         "(same-box bandwidth context, and the known-size kernel that calibrates HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only; --gpus %d is not supported (independent channels shard "
              "across GPUs without communication; no multi-GPU path is built)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from nonlinear_rnn_solve_amd import api, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_mib > 0:
        copy_bench(torch, dev, args)
        return
    if args.kstar:
        kstar_bench(torch, dev, args)
        return
    if args.head:
        return head_bench(torch, dev, args)
    if args.slstm:
        slstm_bench(torch, dev, args)
        return
    wl = synth.WORKLOADS[args.workload]
    inp = synth.workload_inputs(wl)
    if args.variants:
        variants_bench(torch, dev, args, wl, inp)
        return
    if wl.dtype == "bf16":
        pre = [torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).to(dev) for p in inp.pre]
    else:
        pre = [torch.from_numpy(p).to(dev) for p in inp.pre]
    w = torch.from_numpy(inp.w).to(dev) if inp.w is not None else None
    b = torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None
    g = torch.from_numpy(inp.g).to(dev) if inp.g is not None else None
    N = wl.B * wl.T * wl.D
    out = torch.empty((inp.S, wl.B, wl.T, wl.D), dtype=torch.float32, device=dev)
    if wl.cell == "linear":
        out = out[0]

    stream = torch.cuda.current_stream(dev)
    iter_events = []     # per step: list of (k, start, end) around the solve's (or the scan's) launches
    vjp_events = []

    # Timed steps are enqueued back to back with no host synchronisation (as a training loop would run
    # them): the iteration count is taken from a reported solve before and after the timed region (the
    # solve is deterministic, so every step runs the same launches), and the per-launch HIP events
    # recorded in the timed region give the kernel durations.
    def step(record, report=False):
        rec = []
        if wl.cell == "linear":
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            api.linear_scan(pre[0], pre[1], out=out)
            e1.record(stream)
            rec.append([0, e0, e1])
            iters = 1
        else:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            _, rep = api.newton_solve(wl.cell, pre, w, b, max_iters=wl.max_iters, tol=wl.tol, out=out,
                                      report=report, fuse_iters=fuse[0])
            e1.record(stream)
            rec.append([0, e0, e1])   # the solve's launches
            iters = rep.iters if rep is not None else None
            if wl.vjp:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                api.scan_vjp(wl.cell, pre, out, g, w, b, want_s0=False)
                e1.record(stream)
                if record:
                    vjp_events.append((e0, e1))
        if record:
            iter_events.append(rec)
        return iters

    fuse = [0]   # the library's own launch length
    for _ in range(args.warmup):
        step(False)
    iters = step(False, report=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    if step(False, report=True) != iters:
        raise RuntimeError("the iteration count changed between steps")

    # the solve's launches (or the scan), timed by HIP events on the launch stream in every timed step
    kern_ms = float(np.mean([e0.elapsed_time(e1) for rec in iter_events for k, e0, e1 in rec]))
    value = N * iters / (ms_per_step * 1e-3)
    traffic = measured_traffic(wl.name)
    config = {"workload": wl.name, "cell": wl.cell, "B": wl.B, "T": wl.T, "D": wl.D, "storage": wl.dtype,
              "tol": wl.tol, "max_iters": wl.max_iters, "iters": iters, "vjp": wl.vjp}
    if wl.cell == "linear":
        per_elem = algo_bytes(wl.cell, wl.dtype)
        achieved = per_elem * N / (kern_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": "k_tile<LinearOp>",
                    "bytes_per_elem": per_elem, "algorithmic_bytes": per_elem * N, "kernel_ms": kern_ms,
                    "copy_gbs": copy_gbs(torch, dev)}
    else:
        config["fuse_iters"] = 0
        per_elem = solve_bytes(wl.cell, wl.dtype, iters)
        achieved = per_elem * N / (kern_ms * 1e-3) / 1e9
        flops = FLOPS_PER_ELEM_ITER[wl.cell] * N * iters
        tflops = flops / (kern_ms * 1e-3) / 1e12
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                    "kernel": "the Newton solve's launches (k_fused<NewtonOp> over the speculated iterations, "
                              "its re-run launch, k_tile<NewtonOp> for each further one)",
                    "bytes_per_elem": per_elem,
                    "bytes_per_elem_note": "%d iterations: %d B for iteration 0 (no H^0 read) + %d B per later one"
                                           % (iters, iteration_bytes(wl.cell, wl.dtype, True),
                                              iteration_bytes(wl.cell, wl.dtype, False)),
                    "algorithmic_bytes": per_elem * N, "kernel_ms": kern_ms,
                    "frac_note": "effective: the method's bytes for one HBM pass per iteration over the solve's "
                                 "time; the fused pass reads the gate inputs once for all its iterations and keeps "
                                 "the trajectory on chip, so a value above 1 is the margin over that bound, and the "
                                 "pass is bound by vector ALU issue instead (alu, valu_busy)",
                    "alu": {"achieved": tflops, "peak": VALU_FP32_NONPACKED_TFLOPS, "unit": "TFLOP/s",
                            "frac": tflops / VALU_FP32_NONPACKED_TFLOPS,
                            "flops_per_elem_iter": FLOPS_PER_ELEM_ITER[wl.cell], "algorithmic_flops": flops,
                            "issue": (measured_record(wl.name) or {}).get("issue")},
                    "copy_gbs": copy_gbs(torch, dev)}
    line = {
        "metric": METRIC, "value": value, "unit": "channel-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": config, "roofline": roofline,
    }
    if vjp_events:
        vms = float(np.mean([a.elapsed_time(b2) for a, b2 in vjp_events]))
        line["vjp"] = {"ms": vms, "bytes_per_elem": vjp_bytes(wl.cell, wl.dtype),
                       "gbs": vjp_bytes(wl.cell, wl.dtype) * N / (vms * 1e-3) / 1e9,
                       "frac_hbm": vjp_bytes(wl.cell, wl.dtype) * N / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if wl.cell != "linear":
        # context, after the timed region: the same step with the launch length set to the previous solve's
        # iteration count (one fused launch for the whole solve), and the one-launch-per-iteration kernel
        fuse[0] = min(iters, api.MAX_FUSE)
        if step(False, report=True) != iters:
            raise RuntimeError("the iteration count changed with the fused launch length")
        iter_events.clear()
        vjp_events.clear()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(True)
        torch.cuda.synchronize()
        pm = (time.perf_counter() - t0) * 1e3 / args.steps
        pk = float(np.mean([e0.elapsed_time(e1) for rec in iter_events for k, e0, e1 in rec]))
        line["fuse_prev"] = {"fuse_iters": fuse[0], "ms_per_step": pm, "value": N * iters / (pm * 1e-3),
                             "solve_ms": pk, "gbs": per_elem * N / (pk * 1e-3) / 1e9,
                             "frac_hbm": per_elem * N / (pk * 1e-3) / 1e9 / HBM_PEAK_GBS}
        _, _, it_ms = time_solve(torch, api, wl.cell, pre, w, b, g, out, 1, 1, max_iters=wl.max_iters,
                                 tol=wl.tol, fuse_iters=1)
        pe = algo_bytes(wl.cell, wl.dtype)
        gbs = pe * N / (it_ms * 1e-3) / 1e9
        line["per_iteration_kernel"] = {"kernel": "k_tile<NewtonOp> (iterations k>=1, fuse_iters=1)", "ms": it_ms,
                                        "bytes_per_elem": pe, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, inp, iters, args.cpu_channels)
    print(json.dumps(line), flush=True)


def device_inputs(torch, dev, inp):
    if inp.dtype == "bf16":
        pre = [torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).to(dev) for p in inp.pre]
    else:
        pre = [torch.from_numpy(p).to(dev) for p in inp.pre]
    w = torch.from_numpy(inp.w).to(dev) if inp.w is not None else None
    b = torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None
    g = torch.from_numpy(inp.g).to(dev) if inp.g is not None else None
    return pre, w, b, g


def time_solve(torch, api, cell, pre, w, b, g, out, steps, warmup, vjp=False, **opts):
    """Mean wall time of one solve (+ VJP) through the plain entry point (fused as opts ask), its
    iteration count, and the mean duration of the steady-state iteration kernel of one launch per
    iteration (a few extra solves through the step-wise entry points, HIP events on the launch stream)."""
    stream = torch.cuda.current_stream(out.device)
    recs = []

    def one(record, report=False, hooked=False):
        rec = []

        def hook(k, phase):
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(stream)
            if phase == "before":
                rec.append([k, ev, None])
            else:
                rec[-1][2] = ev
        _, rep_ = api.newton_solve(cell, pre, w, b, out=out, on_iteration=hook if hooked else None, report=report,
                                   **opts)
        if vjp:
            api.scan_vjp(cell, pre, out, g, w, b, want_s0=False, cu_seqlens=opts.get("cu_seqlens"))
        if record:
            recs.append(rec)
        return rep_.iters if rep_ is not None else None
    for _ in range(warmup):
        one(False)
    iters = one(False, report=True)       # the solve is deterministic: every timed step runs these launches
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one(False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    if one(False, report=True) != iters:
        raise RuntimeError("the iteration count changed between solves")
    for _ in range(3):
        one(True, hooked=True)
    torch.cuda.synchronize()
    # steady-state iterations (k >= 1) when there are any: iteration 0 of a zero start reads no iterate
    durs = [e0.elapsed_time(e1) for rec in recs for k, e0, e1 in rec if (1 if iters > 1 else 0) <= k < iters]
    return ms, iters, float(np.mean(durs))


def variants_bench(torch, dev, args, wl, inp):
    """The workload's solve (and VJP) with each option the method adds, one JSON line each."""
    from nonlinear_rnn_solve_amd import api, synth
    pre, w, b, g = device_inputs(torch, dev, inp)
    N = wl.B * wl.T * wl.D
    out = torch.empty((inp.S, wl.B, wl.T, wl.D), dtype=torch.float32, device=dev)
    cu = synth.packed_offsets(wl.T, 2700, 2048)
    tcu = torch.from_numpy(cu).to(dev)
    tol = wl.tol if wl.tol > 0 else 0.0
    base = dict(max_iters=wl.max_iters, tol=tol)
    _, rep = api.newton_solve(wl.cell, pre, w, b, out=out, **base)
    variants = [
        ("zero start, the library's launch length (benchmark line)", base),
        ("zero start, launch length = the previous solve's %d iterations" % rep.iters,
         dict(base, fuse_iters=min(rep.iters, api.MAX_FUSE))),
        ("zero start, one launch per iteration", dict(base, fuse_iters=1)),
        ("warm start", dict(base, warm_start=True)),
        ("measured budget K*(T), zero start", dict(max_iters=None)),
        ("measured budget K*(T), warm start", dict(max_iters=None, warm_start=True)),
        ("packed sequences, mean length 2048 (%d sequences)" % (len(cu) - 1), dict(base, cu_seqlens=tcu)),
    ]
    # one untimed pass of the first variant: the first one timed otherwise ran 2-7% slower than the same launches
    # timed second (a device still warming up)
    time_solve(torch, api, wl.cell, pre, w, b, g, out, args.steps, args.warmup, vjp=wl.vjp, **base)
    for name, opts in variants:
        ms, iters, kern = time_solve(torch, api, wl.cell, pre, w, b, g, out, args.steps, args.warmup,
                                     vjp=wl.vjp, **opts)
        per_elem = algo_bytes(wl.cell, wl.dtype)
        print(json.dumps({"workload": wl.name, "variant": name, "ms_per_solve": ms, "iters": iters,
                          "channel_tokens_per_s": N * iters / (ms * 1e-3), "vjp": wl.vjp,
                          "iteration_kernel_ms": kern,
                          "iteration_gbs": per_elem * N / (kern * 1e-3) / 1e9}), flush=True)


def kstar_bench(torch, dev, args):
    """Wall time of a solve at the measured budget K*(T), zero and warm start, on the grid of lengths
    the budget was measured on (B = 1, D = 1024; GRU bf16 gate inputs, LSTM fp32)."""
    from nonlinear_rnn_solve_amd import api, synth
    for cell, dtype in (("gru", "bf16"), ("lstm", "f32")):
        for T in (1024, 4096, 16384, 65536, 131072):
            inp = synth.make_inputs(cell, 1, T, 1024, dtype=dtype, seed=3000 + T // 1024 + (500 if cell == "lstm" else 0))
            pre, w, b, _ = device_inputs(torch, dev, inp)
            out = torch.empty((inp.S, 1, T, 1024), dtype=torch.float32, device=dev)
            for warm in (False, True):
                ms, iters, kern = time_solve(torch, api, cell, pre, w, b, None, out, args.steps, args.warmup,
                                             max_iters=None, warm_start=warm)
                print(json.dumps({"cell": cell, "storage": dtype, "B": 1, "T": T, "D": 1024,
                                  "init": "warm" if warm else "zero", "kstar": iters, "ms_per_solve": ms,
                                  "iteration_kernel_ms": kern,
                                  "channel_tokens_per_s": T * 1024 * iters / (ms * 1e-3)}), flush=True)
            del pre, out
            torch.cuda.empty_cache()


def slstm_bench(torch, dev, args):
    """The diagonal sLSTM (fp32, B=8, D=256, as in the pararnn-torch README's sLSTM benchmark) over a
    grid of lengths: 8 Picard sweeps, then Newton until the max residual is below 1e-5 (at most 40
    iterations in all), then the VJP.  One JSON line per length."""
    from nonlinear_rnn_solve_amd import api, synth
    B, D = 8, 256
    per_elem = 4 * 4 + 4 * 4 + 4 * 4          # U (4 planes) + (c, n, m, h)^k + (c, n, m, h)^{k+1}
    for T in (1024, 4096, 16384, 65536):
        inp = synth.make_inputs("slstm", B, T, D, seed=4000 + T // 1024, with_grad=True)
        pre, w, b, g = device_inputs(torch, dev, inp)
        out = torch.empty((4, B, T, D), dtype=torch.float32, device=dev)
        ms, iters, kern = time_solve(torch, api, "slstm", pre, w, b, g, out, args.steps, args.warmup, vjp=True,
                                     max_iters=40, tol=1e-5, picard_iters=8)
        _, rep_ = api.newton_solve("slstm", pre, w, b, out=out, max_iters=40, tol=1e-5, picard_iters=8,
                                   final_residual=True)
        stream = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        api.scan_vjp("slstm", pre, out, g, w, b, want_s0=False)
        e1.record(stream)
        torch.cuda.synchronize()
        N = B * T * D
        print(json.dumps({"cell": "slstm", "storage": "f32", "B": B, "T": T, "D": D, "picard": 8, "tol": 1e-5,
                          "iters": iters, "converged": rep_.converged, "final_residual": rep_.final_residual,
                          "ms_per_solve_and_vjp": ms, "iteration_kernel_ms": kern,
                          "iteration_gbs": per_elem * N / (kern * 1e-3) / 1e9, "vjp_ms": e0.elapsed_time(e1),
                          "channel_tokens_per_s": N * iters / (ms * 1e-3),
                          "cpu_oracle": slstm_oracle_rate(inp, 8)}), flush=True)
        del pre, out, g
        torch.cuda.empty_cache()


MFMA_FP32_PEAK_TFLOPS = 157.3


def head_bench(torch, dev, args):
    """The head-wise block GRU (head size 64, fp32) on three shapes: the pararnn-torch README's example
    (a head GRU of width 512 with 8 heads, on 4 sequences of 64 steps), a larger batch of such short
    sequences, and longer sequences.  Newton from the zero guess until the max residual is below 1e-5
    (at most 8 iterations), then the VJP.  The iteration is MFMA-bound: per step and head it forms the
    dense Jacobian block (A_c diag(s) A_r, 2 hs^3 flops) and multiplies it into the chunk's product
    (2 hs^3), so iteration_tflops = 4 hs^3 B T H / iteration time against the fp32 MFMA peak (the
    gate, carry and finishing matrix-vector work is counted in the time, not in the flops)."""
    from nonlinear_rnn_solve_amd import api, synth
    hs, D = 64, 512
    for B, T in ((4, 64), (16, 64), (16, 1024)):
        inp = synth.make_inputs("head_gru", B, T, D, seed=5000 + B + T, with_grad=True, head_size=hs)
        pre, w, b, g = device_inputs(torch, dev, inp)
        out = torch.empty((1, B, T, D), dtype=torch.float32, device=dev)
        ms, iters, kern = time_solve(torch, api, "head_gru", pre, w, b, g, out, args.steps, args.warmup, vjp=True,
                                     max_iters=8, tol=1e-5)
        ms_solve, _, _ = time_solve(torch, api, "head_gru", pre, w, b, g, out, args.steps, args.warmup,
                                    max_iters=8, tol=1e-5)
        flops = 4.0 * hs ** 3 * B * T * (D // hs)
        N = B * T * D
        cpu = head_oracle_rate(inp, iters)
        print(json.dumps({"cell": "head_gru", "storage": "f32", "B": B, "T": T, "D": D, "head_size": hs,
                          "tol": 1e-5, "iters": iters, "ms_per_solve": ms_solve, "ms_per_solve_and_vjp": ms,
                          "iteration_ms": kern, "iteration_tflops": flops / (kern * 1e-3) / 1e12,
                          "mfma_fp32_peak_tflops": MFMA_FP32_PEAK_TFLOPS,
                          "frac": flops / (kern * 1e-3) / 1e12 / MFMA_FP32_PEAK_TFLOPS,
                          "channel_tokens_per_s": N * iters / (ms * 1e-3), "cpu_oracle": cpu}), flush=True)
        del pre, out, g
        torch.cuda.empty_cache()


def head_oracle_rate(inp, iters):
    """The fp64 oracle's Newton solve + VJP on one batch row (every head, full T) of a head-GRU
    workload, as channel-tokens/s (B*T*D*K per second scaled to the sample), for context."""
    import oracle
    threads = cpu_threads()
    pre = [np.ascontiguousarray(p[:1]) for p in inp.pre]
    prob = oracle.Problem("head_gru", pre, inp.w, inp.bias, head_size=inp.head_size)
    t0 = time.perf_counter()
    H, res, k, conv, rc = oracle.newton(prob, 8, tol=1e-5, nthreads=threads)
    oracle.vjp(prob, H, np.ascontiguousarray(inp.g[:1]), want_lambda=False, nthreads=threads)
    sec = time.perf_counter() - t0
    return {"value": inp.T * inp.D * k / sec, "unit": "channel-tokens/s", "cores": threads, "kind": "oracle",
            "sample": "1 of %d batch rows, full T=%d, Newton (%d iterations) + VJP; %.2f s" % (inp.B, inp.T, k, sec)}


def slstm_oracle_rate(inp, picard, n_channels=64):
    """The fp64 oracle's sLSTM solve (Picard sweeps, then Newton to 1e-5) + VJP on a sample of channels at
    full T, as channel-tokens/s, for context."""
    import oracle
    threads = cpu_threads()
    ds = np.arange(min(n_channels, inp.D))
    pre = [np.ascontiguousarray(p[:1, :, ds]) for p in inp.pre]
    prob = oracle.Problem("slstm", pre, inp.w[:, ds], inp.bias[:, ds])
    t0 = time.perf_counter()
    H, res, k, conv, rc = oracle.newton(prob, 40, tol=1e-5, picard=picard, nthreads=threads)
    oracle.vjp(prob, H, np.ascontiguousarray(inp.g[:1, :, ds]), want_lambda=False, nthreads=threads)
    sec = time.perf_counter() - t0
    return {"value": len(ds) * inp.T * k / sec, "unit": "channel-tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d channels of batch row 0, full T=%d, %d updates + VJP; %.2f s" % (len(ds), inp.T, k, sec)}


def copy_gbs(torch, dev, mib=1024, reps=5):
    """Device-to-device copy bandwidth on this GPU (read + write bytes / time), for context."""
    n = mib * (1 << 20) // 4
    src = torch.empty(n, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def copy_bench(torch, dev, args):
    n = args.copy_mib * (1 << 20) // 4
    src = torch.randn(n, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = 2 * n * 4
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "ms": ms,
                      "gbs": nbytes / (ms * 1e-3) / 1e9, "steps": args.steps}), flush=True)


def cpu_baseline(wl, inp, iters, n_channels):
    """The fp64 oracle (as it stands) on a sample of channels of the same workload, full T."""
    import oracle
    threads = cpu_threads()
    if n_channels <= 0:
        # about 10-30 s of work: the oracle costs roughly 1e-7 s per element-iteration per thread
        per_ch = wl.T * (max(iters, 1) + (2 if wl.vjp else 0)) * 2.0e-7
        n_channels = int(max(threads, min(wl.B * wl.D, 15.0 * threads / per_ch)))
    rng = np.random.default_rng(0)
    all_ch = [(b, d) for b in range(wl.B) for d in range(wl.D)]
    pick = sorted(rng.choice(len(all_ch), size=min(n_channels, len(all_ch)), replace=False))
    bs = np.array([all_ch[i][0] for i in pick])
    ds = np.array([all_ch[i][1] for i in pick])
    pre = [np.ascontiguousarray(p[bs, :, ds].T[None]) for p in inp.pre]
    dt = oracle.BF16 if wl.dtype == "bf16" else oracle.F32
    t0 = time.perf_counter()
    if wl.cell == "linear":
        oracle.linear_scan(pre[0], pre[1], dtype=dt, nthreads=threads)
        k = 1
    else:
        prob = oracle.Problem(wl.cell, pre, inp.w[:, ds], inp.bias[:, ds], dtype=dt)
        H, res, k, conv, rc = oracle.newton(prob, wl.max_iters, tol=wl.tol, nthreads=threads)
        if wl.vjp:
            oracle.vjp(prob, H, np.ascontiguousarray(inp.g[bs, :, ds].T[None]), want_lambda=False, nthreads=threads)
    sec = time.perf_counter() - t0
    n = len(pick) * wl.T
    # the exact solution by the sequential fp64 unroll on the same sample, for context
    t1 = time.perf_counter()
    if wl.cell == "linear":
        oracle.linear_scan(pre[0], pre[1], dtype=dt, nthreads=threads)
    else:
        oracle.unroll(prob, nthreads=threads)
    usec = time.perf_counter() - t1
    return {"value": n * k / sec, "unit": "channel-tokens/s", "cores": threads, "nproc": os.cpu_count(),
            "kind": "oracle", "unroll_value": n / usec,
            "sample": "%d of %d channels, full T=%d, %s%s; %.1f s" % (
                len(pick), wl.B * wl.D, wl.T, "linear scan" if wl.cell == "linear" else
                "Newton (%d iterations)" % k, " + VJP" if wl.vjp else "", sec)}


if __name__ == "__main__":
    main()
