#!/usr/bin/env python3
"""Benchmark of the packed trellis-coded linear layer on one MI355X.

Default workload: fused gate/up + SwiGLU matvec, two 17408 x 5120 matrices,
k = 2, L = 12, T = 256; one step = one call at each M in 1, 2, 3, 4.  The
value is packed-code bytes per second over the whole step (inputs resident
in HBM; code buffers rotate over >= 1 GiB of replicas so the 256 MB
Infinity Cache cannot serve repeats).  Other workloads (--workload) print
the same JSON line for their own metric.

The JSON line carries:
  roofline      the dominant kernel's algorithmic bytes (or flops) per launch
                over its mean launch time (HIP events on the launch stream,
                every launch of the timed region), against the MI355X peak;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same
                workload on this host (a baseline, not a target).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode matvec GB/s of packed codes (% HBM peak) at M=1..4; prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
L, T = 12, 256
ROTATE_BYTES = 1 << 30


def _ensure_built():
    from trellis_coded_quantized_amd import LIB_PATH
    if not os.path.exists(LIB_PATH) or not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        import __graft_entry__
        __graft_entry__.build()


def _dev_tensors(np, torch, dev):
    def codes(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev)

    def half(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.float16)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    return codes, half, bf16


class EventTimer:
    """Per-launch HIP event pairs on the current (launch) stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __call__(self, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.append((a, b))

    def mean_ms(self):
        self.torch.cuda.synchronize()
        if not self.pairs:
            return float("nan")
        return sum(a.elapsed_time(b) for a, b in self.pairs) / len(self.pairs)


# ------------------------------------------------------------- workloads

def workload_gateup(args, np, torch, dev):
    import oracle
    import trellis_coded_quantized_amd as tq
    import trellis_inputs as ti

    w = ti.gateup()
    g, u = w.mats
    codes, half, bf16 = _dev_tensors(np, torch, dev)
    code_bytes = g.codes.nbytes + u.codes.nbytes
    nrep = max(1, math.ceil(ROTATE_BYTES / code_bytes))
    gcs = [codes(g.codes)]
    ucs = [codes(u.codes)]
    for _ in range(nrep - 1):
        gcs.append(gcs[0].clone())
        ucs.append(ucs[0].clone())
    gs, us, x = half(g.scales), half(u.scales), bf16(w.x[0])
    Ms = (1, 2, 3, 4)
    outs = {M: torch.empty((M, g.R), dtype=torch.bfloat16, device=dev) for M in Ms}
    state = {"i": 0}
    timer = EventTimer(torch)
    per_m = {M: EventTimer(torch) for M in Ms}

    def call(M):
        i = state["i"] % nrep
        state["i"] += 1
        tq.gateup_swiglu(gcs[i], gs, ucs[i], us, x[:M], g.k, out=outs[M])

    def step(timed):
        for M in Ms:
            if timed:
                timer(lambda: call(M))
                per_m[M].pairs.append(timer.pairs[-1])
            else:
                call(M)

    def cpu_baseline():
        def run(n):
            t0 = time.perf_counter()
            oracle.gateup_swiglu(g.codes, g.scales, u.codes, u.scales, w.x[0], 4, g.R, g.C, g.k, L, T,
                                 rows=np.arange(n))
            return time.perf_counter() - t0
        probe = 32
        dt = run(probe)
        n = int(min(g.R, max(probe, probe * args.cpu_seconds / max(dt, 1e-6))))
        dt = run(n)
        nbytes = 2 * n * g.codes.shape[1] * 4
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"gate+up rows 0..{n - 1} of {g.R} at M=4 (all four vectors per pass), "
                          f"{nbytes} code bytes in {dt:.2f} s"}

    def report(ms_step):
        launch_ms = timer.mean_ms()
        per_launch_bytes = code_bytes
        achieved = per_launch_bytes / (launch_ms * 1e-3) / 1e9
        detail = {f"M{M}": {"us_per_call": per_m[M].mean_ms() * 1e3,
                            "GBps": per_launch_bytes / (per_m[M].mean_ms() * 1e-3) / 1e9} for M in Ms}
        return {
            "value": 4 * code_bytes / (ms_step * 1e-3) / 1e9, "unit": "GB/s",
            "dtype": "f32",
            "config": {"workload": w.name, "M": list(Ms), "R": g.R, "C": g.C, "k": g.k, "L": L, "T": T,
                       "code_bytes_per_call": code_bytes, "replicas": nrep},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                         "kernel": "gateup (all M)", "mean_launch_us": launch_ms * 1e3},
            "detail": detail,
        }

    return step, cpu_baseline, report


def workload_prefill(args, np, torch, dev):
    import oracle
    import trellis_coded_quantized_amd as tq
    import trellis_inputs as ti

    M = args.m or 2048
    w = ti.prefill(Ms=(M,))
    m = w.mats[0]
    codes, half, bf16 = _dev_tensors(np, torch, dev)
    dc, ds, dx = codes(m.codes), half(m.scales), bf16(w.x[0])
    out = torch.empty((M, m.R), dtype=torch.bfloat16, device=dev)
    algo = tq.PREFILL_EXPAND_GEMM if args.algo == "expand_gemm" else tq.PREFILL_FUSED
    nbytes = tq.prefill_workspace_bytes(m.R, m.C, M, m.k, algo)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    timer = EventTimer(torch)
    flops = 2.0 * M * m.R * m.C

    def call():
        tq.prefill(dc, ds, dx, m.k, algo=algo, out=out, workspace=ws)

    def step(timed):
        if timed:
            timer(call)
        else:
            call()

    def cpu_baseline():
        ms = np.arange(M)
        def run(n):
            t0 = time.perf_counter()
            oracle.prefill_sums(m.codes, m.scales, w.x[0], M, m.R, m.C, m.k, L, T, ms, np.arange(n))
            return time.perf_counter() - t0
        dt = run(4)
        n = int(min(m.R, max(4, 4 * args.cpu_seconds / max(dt, 1e-6))))
        dt = run(n)
        f = 2.0 * M * n * m.C
        return {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{n} of {m.R} weight rows at M={M}: {f:.3e} flop in {dt:.2f} s"}

    def report(ms_step):
        launch_ms = timer.mean_ms()
        achieved = flops / (launch_ms * 1e-3) / 1e12
        return {
            "value": flops / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s", "dtype": "bf16",
            "config": {"workload": w.name, "M": M, "R": m.R, "C": m.C, "k": m.k, "L": L, "T": T,
                       "algo": args.algo},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None,
                         "kernel": f"prefill {args.algo}", "mean_launch_us": launch_ms * 1e3},
        }

    return step, cpu_baseline, report


def _matvec_workload(w, Ms, args, np, torch, dev, label):
    """Chain of matvec calls (axis 0 or 1) per step, codes rotated over
    >= 1 GiB of replicas; dominant kernel = the whole call."""
    import oracle
    import trellis_coded_quantized_amd as tq

    codes, half, bf16 = _dev_tensors(np, torch, dev)
    code_bytes = sum(m.codes.nbytes for m in w.mats)
    nrep = max(1, math.ceil(ROTATE_BYTES / code_bytes))
    reps = [[codes(m.codes) for m in w.mats]]
    for _ in range(nrep - 1):
        reps.append([c.clone() for c in reps[0]])
    scs = [half(m.scales) for m in w.mats]
    xs = [bf16(x) for x in w.x]
    outs = {}
    wss = []
    for i, m in enumerate(w.mats):
        n_out = m.R if m.axis == 1 else m.C
        for M in Ms:
            outs[(i, M)] = torch.empty((M, n_out), dtype=torch.bfloat16, device=dev)
        if m.axis == 0:
            nb = tq.load_library().trellis_matvec_axis0_workspace_bytes(m.R, m.C, max(Ms), m.k, L, T)
        else:
            nb = tq.load_library().trellis_matvec_axis1_workspace_bytes(m.R, m.C, max(Ms), m.k, L, T)
        wss.append(torch.empty(max(nb, 256), dtype=torch.uint8, device=dev))
    state = {"i": 0}
    timer = EventTimer(torch)

    def call(M):
        rep = reps[state["i"] % nrep]
        state["i"] += 1
        for i, m in enumerate(w.mats):
            fn = tq.matvec_axis1 if m.axis == 1 else tq.matvec_axis0
            fn(rep[i], scs[i], xs[i][:M], m.k, out=outs[(i, M)], workspace=wss[i])

    def step(timed):
        for M in Ms:
            if timed:
                timer(lambda: call(M))
            else:
                call(M)

    def cpu_baseline():
        m, x = w.mats[0], w.x[0]
        ref = oracle.matvec_axis1 if m.axis == 1 else oracle.matvec_axis0
        n_all = m.R if m.axis == 1 else m.C
        def run(n):
            t0 = time.perf_counter()
            sel = np.arange(n)
            if m.axis == 1:
                ref(m.codes, m.scales, x, max(Ms), m.R, m.C, m.k, L, T, rows=sel)
            else:
                ref(m.codes, m.scales, x, max(Ms), m.R, m.C, m.k, L, T, cols=sel)
            return time.perf_counter() - t0
        dt = run(16)
        n = int(min(n_all, max(16, 16 * args.cpu_seconds / max(dt, 1e-6))))
        dt = run(n)
        nbytes = m.codes.nbytes * n // n_all
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{n} of {n_all} outputs of the first matrix at M={max(Ms)}, {dt:.2f} s"}

    def report(ms_step):
        launch_ms = timer.mean_ms()
        achieved = code_bytes / (launch_ms * 1e-3) / 1e9
        return {
            "value": len(Ms) * code_bytes / (ms_step * 1e-3) / 1e9, "unit": "GB/s", "dtype": "f32",
            "config": {"workload": w.name, "M": list(Ms), "k": w.mats[0].k, "L": L, "T": T,
                       "matrices": [f"axis{m.axis} {m.R}x{m.C}" for m in w.mats],
                       "code_bytes_per_call": code_bytes, "replicas": nrep},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": label,
                         "mean_launch_us": launch_ms * 1e3},
        }

    return step, cpu_baseline, report


def workload_axis0(args, np, torch, dev):
    import trellis_inputs as ti
    Ms = (args.m,) if args.m else (1, 2, 3, 4)
    return _matvec_workload(ti.axis0(), Ms, args, np, torch, dev, "axis0 scatter + fold")


def workload_layer_chain(args, np, torch, dev):
    import trellis_inputs as ti
    return _matvec_workload(ti.layer_chain(), (4,), args, np, torch, dev, "4-matrix chain")


def workload_axis1_m1(args, np, torch, dev):
    import trellis_inputs as ti
    return _matvec_workload(ti.axis1_m1(), (1,), args, np, torch, dev, "axis1 reduce")


def workload_copy(args, np, torch, dev):
    """Plain device-to-device copy of 1 GiB: the HBM reference point, and the
    known-size kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    nbytes = ROTATE_BYTES
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    timer = EventTimer(torch)

    def step(timed):
        if timed:
            timer(lambda: dst.copy_(src))
        else:
            dst.copy_(src)

    def cpu_baseline():
        return None

    def report(ms_step):
        launch_ms = timer.mean_ms()
        achieved = 2 * nbytes / (launch_ms * 1e-3) / 1e9
        return {
            "value": 2 * nbytes / (ms_step * 1e-3) / 1e9, "unit": "GB/s", "dtype": "u8",
            "config": {"workload": "device copy", "bytes_read": nbytes, "bytes_written": nbytes},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "copy",
                         "mean_launch_us": launch_ms * 1e3},
        }

    return step, cpu_baseline, report


WORKLOADS = {"copy": workload_copy, "gateup": workload_gateup, "prefill": workload_prefill, "axis0": workload_axis0,
             "layer_chain": workload_layer_chain, "axis1_m1": workload_axis1_m1}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gateup", choices=sorted(WORKLOADS))
    ap.add_argument("--m", type=int, default=0, help="prefill rows (default 2048)")
    ap.add_argument("--algo", default="fused", choices=["fused", "expand_gemm"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested; this build measures one GPU only "
              f"(the path runs on a single MI355X, see the sharding notes in the design).", file=sys.stderr)
        sys.exit(2)

    _ensure_built()
    import numpy as np
    import torch

    dev = "cuda:0"
    torch.cuda.set_device(0)
    step, cpu_baseline, report = WORKLOADS[args.workload](args, np, torch, dev)
    print(f"[bench] {args.workload}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    res = report(ms_step)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
    line = {
        "metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": res["dtype"],
        "data": "synthetic: seeded uniform uint32 codes, fp16 scales U[0.005, 0.02], bf16 x ~ N(0, 1)",
        "config": res["config"], "roofline": res["roofline"], "cpu_baseline": cpu,
    }
    if "detail" in res:
        line["detail"] = res["detail"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
