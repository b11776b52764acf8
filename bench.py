#!/usr/bin/env python3
"""Benchmark of the packed trellis-coded linear layer on one MI355X.

Default workload: fused gate/up + SwiGLU matvec, two 17408 x 5120 matrices,
k = 2, L = 12, T = 256; one step = one call at each M in 1, 2, 3, 4.  The
value is packed-code bytes per second over the whole step (inputs resident
in HBM; code buffers rotate over >= 1 GiB of replicas so the 256 MB
Infinity Cache cannot serve repeats).  Other workloads (--workload) print
the same JSON line for their own metric: the 512 x 2048 reduce matvec, the
17408 x 5120 k = 3 down-projection scatter (row-major or interleaved), the
k = 4 decoder-layer chain, the MLP (gate/up + SwiGLU, then the down
projection, in one call), the axis-1 and axis-0 prefills (fused or
expansion + GEMM), the two measurement probes (decode_free, decode_only)
and a plain device copy used as the HBM reference point.

Steps run as HIP graphs (one graph per replica offset, captured after an
eager warm-up) so the Python call overhead of the binding stays out of the
measurement, as it would in a serving loop; --eager times the plain calls.
Expansion + GEMM runs eagerly, after one trellis_prefill_tune call in
set-up picks the GEMM.

The JSON line carries:
  roofline      the dominant kernel's algorithmic bytes (or flops) per launch
                over its mean launch time (HIP events on the launch stream,
                every step of the timed region), against the MI355X peak of
                its bound (matvecs: HBM 8 TB/s; prefill: bf16 MFMA 2.5
                PFLOP/s).  Matvecs add two ALU ceilings of their decode: the
                VALU slot model (alu_model_*) and the rate of the
                register-only decode probe measured in the same run
                (alu_*).  traffic = HBM bytes per launch from the committed
                rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/, or
                null when the kernel sources changed since those counters
                were taken;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same
                workload on this host (a baseline, not a target), with the
                host's CPU model.
The default (gate/up) line adds bound_location (the decode-free kernel and
the decode-only probe on the same weights) and prefill, the metric's second
half: 17408 x 5120, k = 2, M = 2048, fused and expansion + GEMM, each with
its own MFMA roofline, and the oracle's CPU baseline for it.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode matvec GB/s of packed codes (% HBM peak) at M=1..4; prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# VALU issue slots of the chip: 256 CUs x 4 SIMDs x 16 lanes at 2.4 GHz.  The
# decode of one weight takes 4.5 of them on gfx950 (window extract 1, the 1MAD
# multiply-add v_mad_u64_u32 2 (half rate), the byte sums of a weight pair to
# f16 integer codes 3 per pair); the products with x run on MFMA.  This slot
# model is one ALU ceiling; the other is the rate the register-only decode
# probe measures on the box in the same run (trellis_probe_decode_only).
VALU_LANE_SLOTS_PER_S = 256 * 4 * 16 * 2.4e9
DECODE_SLOTS_PER_WEIGHT = 4.5


def decode_alu_model_gbs(code_bytes_per_weight):
    """Packed-code GB/s at which the decode alone fills every VALU issue slot."""
    return VALU_LANE_SLOTS_PER_S / DECODE_SLOTS_PER_WEIGHT * code_bytes_per_weight / 1e9
L, T = 12, 256
ROTATE_BYTES = 1 << 30
CSRC = os.path.join(ROOT, "trellis_coded_quantized_amd", "csrc")
DATA = "synthetic: seeded uniform uint32 codes, fp16 scales U[0.005, 0.02], bf16 x ~ N(0, 1)"


def _ensure_built():
    from trellis_coded_quantized_amd import LIB_PATH
    if not os.path.exists(LIB_PATH) or not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        import __graft_entry__
        __graft_entry__.build()


def sources_sha256(files):
    """Digest of the kernel sources a counter summary was taken with."""
    h = hashlib.sha256()
    for f in sorted(files):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def committed_traffic(profile, files):
    """HBM bytes per launch from profiles/<profile>, if its source digest
    matches the sources built now; None otherwise."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    tb = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not sha or not tb or sha.group(1) != sources_sha256(files):
        return None
    return float(tb.group(1))


def _dev_tensors(np, torch, dev):
    def codes(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev)

    def half(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.float16)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    return codes, half, bf16


class Workload:
    """One benchmark workload.  step(s) enqueues step s (replicas chosen by s)
    on the current stream; `period` distinct steps repeat."""
    name = ""
    unit = "GB/s"
    bound = "hbm"
    dtype = "f32"
    graph = True
    period = 1
    kernels_per_step = 1
    units_per_step = 0.0          # algorithmic bytes (GB/s) or flops (TFLOP/s)
    kernel = ""
    profile = None                # profiles/ summary holding the traffic counters
    profile_sources = ()
    config = {}

    def step(self, s):
        raise NotImplementedError

    def cpu_baseline(self, seconds):
        return None


def _nrep(bytes_per_copy):
    return max(1, math.ceil(ROTATE_BYTES / bytes_per_copy))


AXIS1_SOURCES = ("axis1.hip", "axis1_kernel.hpp", "copy_ring.hpp", "mfma_common.hpp", "trellis_device.hpp")
AXIS0_SOURCES = ("axis0.hip", "axis0_kernel.hpp", "copy_ring.hpp", "mfma_common.hpp", "trellis_device.hpp")
PREFILL_SOURCES = ("prefill.hip", "mfma_common.hpp", "trellis_device.hpp")


class GateUp(Workload):
    bound = "hbm"

    def __init__(self, args, np, torch, dev):
        import trellis_coded_quantized_amd as tq
        import trellis_inputs as ti
        self.np, self.tq = np, tq
        self.w = w = ti.gateup()
        self.g, self.u = g, u = w.mats
        codes, half, bf16 = _dev_tensors(np, torch, dev)
        self.code_bytes = g.codes.nbytes + u.codes.nbytes
        self.bytes_per_weight = g.k / 8
        self.nrep = _nrep(self.code_bytes)
        self.gcs = [codes(g.codes)]
        self.ucs = [codes(u.codes)]
        for _ in range(self.nrep - 1):
            self.gcs.append(self.gcs[0].clone())
            self.ucs.append(self.ucs[0].clone())
        self.gs, self.us, self.x = half(g.scales), half(u.scales), bf16(w.x[0])
        self.Ms = (1, 2, 3, 4)
        self.outs = {M: torch.empty((M, g.R), dtype=torch.bfloat16, device=dev) for M in self.Ms}
        self.period = self.nrep // math.gcd(self.nrep, len(self.Ms))
        self.kernels_per_step = len(self.Ms)
        self.units_per_step = len(self.Ms) * self.code_bytes
        self.name = w.name
        self.kernel = "axis1_kernel (gate/up + SwiGLU), one launch per M"
        self.profile = "axis1_gateup_17408x5120_k2.md"
        self.profile_sources = AXIS1_SOURCES
        self.config = {"workload": w.name, "M": list(self.Ms), "R": g.R, "C": g.C, "k": g.k, "L": L, "T": T,
                       "code_bytes_per_call": self.code_bytes, "replicas": self.nrep}

    def step(self, s):
        for j, M in enumerate(self.Ms):
            i = (s * len(self.Ms) + j) % self.nrep
            self.tq.gateup_swiglu(self.gcs[i], self.gs, self.ucs[i], self.us, self.x[:M], self.g.k,
                                  out=self.outs[M])

    def cpu_baseline(self, seconds):
        import oracle
        g, u, w, np = self.g, self.u, self.w, self.np
        t0 = time.perf_counter()
        nbytes, passes = 0, 0
        while True:                            # whole steps (M = 1, 2, 3, 4 over every row)
            for M in self.Ms:
                oracle.gateup_swiglu(g.codes, g.scales, u.codes, u.scales, w.x[0], M, g.R, g.C, g.k, L, T)
                nbytes += self.code_bytes
            passes += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{passes} whole steps (gate+up, all {g.R} rows, M = 1..4), {nbytes} code bytes "
                          f"in {dt:.2f} s"}


class Matvec(Workload):
    """Calls of the axis-1 / axis-0 matvec entry points, one per matrix, per M."""

    bound = "hbm"

    def __init__(self, w, Ms, label, profile, sources, args, np, torch, dev):
        import trellis_coded_quantized_amd as tq
        self.np, self.tq, self.w, self.Ms = np, tq, w, Ms
        self.bytes_per_weight = sum(m.codes.nbytes for m in w.mats) / sum(m.R * m.C for m in w.mats)
        codes, half, bf16 = _dev_tensors(np, torch, dev)
        self.code_bytes = sum(m.codes.nbytes for m in w.mats)
        self.nrep = _nrep(self.code_bytes)
        self.reps = [[codes(self._stored(m)) for m in w.mats]]
        for _ in range(self.nrep - 1):
            self.reps.append([c.clone() for c in self.reps[0]])
        self.scs = [half(m.scales) for m in w.mats]
        self.xs = [bf16(x) for x in w.x]
        self.outs, self.wss = {}, []
        lib = tq.load_library()
        for i, m in enumerate(w.mats):
            n_out = m.R if m.axis == 1 else m.C
            for M in Ms:
                self.outs[(i, M)] = torch.empty((M, n_out), dtype=torch.bfloat16, device=dev)
            fn = lib.trellis_matvec_axis0_workspace_bytes if m.axis == 0 else lib.trellis_matvec_axis1_workspace_bytes
            nb = fn(m.R, m.C, max(Ms), m.k, L, T)
            self.wss.append(torch.empty(max(nb, 256), dtype=torch.uint8, device=dev))
        self.period = self.nrep // math.gcd(self.nrep, len(Ms))
        self.kernels_per_step = len(Ms) * len(w.mats)
        self.units_per_step = len(Ms) * self.code_bytes
        self.name, self.kernel = w.name, label
        self.profile, self.profile_sources = profile, sources
        self.config = {"workload": w.name, "M": list(Ms), "k": w.mats[0].k, "L": L, "T": T,
                       "matrices": [f"axis{m.axis} {m.R}x{m.C}" for m in w.mats],
                       "code_bytes_per_call": self.code_bytes, "replicas": self.nrep}

    interleaved = False

    def _stored(self, m):
        """codes as stored: row-major, or the block-interleaved k = 3 axis-0 layout"""
        if not self.interleaved:
            return m.codes
        wpb = 256 * m.k // 32
        return self.np.ascontiguousarray(m.codes.reshape(m.R, m.C // 512, 2 * wpb).transpose(1, 0, 2))

    def step(self, s):
        for j, M in enumerate(self.Ms):
            rep = self.reps[(s * len(self.Ms) + j) % self.nrep]
            for i, m in enumerate(self.w.mats):
                fn = self.tq.matvec_axis1 if m.axis == 1 else self.tq.matvec_axis0
                fn(rep[i], self.scs[i], self.xs[i][:M], m.k, out=self.outs[(i, M)], workspace=self.wss[i])

    def cpu_baseline(self, seconds):
        import oracle
        np = self.np
        t0 = time.perf_counter()
        nbytes, passes = 0, 0
        while True:                            # whole steps: every matrix, every M
            for M in self.Ms:
                for m, x in zip(self.w.mats, self.w.x):
                    ref = oracle.matvec_axis1 if m.axis == 1 else oracle.matvec_axis0
                    ref(m.codes, m.scales, x, M, m.R, m.C, m.k, L, T)
                    nbytes += m.codes.nbytes
            passes += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{passes} whole steps ({len(self.w.mats)} matrices x M in {list(self.Ms)}), "
                          f"{nbytes} code bytes in {dt:.2f} s"}


class Mlp(Workload):
    """The decoder-layer MLP for M = 1..4: gate/up + SwiGLU (17408 x 5120, k = 2), then the
    down projection stored transposed (17408 x 5120, k = 3), one trellis_mlp_decode call each."""
    bound = "hbm"

    def __init__(self, args, np, torch, dev):
        import trellis_coded_quantized_amd as tq
        import trellis_inputs as ti
        self.np, self.tq = np, tq
        w = ti.gateup()
        self.g, self.u = g, u = w.mats
        self.d = d = ti.axis0().mats[0]
        self.x = w.x[0]
        codes, half, bf16 = _dev_tensors(np, torch, dev)
        self.code_bytes = g.codes.nbytes + u.codes.nbytes + d.codes.nbytes
        weights = 2 * g.R * g.C + d.R * d.C
        self.bytes_per_weight = self.code_bytes / weights
        self.nrep = _nrep(self.code_bytes)
        self.reps = [[codes(g.codes), codes(u.codes), codes(d.codes)]]
        for _ in range(self.nrep - 1):
            self.reps.append([c.clone() for c in self.reps[0]])
        self.gs, self.us, self.ds = half(g.scales), half(u.scales), half(d.scales)
        self.dx = bf16(self.x)
        self.Ms = (1, 2, 3, 4)
        lib = tq.load_library()
        self.outs = {M: torch.empty((M, d.C), dtype=torch.bfloat16, device=dev) for M in self.Ms}
        self.wss = {M: torch.zeros(lib.trellis_mlp_decode_workspace_bytes(g.R, g.C, d.C, M, g.k, d.k, L, T),
                                   dtype=torch.uint8, device=dev) for M in self.Ms}
        self.period = self.nrep // math.gcd(self.nrep, len(self.Ms))
        self.kernels_per_step = len(self.Ms)
        self.units_per_step = len(self.Ms) * self.code_bytes
        self.name = "mlp_17408x5120_k2_k3"
        self.kernel = "trellis_mlp_decode (gate/up + SwiGLU, axis-0 down + fold), one call per M"
        self.config = {"workload": self.name, "M": list(self.Ms), "R": g.R, "C": g.C, "C_out": d.C,
                       "k_gate_up": g.k, "k_down": d.k, "L": L, "T": T, "code_bytes_per_call": self.code_bytes,
                       "replicas": self.nrep}

    def step(self, s):
        for j, M in enumerate(self.Ms):
            gc, uc, dc = self.reps[(s * len(self.Ms) + j) % self.nrep]
            self.tq.mlp_decode(gc, self.gs, uc, self.us, dc, self.ds, self.dx[:M], self.g.k, self.d.k,
                               out=self.outs[M], workspace=self.wss[M])

    def cpu_baseline(self, seconds):
        import oracle
        g, u, d, np = self.g, self.u, self.d, self.np
        t0 = time.perf_counter()
        nbytes, passes = 0, 0
        while True:
            for M in self.Ms:
                _, _, hidden = oracle.gateup_swiglu(g.codes, g.scales, u.codes, u.scales, self.x, M, g.R, g.C, g.k,
                                                    L, T)
                oracle.matvec_axis0(d.codes, d.scales, hidden, M, d.R, d.C, d.k, L, T)
                nbytes += self.code_bytes
            passes += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{passes} whole steps (gate/up then down, M = 1..4), {nbytes} code bytes in {dt:.2f} s"}


def _prefill_algo(tq, name):
    return {"fused": tq.PREFILL_FUSED, "expand_gemm": tq.PREFILL_EXPAND_GEMM, "auto": tq.PREFILL_AUTO}[name]


def _runs_fused(tq, algo, workspace_bytes):
    """Whether a prefill call with `algo` runs the fused kernels: AUTO is resolved by the
    library, and its workspace query answers for the algorithm it picks."""
    if algo != tq.PREFILL_AUTO:
        return algo == tq.PREFILL_FUSED
    return workspace_bytes(algo) == workspace_bytes(tq.PREFILL_FUSED)


class Prefill(Workload):
    unit, bound, dtype = "TFLOP/s", "mfma", "bf16"

    def __init__(self, args, np, torch, dev):
        import trellis_coded_quantized_amd as tq
        import trellis_inputs as ti
        self.np, self.tq = np, tq
        M = args.m or 2048
        self.M = M
        self.w = w = ti.prefill(Ms=(M,))
        self.m = m = w.mats[0]
        codes, half, bf16 = _dev_tensors(np, torch, dev)
        self.dc, self.ds, self.dx = codes(m.codes), half(m.scales), bf16(w.x[0])
        self.out = torch.empty((M, m.R), dtype=torch.bfloat16, device=dev)
        self.algo = _prefill_algo(tq, args.algo)
        wsb = lambda a: tq.prefill_workspace_bytes(m.R, m.C, M, m.k, a)
        nbytes = wsb(self.algo)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        self.graph = _runs_fused(tq, self.algo, wsb)
        if not self.graph:                     # pick the fastest hipBLASLt candidate once, in set-up
            tq.prefill(self.dc, self.ds, self.dx, m.k, out=self.out, workspace=self.ws, tune=True)
        self.kernels_per_step = 1 if self.graph else 2
        self.units_per_step = 2.0 * M * m.R * m.C
        self.name = w.name
        self.kernel = ("prefill_xlayout_kernel + prefill_fused_kernel (+ prefill_fold_kernel for split tiles), one step" if self.graph
                       else "expand_kernel + hipBLASLt GEMM (per call)")
        self.profile = "prefill_17408x5120_k2_m2048.md" if (self.graph and M == 2048) else None
        self.profile_sources = PREFILL_SOURCES
        self.config = {"workload": w.name, "M": M, "R": m.R, "C": m.C, "k": m.k, "L": L, "T": T,
                       "algo": args.algo}
        if args.algo == "auto":
            self.config["auto_picked"] = "fused" if self.graph else "expand_gemm"

    def step(self, s):
        self.tq.prefill(self.dc, self.ds, self.dx, self.m.k, algo=self.algo, out=self.out, workspace=self.ws)

    def cpu_baseline(self, seconds):
        import oracle
        np, m, M, w = self.np, self.m, self.M, self.w
        ms = np.arange(M)

        def run(n):
            t0 = time.perf_counter()
            oracle.prefill_sums(m.codes, m.scales, w.x[0], M, m.R, m.C, m.k, L, T, ms, np.arange(n))
            return time.perf_counter() - t0
        dt = run(4)
        n = int(min(m.R, max(4, 4 * seconds / max(dt, 1e-6))))
        dt = run(n)
        f = 2.0 * M * n * m.C
        return {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{n} of {m.R} weight rows at M={M}: {f:.3e} flop in {dt:.2f} s"}


class PrefillAxis0(Workload):
    """Axis-0 prefill: the MLP down projection for M rows, stored W^T 17408 x 5120, k = 3,
    x [M, 17408]; the fused decode-to-LDS MFMA kernel (one graph-replayed step), or expansion
    into the workspace followed by one bf16 GEMM (per call, eager)."""
    unit, bound, dtype = "TFLOP/s", "mfma", "bf16"

    def __init__(self, args, np, torch, dev):
        import trellis_coded_quantized_amd as tq
        import trellis_inputs as ti
        self.np, self.tq = np, tq
        M = args.m or 2048
        self.M = M
        self.m = m = ti.axis0().mats[0]
        self.x = ti.activations(np.random.default_rng(2000 + M), M, m.R)
        codes, half, bf16 = _dev_tensors(np, torch, dev)
        self.dc, self.ds, self.dx = codes(m.codes), half(m.scales), bf16(self.x)
        self.out = torch.empty((M, m.C), dtype=torch.bfloat16, device=dev)
        self.algo = _prefill_algo(tq, args.algo)
        wsb = lambda a: tq.load_library().trellis_prefill_axis0_workspace_bytes(m.R, m.C, M, m.k, L, T, a)
        nbytes = wsb(self.algo)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        self.graph = _runs_fused(tq, self.algo, wsb)
        if not self.graph:                     # pick the fastest hipBLASLt candidate once, in set-up
            tq.prefill_axis0(self.dc, self.ds, self.dx, m.k, out=self.out, workspace=self.ws, tune=True)
        self.kernels_per_step = 1 if self.graph else 2
        self.units_per_step = 2.0 * M * m.R * m.C
        self.name = f"prefill_axis0_{m.R}x{m.C}_k{m.k}_m{M}"
        self.kernel = ("prefill_xlayout_kernel + prefill_fused_kernel (+ prefill_fold_kernel for split tiles), one step"
                       if self.graph else "expand_kernel + hipBLASLt GEMM (per call)")
        self.profile = "prefill_axis0_fused_17408x5120_k3_m2048.md" if (self.graph and M == 2048) else None
        self.profile_sources = PREFILL_SOURCES
        self.config = {"workload": self.name, "M": M, "R_in": m.R, "C_out": m.C, "k": m.k, "L": L, "T": T,
                       "algo": args.algo}
        if args.algo == "auto":
            self.config["auto_picked"] = "fused" if self.graph else "expand_gemm"

    def step(self, s):
        self.tq.prefill_axis0(self.dc, self.ds, self.dx, self.m.k, algo=self.algo, out=self.out, workspace=self.ws)

    def cpu_baseline(self, seconds):
        import oracle
        np, m, M = self.np, self.m, self.M

        def run(n):
            t0 = time.perf_counter()
            oracle.prefill_axis0_sums(m.codes, m.scales, self.x, M, m.R, m.C, m.k, L, T, np.arange(M), np.arange(n))
            return time.perf_counter() - t0
        dt = run(4)
        n = int(min(m.C, max(4, 4 * seconds / max(dt, 1e-6))))
        dt = run(n)
        f = 2.0 * M * n * m.R
        return {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{n} of {m.C} output columns at M={M}: {f:.3e} flop in {dt:.2f} s"}


class DecodeFree(GateUp):
    """The gate/up workload through the decode-free kernel (the pages' variant 4
    timing floor): the same copies, MFMAs, prologue and epilogue, no decode."""

    def __init__(self, args, np, torch, dev):
        super().__init__(args, np, torch, dev)
        self.name = self.config["workload"] = "decode_free_gateup_17408x5120_k2"
        self.kernel = "axis1_kernel without the decode (gate/up), one launch per M"
        self.profile = None

    def step(self, s):
        for j, M in enumerate(self.Ms):
            i = (s * len(self.Ms) + j) % self.nrep
            self.tq.probe_gateup_decode_free(self.gcs[i], self.gs, self.ucs[i], self.us, self.x[:M], self.g.k,
                                             out=self.outs[M])

    def cpu_baseline(self, seconds):
        return None


class DecodeOnly(Workload):
    """The register-only decode probe: the matvec loop's decode and MFMAs with no
    memory traffic, one workgroup of 8 waves per compute unit.  Its rate is the
    ALU ceiling of the matvec kernels, reported as packed-code GB/s at k = 2."""
    unit, bound, dtype = "GB/s", "alu", "u32"
    ITERS = 4096

    def __init__(self, args, np, torch, dev):
        import trellis_coded_quantized_amd as tq
        self.np, self.tq, self.k = np, tq, 2
        self.blocks = torch.cuda.get_device_properties(dev).multi_processor_count
        rng = np.random.default_rng(77)
        n = self.blocks * tq.PROBE_THREADS
        self.runs = torch.from_numpy(rng.integers(0, 2 ** 32, (n, self.k + 1), dtype=np.uint32).view(np.int32)).to(dev)
        self.weights_per_step = float(n) * self.ITERS * 32
        self.units_per_step = self.weights_per_step * self.k / 8      # packed-code bytes at k = 2
        self.name = "decode_only_probe"
        self.kernel = "decode_only_kernel (register-only decode + MFMA)"
        self.config = {"workload": self.name, "blocks": self.blocks, "threads_per_block": tq.PROBE_THREADS,
                       "iters": self.ITERS, "k": self.k, "weights_per_launch": self.weights_per_step}

    def step(self, s):
        self.tq.probe_decode_only(self.runs, self.k, self.ITERS)


class Copy(Workload):
    """Plain device-to-device copy of 1 GiB: the HBM reference point, and the
    known-size kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    dtype = "u8"
    bound = "hbm"
    graph = False

    def __init__(self, args, np, torch, dev):
        self.src = torch.empty(ROTATE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        self.dst = torch.empty_like(self.src)
        self.units_per_step = 2.0 * ROTATE_BYTES
        self.name = "device copy"
        self.kernel = "copy"
        self.config = {"workload": "device copy", "bytes_read": ROTATE_BYTES, "bytes_written": ROTATE_BYTES}

    def step(self, s):
        self.dst.copy_(self.src)


def workload_axis0(args, np, torch, dev):
    import trellis_inputs as ti
    Ms = (args.m,) if args.m else (1, 2, 3, 4)
    return Matvec(ti.axis0(), Ms, "axis0 scatter + fold", "axis0_scatter_17408x5120_k3.md", AXIS0_SOURCES,
                  args, np, torch, dev)


class MatvecInterleaved(Matvec):
    interleaved = True


def workload_axis0_il(args, np, torch, dev):
    import trellis_inputs as ti
    Ms = (args.m,) if args.m else (1, 2, 3, 4)
    wl = MatvecInterleaved(ti.axis0(), Ms, "axis0 scatter + fold, block-interleaved codes [C/512, R, 48]", None,
                           AXIS0_SOURCES, args, np, torch, dev)
    wl.name = wl.config["workload"] = "axis0_interleaved_17408x5120_k3"
    return wl


class LayerChainGrouped(Matvec):
    """The decoder-layer set with its three axis-1 projections in one grouped
    launch over one x (as q / k / v read the same hidden state), then the
    axis-0 call: 2 calls, 3 kernels per step."""

    def __init__(self, *a):
        super().__init__(*a)
        self.kernels_per_step = 2 * len(self.Ms)

    def step(self, s):
        for j, M in enumerate(self.Ms):
            rep = self.reps[(s * len(self.Ms) + j) % self.nrep]
            a1 = [i for i, m in enumerate(self.w.mats) if m.axis == 1]
            self.tq.matvec_axis1_group([rep[i] for i in a1], [self.scs[i] for i in a1], self.xs[a1[0]][:M],
                                       self.w.mats[a1[0]].k, outs=[self.outs[(i, M)] for i in a1])
            for i, m in enumerate(self.w.mats):
                if m.axis == 0:
                    self.tq.matvec_axis0(rep[i], self.scs[i], self.xs[i][:M], m.k, out=self.outs[(i, M)],
                                         workspace=self.wss[i])


def workload_layer_chain(args, np, torch, dev):
    import trellis_inputs as ti
    return Matvec(ti.layer_chain(), (4,), "4-launch chain (3 x axis1_kernel, axis0 scatter + fold)", None,
                  AXIS1_SOURCES, args, np, torch, dev)


def workload_layer_chain_grouped(args, np, torch, dev):
    import trellis_inputs as ti
    wl = LayerChainGrouped(ti.layer_chain(), (4,), "grouped axis1_kernel (3 projections, one launch), then axis0 "
                           "scatter + fold", None, AXIS1_SOURCES, args, np, torch, dev)
    wl.name = wl.config["workload"] = "layer_chain_k4_m4_grouped"
    wl.config["axis1"] = "one grouped launch over a shared x"
    return wl


def workload_axis1_m1(args, np, torch, dev):
    import trellis_inputs as ti
    return Matvec(ti.axis1_m1(), (1,), "axis1_kernel (reduce)", None, AXIS1_SOURCES, args, np, torch, dev)


WORKLOADS = {"copy": Copy, "gateup": GateUp, "prefill": Prefill, "axis0": workload_axis0, "mlp": Mlp,
             "prefill_axis0": PrefillAxis0, "axis0_il": workload_axis0_il,
             "layer_chain": workload_layer_chain, "layer_chain_grouped": workload_layer_chain_grouped,
             "axis1_m1": workload_axis1_m1, "decode_free": DecodeFree, "decode_only": DecodeOnly}


MATVEC_WORKLOADS = ("gateup", "axis0", "axis0_il", "layer_chain", "layer_chain_grouped", "mlp", "axis1_m1",
                    "decode_free")


def steps_per_graph(steps, cap=5):
    """Steps captured in one graph: the largest divisor of `steps` up to cap,
    so that exactly `steps` steps are timed."""
    return max(d for d in range(1, min(cap, max(steps, 1)) + 1) if steps % d == 0)


def time_workload(wl, steps, warmup, eager, torch, label):
    """Warm up, capture graphs of G consecutive steps (G divides `steps`;
    the graphs cycle through every replica offset) unless eager or the
    workload cannot be captured, then time exactly `steps` steps between
    device synchronisations.  Several steps per graph keep the per-replay
    launch cost (and torch's per-replay fill kernel) off each step, as a
    model's layer graph would.  Returns (ms per step, mean launch ms from HIP
    events on the launch stream, mode)."""
    print(f"[bench] {label}: warmup {warmup}", file=sys.stderr, flush=True)
    for s in range(warmup):
        wl.step(s)
    torch.cuda.synchronize()
    graphs = None
    G = steps_per_graph(steps)
    if wl.graph and not eager:
        graphs = []
        for r in range(wl.period):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in range(G):
                    wl.step(r * G + s)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
    mode = f"graph ({G} steps per replay)" if graphs else "eager"
    print(f"[bench] {label}: timing {steps} steps ({mode})", file=sys.stderr, flush=True)
    nrec = steps // G if graphs else steps
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nrec)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(nrec):
        a, b = events[i]
        a.record()
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            wl.step(i)
        b.record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / max(steps, 1)
    step_ms = sum(a.elapsed_time(b) for a, b in events) / max(steps, 1)
    return ms_step, step_ms / wl.kernels_per_step, mode


def roofline_of(wl, launch_ms, probe_weights_per_s=None):
    """The dominant kernel's achieved rate against the MI355X peak of its bound;
    matvecs also against the two ALU ceilings of their decode."""
    scale = 1e9 if wl.unit == "GB/s" else 1e12
    achieved = wl.units_per_step / wl.kernels_per_step / (launch_ms * 1e-3) / scale
    peak = {"hbm": HBM_PEAK_GBS, "mfma": BF16_PEAK_TFLOPS}.get(wl.bound)
    traffic = committed_traffic(wl.profile, wl.profile_sources) if wl.profile else None
    r = {"bound": wl.bound, "achieved": achieved, "peak": peak, "unit": wl.unit,
         "frac": achieved / peak if peak else None, "traffic": traffic, "kernel": wl.kernel,
         "mean_launch_us": launch_ms * 1e3}
    bpw = getattr(wl, "bytes_per_weight", None)
    if bpw:
        model = decode_alu_model_gbs(bpw)
        r.update({"alu_model_peak": model, "alu_model_frac": achieved / model,
                  "alu_model_basis": f"{VALU_LANE_SLOTS_PER_S:.4g} VALU lane-slots/s / {DECODE_SLOTS_PER_WEIGHT} "
                                     f"slots per weight x {bpw:.4g} code bytes per weight"})
        if probe_weights_per_s:
            probe = probe_weights_per_s * bpw / 1e9
            r.update({"alu_peak": probe, "alu_frac": achieved / probe,
                      "alu_basis": "decode_only_kernel rate measured in this run x code bytes per weight"})
    return r


def cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cpus": os.cpu_count()}


def probe_rate(np, torch, dev, args):
    """Decoded weights per second of the register-only decode probe."""
    wl = DecodeOnly(args, np, torch, dev)
    _, launch_ms, _ = time_workload(wl, 10, 2, True, torch, "decode_only probe")
    return wl.weights_per_step / (launch_ms * 1e-3), wl


def prefill_leg(np, torch, dev, args, cpu_seconds):
    """The prefill half of the metric: 17408 x 5120, k = 2, M = 2048, fused and
    expansion + tuned GEMM, each against the bf16 MFMA peak."""
    legs = {}
    cpu = None
    for algo in ("fused", "expand_gemm"):
        a = argparse.Namespace(m=2048, algo=algo)
        wl = Prefill(a, np, torch, dev)
        ms_step, launch_ms, mode = time_workload(wl, 20, 3, False, torch, f"prefill {algo}")
        legs[algo] = {"value": wl.units_per_step / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s",
                      "ms_per_call": ms_step, "mode": mode, "roofline": roofline_of(wl, launch_ms)}
        if cpu is None and cpu_seconds > 0:
            print("[bench] prefill cpu baseline (oracle)", file=sys.stderr, flush=True)
            cpu = wl.cpu_baseline(cpu_seconds)
            cpu.update(cpu_info())
        del wl
        torch.cuda.empty_cache()
    return {"workload": "prefill_17408x5120_k2_m2048", "M": 2048, "R": 17408, "C": 5120, "k": 2,
            "flop_per_call": 2.0 * 2048 * 17408 * 5120, **legs, "cpu_baseline": cpu}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gateup", choices=sorted(WORKLOADS))
    ap.add_argument("--m", type=int, default=0, help="prefill rows (default 2048) / axis0 M")
    ap.add_argument("--algo", default="fused", choices=["fused", "expand_gemm", "auto"])
    ap.add_argument("--eager", action="store_true", help="time plain calls instead of graph replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="gateup only: skip the prefill leg and the bound-location probes")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested; only one GPU is measured: the library runs on a "
              f"single MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    _ensure_built()
    import numpy as np
    import torch

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = WORKLOADS[args.workload](args, np, torch, dev)
    ms_step, launch_ms, mode = time_workload(wl, args.steps, args.warmup, args.eager, torch, args.workload)
    rate = None
    if args.workload in MATVEC_WORKLOADS:
        rate, _ = probe_rate(np, torch, dev, args)
    roof = roofline_of(wl, launch_ms, rate)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = wl.cpu_baseline(args.cpu_seconds)
        if cpu is not None:
            cpu.update(cpu_info())
    scale = 1e9 if wl.unit == "GB/s" else 1e12
    line = {
        "metric": METRIC, "value": wl.units_per_step / (ms_step * 1e-3) / scale, "unit": wl.unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": DATA, "config": dict(wl.config, mode=mode), "roofline": roof, "cpu_baseline": cpu,
    }
    if args.workload == "gateup" and not args.no_extras:
        df = DecodeFree.__new__(DecodeFree)          # the same buffers through the decode-free kernel
        df.__dict__.update(wl.__dict__)
        df.name = "decode_free_gateup_17408x5120_k2"
        df.kernel = "axis1_kernel without the decode (gate/up)"
        _, df_launch, _ = time_workload(df, args.steps, args.warmup, args.eager, torch, "decode_free")
        line["bound_location"] = {
            "kernel_launch_us": launch_ms * 1e3,
            "decode_free_launch_us": df_launch * 1e3,
            "decode_free_gbs": wl.code_bytes / (df_launch * 1e-3) / 1e9,
            "decode_only_weights_per_s": rate,
            "decode_only_launch_us_same_weights": 2 * 17408 * 5120 / rate * 1e6,
            "note": "decode-free = the kernel's copies, MFMAs, prologue and epilogue; decode-only = its decode "
                    "alone on the same weight count (register-only probe)",
        }
        line["prefill"] = prefill_leg(np, torch, dev, args, 0.0 if args.no_cpu_baseline else 10.0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
