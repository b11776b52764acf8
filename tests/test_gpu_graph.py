"""HIP graph replay of the matvec entry points (the form bench.py times).

A graph captured around a C-ABI call must reproduce the eager result on
every replay, with eager work and synchronisations between the replays
(nothing in the captured launches may depend on state that only the first
replay sets up).  The kernels are deterministic, so replays are compared bit
for bit with the eager output of the same call.
"""
import numpy as np
import pytest
import torch

import trellis_coded_quantized_amd as tq
import trellis_inputs as ti

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


def _d(a, dtype):
    view = {torch.int32: np.int32, torch.float16: np.int16, torch.bfloat16: np.int16}[dtype]
    t = torch.from_numpy(np.ascontiguousarray(a).view(view)).to(DEV)
    return t.view(dtype)


def _check_replays(call, out, disturb):
    call()
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(REPLAYS):
        out.zero_()
        disturb()                              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bits = torch.int32 if out.dtype == torch.float32 else torch.int16
        assert torch.equal(out.view(bits), want.view(bits)), f"replay {rep} differs from the eager result"


@pytest.mark.parametrize("M", [1, 4])
def test_graph_gateup(M):
    rng = np.random.default_rng(71)
    R, C, k = 1000, 2560, 2
    gc, gs = ti.codes(rng, R, C, k), ti.scales(rng, R)
    uc, us = ti.codes(rng, R, C, k), ti.scales(rng, R)
    x = ti.activations(rng, M, C)
    dgc, dgs, duc, dus = _d(gc, torch.int32), _d(gs, torch.float16), _d(uc, torch.int32), _d(us, torch.float16)
    dx = _d(x, torch.bfloat16)
    out = torch.empty((M, R), dtype=torch.bfloat16, device=DEV)
    other = torch.empty((M, R), dtype=torch.bfloat16, device=DEV)
    _check_replays(lambda: tq.gateup_swiglu(dgc, dgs, duc, dus, dx, k, out=out), out,
                   lambda: tq.gateup_swiglu(duc, dus, dgc, dgs, dx, k, out=other))


@pytest.mark.parametrize("k", [2, 4])
def test_graph_axis1(k):
    rng = np.random.default_rng(72)
    R, C, M = 777, 5120, 3
    c, s = ti.codes(rng, R, C, k), ti.scales(rng, R)
    x = ti.activations(rng, M, C)
    dc, ds, dx = _d(c, torch.int32), _d(s, torch.float16), _d(x, torch.bfloat16)
    out = torch.empty((M, R), dtype=torch.float32, device=DEV)
    junk = torch.empty((M, R), dtype=torch.float32, device=DEV)
    _check_replays(lambda: tq.matvec_axis1(dc, ds, dx, k, out_dtype=torch.float32, out=out), out,
                   lambda: tq.matvec_axis1(dc, ds, dx.flip(0).contiguous(), k, out_dtype=torch.float32, out=junk))


def test_graph_axis0():
    rng = np.random.default_rng(73)
    R, C, M, k = 3000, 1280, 4, 3
    c, s = ti.codes(rng, R, C, k), ti.scales(rng, R)
    x = ti.activations(rng, M, R)
    dc, ds, dx = _d(c, torch.int32), _d(s, torch.float16), _d(x, torch.bfloat16)
    lib = tq.load_library()
    ws = torch.empty(max(lib.trellis_matvec_axis0_workspace_bytes(R, C, M, k, 12, 256), 256),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((M, C), dtype=torch.bfloat16, device=DEV)
    junk = torch.empty((M, C), dtype=torch.bfloat16, device=DEV)
    _check_replays(lambda: tq.matvec_axis0(dc, ds, dx, k, out=out, workspace=ws), out,
                   lambda: (ws.fill_(0x7F), tq.matvec_axis0(dc, ds, dx.flip(0).contiguous(), k, out=junk,
                                                            workspace=ws)))


@pytest.mark.parametrize("algo,M", [(tq.PREFILL_FUSED, 24), (tq.PREFILL_FUSED, 100), (tq.PREFILL_EXPAND_GEMM, 40)])
def test_graph_prefill(algo, M):
    # 1000 x 1024: at M = 24 the register-direct kernel (column chunks + fold); at M = 100 8 tiles
    # of 128 x 128, all split along C (main kernel + fold); the expand + GEMM plan is tuned by the
    # eager call before capture.
    rng = np.random.default_rng(74)
    R, C, k = 1000, 1024, 3
    c, s = ti.codes(rng, R, C, k), ti.scales(rng, R)
    x = ti.activations(rng, M, C)
    dc, ds, dx = _d(c, torch.int32), _d(s, torch.float16), _d(x, torch.bfloat16)
    ws = torch.empty(max(tq.prefill_workspace_bytes(R, C, M, k, algo), 256), dtype=torch.uint8, device=DEV)
    out = torch.empty((M, R), dtype=torch.bfloat16, device=DEV)
    junk = torch.empty((M, R), dtype=torch.bfloat16, device=DEV)
    _check_replays(lambda: tq.prefill(dc, ds, dx, k, algo=algo, out=out, workspace=ws), out,
                   lambda: (ws.fill_(0x7F), tq.prefill(dc, ds, dx.flip(0).contiguous(), k, algo=algo, out=junk,
                                                        workspace=ws)))


@pytest.mark.parametrize("R_in,C_out", [(384, 1024), (640, 38400)])
def test_graph_prefill_axis0_fused(R_in, C_out):
    # M = 40 (128-row x tiles, two workgroups per CU): 1024 outputs make 8 tiles, all split along
    # the stored rows; 38400 make 300 tiles, dealt out stream-K (pieces folded)
    rng = np.random.default_rng(75)
    M, k = 40, 3
    c, s = ti.codes(rng, R_in, C_out, k), ti.scales(rng, R_in)
    x = ti.activations(rng, M, R_in)
    dc, ds, dx = _d(c, torch.int32), _d(s, torch.float16), _d(x, torch.bfloat16)
    lib = tq.load_library()
    nbytes = lib.trellis_prefill_axis0_workspace_bytes(R_in, C_out, M, k, 12, 256, tq.PREFILL_FUSED)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    out = torch.empty((M, C_out), dtype=torch.bfloat16, device=DEV)
    junk = torch.empty((M, C_out), dtype=torch.bfloat16, device=DEV)
    fused = tq.PREFILL_FUSED
    _check_replays(lambda: tq.prefill_axis0(dc, ds, dx, k, algo=fused, out=out, workspace=ws), out,
                   lambda: (ws.fill_(0x7F), tq.prefill_axis0(dc, ds, dx.flip(0).contiguous(), k, algo=fused,
                                                             out=junk, workspace=ws)))

