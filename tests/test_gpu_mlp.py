"""GPU parity of trellis_mlp_decode: down(silu(gate(x)) * up(x)) for M <= 4.

Both stages are held to the oracle: the hidden vectors (bf16) against the
oracle's gate and up sums through the SwiGLU cast chain, and the output
against the oracle's axis-0 sums of those same hidden vectors (so a 1-ulp
rounding choice in the first stage is not charged to the second).  Without
a `hidden` buffer the call must give the same bits (same kernels, the
hidden vectors in the workspace).
"""
import numpy as np
import pytest
import torch

import oracle
import trellis_coded_quantized_amd as tq
import trellis_inputs as ti
from tests import tolerance as tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
L, T = 12, 256


def _d(a, dtype):
    view = {torch.int32: np.int32, torch.float16: np.int16, torch.bfloat16: np.int16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(a).view(view)).to(DEV).view(dtype)


def _u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_mlp(g, u, d, x, R, C, C_out, M, k_gu, k_down, what, want_gu=None):
    dg, dgs, du, dus = _d(g.codes, torch.int32), _d(g.scales, torch.float16), _d(u.codes, torch.int32), _d(u.scales, torch.float16)
    dd, dds = _d(d.codes, torch.int32), _d(d.scales, torch.float16)
    dx = _d(x[:M], torch.bfloat16)
    hidden = torch.empty((M, R), dtype=torch.bfloat16, device=DEV)
    out = tq.mlp_decode(dg, dgs, du, dus, dd, dds, dx, k_gu, k_down, hidden=hidden)
    out2 = tq.mlp_decode(dg, dgs, du, dus, dd, dds, dx, k_gu, k_down)
    torch.cuda.synchronize()
    if want_gu is None:
        want_gu = oracle.gateup_swiglu(g.codes, g.scales, u.codes, u.scales, x, M, R, C, k_gu, L, T, with_abs=True)
    gw, uw, _, ga, ua = want_gu
    h = _u16(hidden)
    tol.assert_swiglu_close(h, gw[:M], uw[:M], ga[:M], ua[:M], what + " hidden")
    want, cond = oracle.matvec_axis0(d.codes, d.scales, h, M, R, C_out, k_down, L, T, with_abs=True)
    tol.assert_bf16_close(_u16(out), want, cond, what + " out")
    assert np.array_equal(_u16(out), _u16(out2)), what + ": hidden in the workspace changes the output"


class _Mat:
    def __init__(self, codes, scales):
        self.codes, self.scales = codes, scales


def _rand(rng, R, C, k):
    return _Mat(ti.codes(rng, R, C, k), ti.scales(rng, R))


@pytest.mark.parametrize("R,C,C_out,M,k_gu,k_down", [
    (512, 1280, 768, 1, 2, 3),
    (1000, 2560, 1280, 3, 4, 2),
    (88, 768, 512, 4, 3, 4),
    (2048, 5120, 1024, 2, 2, 2),
])
def test_mlp_small(R, C, C_out, M, k_gu, k_down):
    rng = np.random.default_rng(R + C + C_out + M)
    g, u, d = _rand(rng, R, C, k_gu), _rand(rng, R, C, k_gu), _rand(rng, R, C_out, k_down)
    x = ti.activations(rng, M, C)
    check_mlp(g, u, d, x, R, C, C_out, M, k_gu, k_down, f"mlp R={R} C={C} C_out={C_out} M={M} k={k_gu}/{k_down}")


@pytest.fixture(scope="module")
def mlp_workload():
    w = ti.gateup()
    g, u = w.mats
    d = ti.axis0().mats[0]                      # stored W_down^T [17408, 5120], k = 3
    want_gu = oracle.gateup_swiglu(g.codes, g.scales, u.codes, u.scales, w.x[0], 4, g.R, g.C, g.k, L, T,
                                   with_abs=True)
    return w, d, want_gu


@pytest.mark.parametrize("M", [1, 4])
def test_mlp_workload_17408x5120(mlp_workload, M):
    # gate/up 17408 x 5120 (k = 2) and down 5120 x 17408 stored transposed (k = 3)
    w, d, want_gu = mlp_workload
    g, u = w.mats
    check_mlp(g, u, d, w.x[0], g.R, g.C, d.C, M, g.k, d.k, f"mlp workload M={M}", want_gu=want_gu)


def test_mlp_graph_replay():
    rng = np.random.default_rng(77)
    R, C, C_out, M = 1000, 1280, 768, 4
    g, u, d = _rand(rng, R, C, 2), _rand(rng, R, C, 2), _rand(rng, R, C_out, 3)
    x = ti.activations(rng, M, C)
    args = [_d(g.codes, torch.int32), _d(g.scales, torch.float16), _d(u.codes, torch.int32),
            _d(u.scales, torch.float16), _d(d.codes, torch.int32), _d(d.scales, torch.float16)]
    dx = _d(x, torch.bfloat16)
    lib = tq.load_library()
    ws = torch.zeros(lib.trellis_mlp_decode_workspace_bytes(R, C, C_out, M, 2, 3, L, T), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty((M, C_out), dtype=torch.bfloat16, device=DEV)
    tq.mlp_decode(*args, dx, 2, 3, out=out, workspace=ws)
    torch.cuda.synchronize()
    want = out.clone()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        tq.mlp_decode(*args, dx, 2, 3, out=out, workspace=ws)
    for rep in range(3):
        out.zero_()
        ws.fill_(0x5A)                          # the call rewrites its workspace
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {rep}"
