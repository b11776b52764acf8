"""The block-interleaved k = 3 axis-0 code layout [C/512, R, 48] on the GPU.

The layout is a permutation of the row-major words: block b of row r moves
to group b // 2, row r, half b % 2.  Built here from row-major codes with
numpy (the layout's definition), the interleaved calls must give the
oracle's expansion bit for bit and the same matvec bits as the row-major
call on the same symbols (same decode, same accumulation order), which the
row-major tests hold to the oracle; the matvec is also checked against the
oracle directly.
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
L, T, K = 12, 256, 3
WPB = T * K // 32


def interleave(codes, R, C):
    """row-major [R, C*3/32] -> [C/512, R, 48]"""
    return np.ascontiguousarray(codes.reshape(R, C // 512, 2 * WPB).transpose(1, 0, 2))


def _d(a, dtype):
    view = {torch.int32: np.int32, torch.float16: np.int16, torch.bfloat16: np.int16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(a).view(view)).to(DEV).view(dtype)


def _u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_interleave_is_a_permutation_of_blocks():
    rng = np.random.default_rng(5)
    R, C = 3, 1024
    codes = ti.codes(rng, R, C, K)
    il = interleave(codes, R, C)
    for r in range(R):
        for b in range(C // T):
            assert np.array_equal(il[b // 2, r, (b % 2) * WPB:(b % 2 + 1) * WPB], codes[r, b * WPB:(b + 1) * WPB])


@pytest.mark.parametrize("R,C", [(5, 512), (300, 1536), (1000, 5120)])
def test_expand_interleaved(R, C):
    rng = np.random.default_rng(R + C)
    codes, scales = ti.codes(rng, R, C, K), ti.scales(rng, R)
    got = _u16(tq.expand_bf16(_d(interleave(codes, R, C), torch.int32), _d(scales, torch.float16), K))
    assert np.array_equal(got, oracle.expand_bf16(codes, scales, R, C, K, L, T))


@pytest.mark.parametrize("R,C,M", [(1, 512, 1), (200, 1024, 3), (2000, 5120, 4)])
def test_axis0_interleaved(R, C, M):
    rng = np.random.default_rng(3 * R + C + M)
    codes, scales = ti.codes(rng, R, C, K), ti.scales(rng, R)
    x = ti.activations(rng, M, R)
    dil, drm = _d(interleave(codes, R, C), torch.int32), _d(codes, torch.int32)
    ds, dx = _d(scales, torch.float16), _d(x, torch.bfloat16)
    got = tq.matvec_axis0(dil, ds, dx, K, out_dtype=torch.float32)
    ref = tq.matvec_axis0(drm, ds, dx, K, out_dtype=torch.float32)
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    want, cond = oracle.matvec_axis0(codes, scales, x, M, R, C, K, L, T, with_abs=True)
    tol.assert_f32_close(got.cpu().numpy(), want, cond, f"axis0 interleaved R={R} C={C} M={M}")
    got16 = tq.matvec_axis0(dil, ds, dx, K)
    assert torch.equal(got16.view(torch.int16), tq.matvec_axis0(drm, ds, dx, K).view(torch.int16))


def test_axis0_interleaved_workload_17408x5120_k3():
    w = ti.axis0()
    m = w.mats[0]
    dil, drm = _d(interleave(m.codes, m.R, m.C), torch.int32), _d(m.codes, torch.int32)
    ds, dx = _d(m.scales, torch.float16), _d(w.x[0], torch.bfloat16)
    for M in (1, 4):
        got = tq.matvec_axis0(dil, ds, dx[:M], K)
        ref = tq.matvec_axis0(drm, ds, dx[:M], K)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), M


@pytest.mark.parametrize("algo", [tq.PREFILL_FUSED, tq.PREFILL_EXPAND_GEMM, tq.PREFILL_AUTO])
@pytest.mark.parametrize("R,C,M", [(384, 512, 40), (640, 1536, 300), (128, 1024, 5)])
def test_prefill_axis0_interleaved(algo, R, C, M):
    # the axis-0 prefill on block-interleaved codes: bit-identical to the row-major call, and the oracle
    rng = np.random.default_rng(5 * R + C + M + algo)
    codes, scales = ti.codes(rng, R, C, K), ti.scales(rng, R)
    x = ti.activations(rng, M, R)
    ds, dx = _d(scales, torch.float16), _d(x, torch.bfloat16)
    got = tq.prefill_axis0(_d(interleave(codes, R, C), torch.int32), ds, dx, K, algo=algo)
    ref = tq.prefill_axis0(_d(codes, torch.int32), ds, dx, K, algo=algo)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    want, cond = oracle.prefill_axis0_sums(codes, scales, x, M, R, C, K, L, T, np.arange(M), np.arange(C),
                                           with_abs=True)
    tol.assert_bf16_close(_u16(got), want, cond, f"prefill axis0 interleaved R={R} C={C} M={M} algo={algo}")


def test_prefill_axis0_interleaved_down_17408x5120_k3():
    m = ti.axis0().mats[0]
    x = _d(ti.activations(np.random.default_rng(3), 512, m.R), torch.bfloat16)
    ds = _d(m.scales, torch.float16)
    dil, drm = _d(interleave(m.codes, m.R, m.C), torch.int32), _d(m.codes, torch.int32)
    for algo in (tq.PREFILL_FUSED, tq.PREFILL_EXPAND_GEMM):
        got = tq.prefill_axis0(dil, ds, x, K, algo=algo)
        ref = tq.prefill_axis0(drm, ds, x, K, algo=algo)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), algo
