"""GPU parity of trellis_matvec_axis1_group: a projection set over one x in
one launch.

Every output must equal, bit for bit, what trellis_matvec_axis1 writes for
that matrix alone (same kernel, same per-row arithmetic: only the mapping of
row groups to matrices changes), and is held to the oracle as well.  Shapes:
ragged row counts (not multiples of 16) so row groups of different matrices
meet mid-launch, a 64-row matrix that alone would fill 4 workgroups, and the
decoder-layer projection set 10240 / 6144 / 64 x 5120 at k = 4.
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


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def _run(Rs, C, k, M, seed, out_dtype, check_oracle=True):
    rng = np.random.default_rng(seed)
    mats = [(ti.codes(rng, R, C, k), ti.scales(rng, R)) for R in Rs]
    x = ti.activations(rng, M, C)
    dx = _d(x, torch.bfloat16)
    dc = [_d(c, torch.int32) for c, _ in mats]
    ds = [_d(s, torch.float16) for _, s in mats]
    outs = tq.matvec_axis1_group(dc, ds, dx, k, out_dtype=out_dtype)
    singles = [tq.matvec_axis1(c, s, dx, k, out_dtype=out_dtype) for c, s in zip(dc, ds)]
    torch.cuda.synchronize()
    for R, o, s1 in zip(Rs, outs, singles):
        assert o.shape == (M, R)
        np.testing.assert_array_equal(_bits(o), _bits(s1), err_msg=f"R={R}: grouped call differs from the single call")
    if check_oracle:
        for (c, s), R, o in zip(mats, Rs, outs):
            want, cond = oracle.matvec_axis1(c, s, x, M, R, C, k, L, T, with_abs=True)
            if out_dtype == torch.float32:
                tol.assert_f32_close(o.cpu().numpy(), want, cond, f"group R={R}")
            else:
                tol.assert_bf16_close(_bits(o).view(np.uint16), want, cond, f"group R={R}")


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("M", [1, 4])
def test_group_ragged(k, M):
    _run((1000, 520, 64, 33), 1024, k, M, 300 + k + M, torch.float32)


def test_group_of_one_and_bf16_out():
    _run((777,), 2048, 3, 2, 311, torch.bfloat16)
    _run((16, 1, 300), 5120, 2, 3, 312, torch.bfloat16)


def test_group_decoder_layer_projections_k4():
    # the decoder-layer set: 10240, 6144 and 64 rows over one x [4, 5120]
    _run((10240, 6144, 64), 5120, 4, 4, 313, torch.float32)


def test_group_scales_at_odd_offset():
    # one matrix's scales start 2 bytes into an allocation: the launch reads
    # every scale from global memory instead of its LDS copy, and the outputs
    # must not change
    rng = np.random.default_rng(314)
    Rs, C, k, M = (300, 77, 64), 1024, 3, 4
    mats = [(ti.codes(rng, R, C, k), ti.scales(rng, R)) for R in Rs]
    dx = _d(ti.activations(rng, M, C), torch.bfloat16)
    dc = [_d(c, torch.int32) for c, _ in mats]
    ds = [_d(s, torch.float16) for _, s in mats]
    big = torch.empty(Rs[1] + 1, dtype=torch.float16, device=DEV)
    odd = big[1:]
    odd.copy_(ds[1])
    assert odd.data_ptr() % 4 == 2
    want = tq.matvec_axis1_group(dc, ds, dx, k, out_dtype=torch.float32)
    got = tq.matvec_axis1_group(dc, [ds[0], odd, ds[2]], dx, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for R, a, b in zip(Rs, want, got):
        np.testing.assert_array_equal(_bits(b), _bits(a), err_msg=f"R={R}: odd-offset scales changed the outputs")
