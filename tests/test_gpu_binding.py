"""The binding's host checks on device tensors: a caller's output, scales or
workspace of the wrong size, dtype or place is refused with an exception
before anything is launched (the C library cannot see tensor shapes, so a
wrong-sized buffer would otherwise be written out of bounds)."""
import pytest
import torch

import trellis_coded_quantized_amd as tq

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _mats(R=64, C=512, k=2):
    codes = torch.zeros((R, C * k // 32), dtype=torch.int32, device=DEV)
    scales = torch.ones(R, dtype=torch.float16, device=DEV)
    return codes, scales


def test_wrong_output_shapes_are_refused():
    codes, scales = _mats()
    x = torch.zeros((2, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="shape"):
        tq.matvec_axis1(codes, scales, x, 2, out=torch.empty((2, 63), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="shape"):
        tq.gateup_swiglu(codes, scales, codes, scales, x, 2, out=torch.empty((3, 64), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="shape"):
        tq.gateup_swiglu(codes, scales, codes, scales, x, 2, gate_f32=torch.empty((2, 32), device=DEV))
    with pytest.raises(ValueError, match="shape"):
        tq.prefill(codes, scales, x, 2, out=torch.empty((2, 65), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="shape"):
        tq.expand_bf16(codes, scales, 2, out=torch.empty((64, 256), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match=r"outputs for"):
        tq.matvec_axis1_group([codes, codes], [scales, scales], x, 2, outs=[torch.empty((2, 64), device=DEV)])
    with pytest.raises(ValueError, match="shape"):
        tq.matvec_axis1_group([codes], [scales], x, 2, outs=[torch.empty((2, 60), device=DEV)])
    xt = torch.zeros((2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="shape"):
        tq.matvec_axis0(codes, scales, xt, 2, out=torch.empty((2, 500), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="shape"):
        tq.prefill_axis0(codes, scales, xt, 2, out=torch.empty((1, 512), dtype=torch.bfloat16, device=DEV))


def test_wrong_scales_dtypes_and_workspaces_are_refused():
    codes, scales = _mats()
    x = torch.zeros((2, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="stored rows"):
        tq.matvec_axis1(codes, scales[:63], x, 2)
    with pytest.raises(ValueError, match="stored rows"):
        tq.prefill(codes, torch.ones(65, dtype=torch.float16, device=DEV), x, 2)
    with pytest.raises(ValueError, match="out_dtype"):
        tq.matvec_axis1(codes, scales, x, 2, out_dtype=torch.float16)
    with pytest.raises(ValueError, match="workspace"):
        tq.prefill(codes, scales, x, 2, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(TypeError):
        tq.matvec_axis1(codes, scales, x, 2, out=torch.empty((2, 64), dtype=torch.float16, device=DEV))
