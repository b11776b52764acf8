"""trellis_matvec_axis0_noalloc (static device scratch, no workspace argument)
through the C ABI, against trellis_matvec_axis0 with a caller workspace: the
same kernels, so the outputs must agree bit for bit.  Two calls in a row,
the second on a smaller problem, so the second reads a scratch array that
still holds the first call's partials."""
import ctypes

import numpy as np
import pytest
import torch

import trellis_coded_quantized_amd as tq
import trellis_inputs as ti

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
L, T = 12, 256


def _d(a, dtype):
    view = {torch.int32: np.int32, torch.float16: np.int16, torch.bfloat16: np.int16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(a).view(view)).to(DEV).view(dtype)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_noalloc_matches_the_workspace_call_on_two_calls():
    lib = tq.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    cases = [(17408, 5120, 4, 3, 31), (3000, 1280, 2, 2, 32)]       # the second smaller
    for R, C, M, k, seed in cases:
        print(f"[noalloc] R={R} C={C} M={M} k={k}", flush=True)
        rng = np.random.default_rng(seed)
        codes = _d(ti.codes(rng, R, C, k), torch.int32)
        scales = _d(ti.scales(rng, R), torch.float16)
        x = _d(ti.activations(rng, M, R), torch.bfloat16)
        for od, dt in ((tq.OUT_F32, torch.float32), (tq.OUT_BF16, torch.bfloat16)):
            ref = torch.empty((M, C), dtype=dt, device=DEV)
            got = torch.full((M, C), 7.0, dtype=dt, device=DEV)
            wsb = lib.trellis_matvec_axis0_workspace_bytes(R, C, M, k, L, T)
            ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
            assert lib.trellis_matvec_axis0(_p(codes), _p(scales), _p(x), _p(ref), od, R, C, M, k, L, T, _p(ws),
                                            wsb, stream) == tq.OK, lib.trellis_last_error()
            assert lib.trellis_matvec_axis0_noalloc(_p(codes), _p(scales), _p(x), _p(got), od, R, C, M, k, L, T,
                                                    stream) == tq.OK, lib.trellis_last_error()
            torch.cuda.synchronize()
            bits = torch.int32 if dt == torch.float32 else torch.int16
            assert torch.equal(got.view(bits), ref.view(bits)), f"R={R} C={C} M={M} k={k} {dt}"
