"""Host-side checks of the C-ABI library (no GPU, no launches).

The library must load on a machine without a GPU, export every symbol that
include/trellis.h declares, and reject every invalid call on the host
before any launch (status code + message).  Only invalid calls are made
here, so no pointer is ever dereferenced.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import trellis_coded_quantized_amd as tq
from tests import tolerance as tol

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "trellis.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(trellis_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(tq.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = tq.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert "gfx950" in tq.version()


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced
MIS = ctypes.c_void_p((1 << 20) + 4)     # misaligned by 4 bytes


def call_axis1(codes=FAKE, scales=FAKE, x=FAKE, out=FAKE, od=0, R=512, C=2048, M=1, k=2, L=12, T=256):
    lib = tq.load_library()
    return lib.trellis_matvec_axis1(codes, scales, x, out, od, R, C, M, k, L, T, None, 0, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(k=1), tq.EUNSUPPORTED, "k=1"),
    (dict(k=5), tq.EUNSUPPORTED, "k=5"),
    (dict(L=16), tq.EUNSUPPORTED, "L=16"),
    (dict(T=128), tq.EUNSUPPORTED, "T=128"),
    (dict(C=2000), tq.EINVAL, "multiple of the block"),
    (dict(R=0), tq.EINVAL, "empty"),
    (dict(C=0), tq.EINVAL, "empty"),
    (dict(M=0), tq.EINVAL, "M=0"),
    (dict(M=5), tq.EINVAL, "M=5"),
    (dict(od=7), tq.EINVAL, "out_dtype"),
    (dict(codes=None), tq.EINVAL, "codes is NULL"),
    (dict(x=MIS), tq.EINVAL, "x not 16-byte aligned"),
    (dict(out=None), tq.EINVAL, "out is NULL"),
    (dict(R=1 << 31), tq.EINVAL, "too large"),
])
def test_axis1_rejects_on_host(kw, status, needle):
    assert call_axis1(**kw) == status
    assert needle in tq.load_library().trellis_last_error().decode()


def test_gateup_rejects_on_host():
    lib = tq.load_library()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 17408, 5120, 4, 2, 12, 256, None, 0, None]
    bad = list(args)
    bad[2] = None
    assert lib.trellis_gateup_swiglu(*bad) == tq.EINVAL
    assert "ucodes is NULL" in lib.trellis_last_error().decode()
    bad = list(args)
    bad[10] = 5
    assert lib.trellis_gateup_swiglu(*bad) == tq.EINVAL
    bad = list(args)
    bad[6] = ctypes.c_void_p((1 << 20) + 2)
    assert lib.trellis_gateup_swiglu(*bad) == tq.EINVAL
    assert "gate_f32" in lib.trellis_last_error().decode()


def test_axis0_workspace_is_checked():
    lib = tq.load_library()
    need = lib.trellis_matvec_axis0_workspace_bytes(17408, 5120, 4, 3, 12, 256)
    assert need > 0
    rc = lib.trellis_matvec_axis0(FAKE, FAKE, FAKE, FAKE, 0, 17408, 5120, 4, 3, 12, 256, FAKE,
                                  need - 1, None)
    assert rc == tq.EWORKSPACE
    assert "workspace" in lib.trellis_last_error().decode()
    assert lib.trellis_matvec_axis0_workspace_bytes(17408, 5120, 4, 5, 12, 256) == 0


def test_prefill_validation_and_workspace():
    lib = tq.load_library()
    R, C = 17408, 5120
    need = lib.trellis_prefill_workspace_bytes(R, C, 512, 2, 12, 256, tq.PREFILL_EXPAND_GEMM)
    assert need >= R * C * 2
    rc = lib.trellis_prefill(FAKE, FAKE, FAKE, FAKE, R, C, 512, 2, 12, 256, tq.PREFILL_EXPAND_GEMM,
                             FAKE, need - 1, None)
    assert rc == tq.EWORKSPACE
    assert lib.trellis_prefill(FAKE, FAKE, FAKE, FAKE, R, C, 512, 2, 12, 256, 9, None, 0, None) == tq.EINVAL
    assert lib.trellis_prefill(FAKE, FAKE, FAKE, FAKE, R, C, 0, 2, 12, 256, 0, None, 0, None) == tq.EINVAL


def test_expand_and_decode_reject_on_host():
    lib = tq.load_library()
    assert lib.trellis_expand_bf16(FAKE, FAKE, None, 4, 256, 2, 12, 256, None) == tq.EINVAL
    assert lib.trellis_expand_bf16(FAKE, FAKE, FAKE, 4, 256, 3, 12, 255, None) == tq.EUNSUPPORTED
    assert lib.trellis_decode_states(MIS, 4, 256, 2, 12, 256, None, None, None, None) == tq.EINVAL
    assert lib.trellis_last_error().decode().startswith("trellis_decode_states")


# ---- the parity criteria themselves ------------------------------------

def test_tolerance_helpers():
    o = np.array([1.0, -2.5, 3.0e-3, 0.0, 100.0])
    a = np.abs(o)                               # no cancellation: the floor is |o|
    assert tol.f32_rel_error(o * (1 + 5e-6), o, a).max() <= 1e-5
    assert tol.f32_rel_error(o * (1 + 5e-5), o, a).max() > 1e-5
    bits = tol.bf16_bits_from_f64(o)
    assert not tol.bf16_band_violations(bits, o, a).any()
    assert not tol.bf16_band_violations(bits + np.uint16(1), o, a).any()    # one ulp away (positive values)
    two = bits.copy()
    two[0] += 2
    assert tol.bf16_band_violations(two, o, a)[0]
    assert tol.bf16_key(np.array([0x8000], np.uint16))[0] == tol.bf16_key(np.array([0], np.uint16))[0]
    # a cancelling sum is measured against 2^-6 of its terms: an error of 1e-5 / 64 * a passes, 1e-5 / 32 * a
    # does not
    o2, a2 = np.array([1e-9]), np.array([64.0])
    assert tol.f32_rel_error(o2 + 0.99e-5, o2, a2)[0] <= 1e-5
    assert tol.f32_rel_error(o2 + 2e-5, o2, a2)[0] > 1e-5
    assert abs(tol.roundoff_units(o2 + 64 * 2.0 ** -24, o2, a2) - 1.0) < 1e-9


def call_mlp(x=FAKE, out=FAKE, hidden=None, R=1024, C=2048, C_out=1024, M=2, kg=2, kd=3, ws=None, wsb=0):
    lib = tq.load_library()
    return lib.trellis_mlp_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, x, hidden, out, R, C, C_out, M, kg, kd, 12,
                                  256, ws, wsb, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(M=5), tq.EINVAL, "M=5"),
    (dict(M=0), tq.EINVAL, "M=0"),
    (dict(kd=5), tq.EUNSUPPORTED, "k=5"),
    (dict(kg=1), tq.EUNSUPPORTED, "k=1"),
    (dict(C_out=1000), tq.EINVAL, "C=1000"),
    (dict(x=MIS), tq.EINVAL, "x not 16-byte aligned"),
    (dict(hidden=MIS), tq.EINVAL, "hidden not 16-byte aligned"),
])
def test_mlp_decode_rejects(kw, status, needle):
    assert call_mlp(**kw) == status
    assert needle in tq.load_library().trellis_last_error().decode()


def test_mlp_decode_workspace_is_checked():
    lib = tq.load_library()
    need = lib.trellis_mlp_decode_workspace_bytes(1024, 2048, 1024, 2, 2, 3, 12, 256)
    assert need >= 2 * 1024 * 2                  # at least the hidden vectors
    assert call_mlp(ws=FAKE, wsb=need - 1) == tq.EWORKSPACE
    assert lib.trellis_mlp_decode_workspace_bytes(1024, 2048, 1024, 5, 2, 3, 12, 256) == 0


def test_prefill_axis0_fused_needs_whole_steps_and_checks_workspace():
    lib = tq.load_library()
    # the fused kernel takes the stored rows 32 per step, four steps at a time
    assert lib.trellis_prefill_axis0_workspace_bytes(6100, 5120, 64, 4, 12, 256, tq.PREFILL_FUSED) == 0
    st = lib.trellis_prefill_axis0(FAKE, FAKE, FAKE, FAKE, 6100, 5120, 64, 4, 12, 256, tq.PREFILL_FUSED, None, 0, None)
    assert st == tq.EUNSUPPORTED and "multiple of 128" in lib.trellis_last_error().decode()
    fneed = lib.trellis_prefill_axis0_workspace_bytes(6144, 5120, 64, 4, 12, 256, tq.PREFILL_FUSED)
    assert fneed >= 64 * 6144 * 2                # at least x in operand order
    st = lib.trellis_prefill_axis0(FAKE, FAKE, FAKE, FAKE, 6144, 5120, 64, 4, 12, 256, tq.PREFILL_FUSED,
                                   FAKE, fneed - 1, None)
    assert st == tq.EWORKSPACE
    assert lib.trellis_prefill_axis0_workspace_bytes(6144, 5120, 64, 4, 12, 256, 7) == 0
    st = lib.trellis_prefill_axis0(FAKE, FAKE, FAKE, FAKE, 6144, 5120, 64, 4, 12, 256, 7, FAKE, fneed, None)
    assert st == tq.EINVAL and "algo=7" in lib.trellis_last_error().decode()
    need = lib.trellis_prefill_axis0_workspace_bytes(6144, 5120, 64, 4, 12, 256, tq.PREFILL_EXPAND_GEMM)
    assert need >= 6144 * 5120 * 2
    st = lib.trellis_prefill_axis0(FAKE, FAKE, FAKE, FAKE, 6144, 5120, 64, 4, 12, 256, tq.PREFILL_EXPAND_GEMM,
                                   FAKE, need - 1, None)
    assert st == tq.EWORKSPACE
    st = lib.trellis_prefill_axis0(FAKE, FAKE, MIS, FAKE, 6144, 5120, 64, 4, 12, 256, tq.PREFILL_EXPAND_GEMM,
                                   FAKE, need, None)
    assert st == tq.EINVAL and "x not 16-byte aligned" in lib.trellis_last_error().decode()


@pytest.mark.parametrize("k,C,status,needle", [
    (2, 1024, tq.EUNSUPPORTED, "k=3 only"),
    (3, 768, tq.EINVAL, "not a multiple of 512"),
])
def test_interleaved_layout_rejects(k, C, status, needle):
    lib = tq.load_library()
    assert lib.trellis_matvec_axis0_il(FAKE, FAKE, FAKE, FAKE, 0, 1024, C, 2, k, 12, 256, None, 0, None) == status
    assert needle in lib.trellis_last_error().decode()
    assert lib.trellis_expand_bf16_il(FAKE, FAKE, FAKE, 1024, C, k, 12, 256, None) == status
    assert needle in lib.trellis_last_error().decode()


def test_prefill_auto_workspace_follows_the_chosen_algo():
    lib = tq.load_library()
    F, E, A = tq.PREFILL_FUSED, tq.PREFILL_EXPAND_GEMM, tq.PREFILL_AUTO
    ws = lib.trellis_prefill_workspace_bytes
    for M, algo in ((32, F), (128, F), (129, E), (2048, E)):
        assert ws(1024, 2048, M, 2, 12, 256, A) == ws(1024, 2048, M, 2, 12, 256, algo), M
    assert ws(1024, 2048, 32, 2, 12, 256, F) != ws(1024, 2048, 32, 2, 12, 256, E)
    ws0 = lib.trellis_prefill_axis0_workspace_bytes
    for R_in, M, algo in ((6144, 64, F), (6144, 512, F), (6144, 513, E), (6144, 2048, E), (6100, 64, E)):
        assert ws0(R_in, 5120, M, 3, 12, 256, A) == ws0(R_in, 5120, M, 3, 12, 256, algo), (R_in, M)
    assert ws(1024, 2048, 32, 2, 12, 256, 3) == 0


def test_axis1_group_rejects_on_host():
    lib = tq.load_library()
    P = ctypes.c_void_p * 5
    I = ctypes.c_int64 * 5
    ptrs, sc, outs, Rs = P(*[FAKE.value] * 5), P(*[FAKE.value] * 5), P(*[FAKE.value] * 5), I(*[64] * 5)

    def call(n=3, codes=ptrs, R=Rs, k=2, M=4, C=1024, x=FAKE):
        return lib.trellis_matvec_axis1_group(codes, sc, outs, R, n, x, tq.OUT_BF16, C, M, k, 12, 256, None)
    for kw, status, needle in (
            (dict(n=0), tq.EINVAL, "n=0"), (dict(n=5), tq.EINVAL, "n=5"),
            (dict(codes=None), tq.EINVAL, "NULL pointer array"), (dict(k=5), tq.EUNSUPPORTED, "k=5"),
            (dict(M=5), tq.EINVAL, "M=5"), (dict(x=MIS), tq.EINVAL, "x not 16-byte aligned"),
            (dict(R=I(64, 0, 64, 64, 64)), tq.EINVAL, "empty matrix"),
            (dict(codes=P(FAKE.value, MIS.value, FAKE.value, FAKE.value, FAKE.value)), tq.EINVAL, "codes[j]"),
            (dict(C=6144), tq.EUNSUPPORTED, "C=6144")):
        st = call(**kw)
        assert st == status and needle in lib.trellis_last_error().decode(), (kw, st, lib.trellis_last_error())



def test_axis0_noalloc_rejects_on_host():
    lib = tq.load_library()
    # partials of 327680 outputs x 4 vectors need more than the 4 MiB static scratch
    assert lib.trellis_matvec_axis0_noalloc(FAKE, FAKE, FAKE, FAKE, tq.OUT_F32, 32, 327680, 4, 3, 12, 256,
                                            None) == tq.EUNSUPPORTED
    assert "static scratch" in lib.trellis_last_error().decode()
    assert lib.trellis_matvec_axis0_noalloc(None, FAKE, FAKE, FAKE, tq.OUT_F32, 32, 512, 4, 3, 12, 256,
                                            None) == tq.EINVAL
    assert lib.trellis_matvec_axis0_noalloc(FAKE, FAKE, FAKE, FAKE, tq.OUT_F32, 32, 512, 5, 3, 12, 256,
                                            None) == tq.EINVAL
    assert lib.trellis_matvec_axis0_noalloc(FAKE, FAKE, FAKE, FAKE, 7, 32, 512, 4, 3, 12, 256, None) == tq.EINVAL
