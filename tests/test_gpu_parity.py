"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Decoded states, codes, values and bf16 expansions must match bit for bit;
matvec sums within the floored 1e-5 relative criterion in f32 and the bf16
band of tests/tolerance.py; the SwiGLU output within the candidate band of
its cast chain.  Inputs follow trellis_inputs (seeded, synthetic).  Full
workload sizes are compared in full where the oracle takes seconds, and on
sampled outputs for the prefill.
"""
import numpy as np
import pytest
import torch

import oracle
import trellis_coded_quantized_amd as tq
import trellis_inputs as ti
from tests import tolerance as tol

pytestmark = pytest.mark.gpu

L, T = 12, 256
DEV = "cuda:0"


def d_codes(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(DEV)


def d_half(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.float16)


def d_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def h_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rand_matrix(rng, R, C, k):
    return ti.codes(rng, R, C, k), ti.scales(rng, R)


# ------------------------------------------------------------------ decode

def crafted_codes(R, C, k):
    words = C * k // 32
    pats = [0x00000000, 0xFFFFFFFF, 0xAAAAAAAA, 0x55555555, 0x80000001, 0x0F0F0F0F]
    a = np.empty((R, words), np.uint32)
    for r in range(R):
        a[r] = pats[r % len(pats)]
    return a


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("R,C,kind", [(5, 1024, "random"), (6, 256, "crafted"), (1, 256, "random")])
def test_decode_states_bit_exact(k, R, C, kind):
    rng = np.random.default_rng(40 + k)
    codes = ti.codes(rng, R, C, k) if kind == "random" else crafted_codes(R, C, k)
    st, ys, vals = tq.decode_states(d_codes(codes), k)
    ost, oys, ovals = oracle.decode(codes, R, C, k, L, T)
    assert np.array_equal(st.cpu().numpy().view(np.uint16), ost)
    assert np.array_equal(ys.cpu().numpy(), oys)
    assert np.array_equal(vals.cpu().numpy().view(np.uint32), ovals.view(np.uint32))


@pytest.mark.parametrize("wl,k", [("gateup", 2), ("axis0", 3), ("layer_chain", 4)])
def test_decode_states_workload_rows(wl, k):
    w = ti.WORKLOADS[wl]()
    m = w.mats[0]
    for rows in (slice(0, 16), slice(m.R - 16, m.R)):
        sub = np.ascontiguousarray(m.codes[rows])
        st, ys, vals = tq.decode_states(d_codes(sub), k)
        ost, oys, ovals = oracle.decode(sub, sub.shape[0], m.C, k, L, T)
        assert np.array_equal(st.cpu().numpy().view(np.uint16), ost)
        assert np.array_equal(vals.cpu().numpy().view(np.uint32), ovals.view(np.uint32))


# ------------------------------------------------------------------ axis 1

def check_axis1(codes, scales, x, R, C, M, k, what):
    want, cond = oracle.matvec_axis1(codes, scales, x, M, R, C, k, L, T, with_abs=True)
    dc, ds, dx = d_codes(codes), d_half(scales), d_bf16(x)
    got32 = tq.matvec_axis1(dc, ds, dx, k, out_dtype=torch.float32).cpu().numpy()
    print(f"[parity] {what}: {tol.margin_report(got32, want, cond)}", flush=True)
    tol.assert_f32_close(got32, want, cond, what + " f32")
    got16 = h_u16(tq.matvec_axis1(dc, ds, dx, k))
    tol.assert_bf16_close(got16, want, cond, what + " bf16")
    # metamorphic: a negated input gives the negated sums (within the f32
    # criterion: MFMA accumulation is not bitwise sign-symmetric)
    neg = tq.matvec_axis1(dc, ds, d_bf16(x ^ np.uint16(0x8000)), k, out_dtype=torch.float32).cpu().numpy()
    tol.assert_f32_close(neg, -want, cond, what + " negation")


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("R,C,M", [(1, 256, 1), (7, 1280, 4), (130, 768, 3), (67, 2304, 2)])
def test_axis1_small(k, R, C, M):
    rng = np.random.default_rng(R * 31 + C + M * 7 + k)
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, M, C)
    check_axis1(codes, scales, x, R, C, M, k, f"axis1 R={R} C={C} M={M} k={k}")


def test_axis1_workload_512x2048_k2_m1():
    w = ti.axis1_m1()
    m = w.mats[0]
    check_axis1(m.codes, m.scales, w.x[0], m.R, m.C, 1, m.k, w.name)


@pytest.mark.parametrize("R,C,k", [(300, 8192, 2), (100, 17408, 3), (67, 5376, 4)])
def test_axis1_wide_rows_column_chunks(R, C, k):
    # rows wider than 5120 columns run as column chunks (8192: 2 x 4096; 17408: 4 x 4352; 5376: 2816 + 2560)
    # into f32 partials in the workspace, folded by a second kernel
    rng = np.random.default_rng(R + C + k)
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, 4, C)
    for M in (1, 2, 3, 4):
        check_axis1(codes, scales, x[:M], R, C, M, k, f"axis1 R={R} C={C} M={M} k={k}")


def test_axis1_down_projection_stored_axis1_5120x17408_k3():
    # the MLP down projection stored along its inputs (axis 1): 5120 outputs x 17408 inputs
    rng = np.random.default_rng(17408)
    R, C, k = 5120, 17408, 3
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, 4, C)
    check_axis1(codes, scales, x, R, C, 4, k, "axis1 5120x17408 k3 M=4")


@pytest.mark.parametrize("R,C,M,k", [(129, 8192, 4, 2), (40, 17408, 1, 4), (64, 10240, 3, 3)])
def test_gateup_wide_rows_column_chunks(R, C, M, k):
    rng = np.random.default_rng(2 * R + C + M + k)
    g = ti.Matrix(1, R, C, k, *rand_matrix(rng, R, C, k))
    u = ti.Matrix(1, R, C, k, *rand_matrix(rng, R, C, k))
    x = ti.activations(rng, M, C)
    check_gateup(g, u, x, R, C, M, k, f"gateup R={R} C={C} M={M} k={k}")


@pytest.mark.parametrize("R", [33, 160])
def test_axis1_and_gateup_scales_at_odd_offset(R):
    # scales that start 2 bytes into an allocation (not 4-byte aligned) are
    # read from global memory instead of the LDS copy; the outputs must not
    # change at all
    rng = np.random.default_rng(4000 + R)
    C, k, M = 1280, 3, 4
    codes, scales = rand_matrix(rng, R, C, k)
    ucodes, uscales = rand_matrix(rng, R, C, k)
    x = d_bf16(ti.activations(rng, M, C))
    dc, uc = d_codes(codes), d_codes(ucodes)
    big = torch.empty(2 * R + 2, dtype=torch.float16, device=DEV)
    s_odd, u_odd = big[1:R + 1], big[R + 1:2 * R + 1]
    s_odd.copy_(d_half(scales))
    u_odd.copy_(d_half(uscales))
    assert s_odd.data_ptr() % 4 == 2
    a = tq.matvec_axis1(dc, d_half(scales), x, k, out_dtype=torch.float32)
    b = tq.matvec_axis1(dc, s_odd, x, k, out_dtype=torch.float32)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    ga = tq.gateup_swiglu(dc, d_half(scales), uc, d_half(uscales), x, k)
    gb = tq.gateup_swiglu(dc, s_odd, uc, u_odd, x, k)
    assert torch.equal(ga.view(torch.int16), gb.view(torch.int16))


def test_axis1_zero_input_is_exact_zero():
    rng = np.random.default_rng(3)
    codes, scales = rand_matrix(rng, 33, 512, 3)
    x = np.zeros((2, 512), np.uint16)
    got = tq.matvec_axis1(d_codes(codes), d_half(scales), d_bf16(x), 3, out_dtype=torch.float32)
    assert not got.cpu().numpy().any()


# ------------------------------------------------------------------ gate/up

def check_gateup(g, u, x, R, C, M, k, what, want=None):
    if want is None:
        want = oracle.gateup_swiglu(g.codes, g.scales, u.codes, u.scales, x, M, R, C, k, L, T, with_abs=True)
    og, ou, _, ga, ua = want
    dx = d_bf16(x[:M])
    gf = torch.empty((M, R), dtype=torch.float32, device=DEV)
    uf = torch.empty((M, R), dtype=torch.float32, device=DEV)
    out = tq.gateup_swiglu(d_codes(g.codes), d_half(g.scales), d_codes(u.codes), d_half(u.scales),
                           dx, k, gate_f32=gf, up_f32=uf)
    print(f"[parity] {what}: {tol.margin_report(gf.cpu().numpy(), og[:M], ga[:M])}",
          flush=True)
    tol.assert_f32_close(gf.cpu().numpy(), og[:M], ga[:M], what + " gate")
    tol.assert_f32_close(uf.cpu().numpy(), ou[:M], ua[:M], what + " up")
    tol.assert_swiglu_close(h_u16(out), og[:M], ou[:M], ga[:M], ua[:M], what + " swiglu")


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("R,C,M", [(1, 256, 1), (37, 1280, 4), (129, 512, 2)])
def test_gateup_small(k, R, C, M):
    rng = np.random.default_rng(R * 13 + C + M + k)
    g = ti.Matrix(1, R, C, k, *rand_matrix(rng, R, C, k))
    u = ti.Matrix(1, R, C, k, *rand_matrix(rng, R, C, k))
    x = ti.activations(rng, M, C)
    check_gateup(g, u, x, R, C, M, k, f"gateup R={R} C={C} M={M} k={k}")


@pytest.fixture(scope="module")
def gateup_workload():
    w = ti.gateup()
    g, u = w.mats
    want = oracle.gateup_swiglu(g.codes, g.scales, u.codes, u.scales, w.x[0], 4, g.R, g.C, g.k, L, T,
                                with_abs=True)
    return w, want


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_gateup_workload_17408x5120_k2(gateup_workload, M):
    w, want = gateup_workload
    g, u = w.mats
    check_gateup(g, u, w.x[0], g.R, g.C, M, g.k, f"{w.name} M={M}", want=want)


# ------------------------------------------------------------------ axis 0

def check_axis0(codes, scales, x, R, C, M, k, what, want=None):
    if want is None:
        want = oracle.matvec_axis0(codes, scales, x, M, R, C, k, L, T, with_abs=True)
    want, cond = want
    dc, ds, dx = d_codes(codes), d_half(scales), d_bf16(x[:M])
    got32 = tq.matvec_axis0(dc, ds, dx, k, out_dtype=torch.float32).cpu().numpy()
    print(f"[parity] {what}: {tol.margin_report(got32, want[:M], cond[:M])}", flush=True)
    tol.assert_f32_close(got32, want[:M], cond[:M], what + " f32")
    got16 = h_u16(tq.matvec_axis0(dc, ds, dx, k))
    tol.assert_bf16_close(got16, want[:M], cond[:M], what + " bf16")


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("R,C,M", [(1, 256, 1), (3, 768, 4), (200, 512, 2), (1000, 1280, 3)])
def test_axis0_small(k, R, C, M):
    rng = np.random.default_rng(R * 17 + C + M + k)
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, M, R)
    check_axis0(codes, scales, x, R, C, M, k, f"axis0 R={R} C={C} M={M} k={k}")


@pytest.fixture(scope="module")
def axis0_workload():
    w = ti.axis0()
    m = w.mats[0]
    return w, oracle.matvec_axis0(m.codes, m.scales, w.x[0], 4, m.R, m.C, m.k, L, T, with_abs=True)


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_axis0_workload_17408x5120_k3(axis0_workload, M):
    w, want = axis0_workload
    m = w.mats[0]
    check_axis0(m.codes, m.scales, w.x[0], m.R, m.C, M, m.k, f"{w.name} M={M}", want=want)


# ------------------------------------------------------------------ layer chain

def test_layer_chain_k4_m4():
    w = ti.layer_chain()
    outs = []
    for m, x in zip(w.mats, w.x):       # back to back on one stream
        fn = tq.matvec_axis1 if m.axis == 1 else tq.matvec_axis0
        outs.append(fn(d_codes(m.codes), d_half(m.scales), d_bf16(x), m.k, out_dtype=torch.float32))
    torch.cuda.synchronize()
    for m, x, o in zip(w.mats, w.x, outs):
        ref = oracle.matvec_axis1 if m.axis == 1 else oracle.matvec_axis0
        want, cond = ref(m.codes, m.scales, x, 4, m.R, m.C, m.k, L, T, with_abs=True)
        tol.assert_f32_close(o.cpu().numpy(), want, cond, f"{w.name} axis{m.axis} {m.R}x{m.C}")


# ------------------------------------------------------------------ expand

@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("R,C", [(1, 256), (9, 1280)])
def test_expand_bit_exact(k, R, C):
    rng = np.random.default_rng(R + C + k)
    codes, scales = rand_matrix(rng, R, C, k)
    got = h_u16(tq.expand_bf16(d_codes(codes), d_half(scales), k))
    assert np.array_equal(got, oracle.expand_bf16(codes, scales, R, C, k, L, T))


def test_expand_workload_rows_bit_exact():
    w = ti.prefill(Ms=(1,))
    m = w.mats[0]
    got = tq.expand_bf16(d_codes(m.codes), d_half(m.scales), m.k)
    for r0 in (0, m.R // 2, m.R - 32):
        want = oracle.expand_bf16(m.codes, m.scales, m.R, m.C, m.k, L, T, r0=r0, nr=32)
        assert np.array_equal(h_u16(got[r0:r0 + 32]), want), r0


# ------------------------------------------------------------------ prefill

ALGOS = [tq.PREFILL_FUSED, tq.PREFILL_EXPAND_GEMM]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("R,C,M", [(7, 256, 1), (200, 768, 5), (130, 512, 131)])
def test_prefill_small(algo, k, R, C, M):
    rng = np.random.default_rng(R + C + M + k)
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, M, C)
    got = h_u16(tq.prefill(d_codes(codes), d_half(scales), d_bf16(x), k, algo=algo))
    want, cond = oracle.prefill_sums(codes, scales, x, M, R, C, k, L, T, np.arange(M), np.arange(R), with_abs=True)
    tol.assert_bf16_close(got, want, cond, f"prefill algo={algo} R={R} C={C} M={M} k={k}")


@pytest.mark.parametrize("k", [2, 3])
@pytest.mark.parametrize("R,M", [(25600, 300), (38400, 100)])
def test_prefill_fused_stream_pieces(k, R, M):
    # M = 300: 200 tiles of 512 x 128 on a 256-CU part; M = 100: 300 tiles of 128 x 128 with two
    # workgroups per CU.  Either way the leftover tiles fill more than half of the workgroup
    # slots, so the fused kernel deals the steps out in ranges that cross tile boundaries (whole
    # tiles stored directly, the pieces folded).  Sampled rows and x rows.
    rng = np.random.default_rng(90 + k + M)
    C = 1280
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, M, C)
    got = tq.prefill(d_codes(codes), d_half(scales), d_bf16(x), k, algo=tq.PREFILL_FUSED)
    ms = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    rows = np.unique(np.concatenate([[0, 127, 128, 5119, 5120, R - 1], rng.integers(0, R, 120)]))
    want, cond = oracle.prefill_sums(codes, scales, x, M, R, C, k, L, T, ms, rows, with_abs=True)
    sub = h_u16(got[torch.as_tensor(ms, device=DEV)][:, torch.as_tensor(rows, device=DEV)])
    tol.assert_bf16_close(sub, want, cond, f"prefill stream pieces k={k}")


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("R,C,M", [(1000, 1024, 1), (1000, 1024, 32), (777, 512, 9), (777, 512, 16), (40, 256, 17),
                                   (4096, 5120, 32), (1000, 1024, 33), (777, 512, 48), (4096, 5120, 64)])
def test_prefill_direct(k, R, C, M):
    # M <= 64 runs the register-direct kernel: 32-row weight tiles (a ragged last one when
    # R % 32 != 0), column chunks split over workgroups and waves, one (M <= 32) or two x tiles,
    # x read in place up to 16 rows; every output
    rng = np.random.default_rng(500 + R + C + M + k)
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, M, C)
    got = h_u16(tq.prefill(d_codes(codes), d_half(scales), d_bf16(x), k, algo=tq.PREFILL_FUSED))
    want, cond = oracle.prefill_sums(codes, scales, x, M, R, C, k, L, T, np.arange(M), np.arange(R), with_abs=True)
    tol.assert_bf16_close(got, want, cond, f"direct prefill R={R} C={C} M={M} k={k}")


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("R,C", [(1000, 1024), (4096, 5120)])
def test_prefill_direct_x_in_place_matches_layout(k, R, C):
    # up to 16 rows the register-direct kernel reads x in place (no layout pass); from 17 rows
    # through the operand-order copy.  Same kernel arithmetic: the first M rows of a 17-row call
    # must equal an M-row call bit for bit, at the in-place boundary and below it
    rng = np.random.default_rng(700 + R + C + k)
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, 17, C)
    dc, ds, dx = d_codes(codes), d_half(scales), d_bf16(x)
    ref = tq.prefill(dc, ds, dx, k, algo=tq.PREFILL_FUSED)
    for M in (1, 7, 16):
        got = tq.prefill(dc, ds, dx[:M].contiguous(), k, algo=tq.PREFILL_FUSED)
        assert torch.equal(got.view(torch.int16), ref[:M].view(torch.int16)), f"R={R} C={C} k={k} M={M}"


@pytest.mark.parametrize("M", [32, 33, 64, 65, 128, 129, 256, 257])
def test_prefill_fused_tile_size_boundaries(M):
    # M = 32 / 33: one and two x tiles in the register-direct kernel; 64 is its last size, 65 the
    # first on 128-row x tiles;
    # M = 256 is the last size on 128-row tiles (2 row tiles), 257 the first on 512-row tiles
    # (rows 257..511 of the tile padded); 128 / 129 straddle the one-tile case.  Every output.
    R, C, k = 640, 1024, 2
    rng = np.random.default_rng(400 + M)
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, M, C)
    got = h_u16(tq.prefill(d_codes(codes), d_half(scales), d_bf16(x), k, algo=tq.PREFILL_FUSED))
    want, cond = oracle.prefill_sums(codes, scales, x, M, R, C, k, L, T, np.arange(M), np.arange(R), with_abs=True)
    tol.assert_bf16_close(got, want, cond, f"fused prefill tile boundary M={M}")


@pytest.mark.parametrize("M", [256, 257])
def test_prefill_axis0_fused_tile_size_boundaries(M):
    R_in, C_out, k = 512, 768, 4
    rng = np.random.default_rng(410 + M)
    codes, scales = rand_matrix(rng, R_in, C_out, k)
    x = ti.activations(rng, M, R_in)
    got = h_u16(tq.prefill_axis0(d_codes(codes), d_half(scales), d_bf16(x), k, algo=tq.PREFILL_FUSED))
    want, cond = oracle.prefill_axis0_sums(codes, scales, x, M, R_in, C_out, k, L, T, np.arange(M), np.arange(C_out), with_abs=True)
    tol.assert_bf16_close(got, want, cond, f"fused prefill axis0 tile boundary M={M}")


@pytest.fixture(scope="module")
def prefill_workload():
    return ti.prefill()


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("M", [32, 512, 2048])
def test_prefill_workload_17408x5120_k2(prefill_workload, algo, M):
    w = prefill_workload
    m = w.mats[0]
    x = w.x[0][:M]
    got = tq.prefill(d_codes(m.codes), d_half(m.scales), d_bf16(x), m.k, algo=algo)
    rng = np.random.default_rng(M)
    ms = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    rows = np.unique(np.concatenate([[0, 1, m.R - 1], rng.integers(0, m.R, 61)]))
    want, cond = oracle.prefill_sums(m.codes, m.scales, x, M, m.R, m.C, m.k, L, T, ms, rows, with_abs=True)
    sub = h_u16(got[torch.as_tensor(ms, device=DEV)][:, torch.as_tensor(rows, device=DEV)])
    tol.assert_bf16_close(sub, want, cond, f"{w.name} algo={algo} M={M}")


# ------------------------------------------------------------------ axis-0 prefill

@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("R,C,M", [(300, 512, 40), (1000, 1280, 5)])
def test_prefill_axis0_small(k, R, C, M):
    rng = np.random.default_rng(R + C + M + 7 * k)
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, M, R)
    got = h_u16(tq.prefill_axis0(d_codes(codes), d_half(scales), d_bf16(x), k))
    want, cond = oracle.prefill_axis0_sums(codes, scales, x, M, R, C, k, L, T, np.arange(M), np.arange(C), with_abs=True)
    tol.assert_bf16_close(got, want, cond, f"prefill axis0 R={R} C={C} M={M} k={k}")


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("R,C,M", [(384, 512, 40), (1280, 1280, 5), (640, 768, 300), (128, 256, 1)])
def test_prefill_axis0_fused_small(k, R, C, M):
    # R stored rows (the contraction, a multiple of 128), C outputs; M = 300 takes the 512-row x
    # tiles, the others the 128-row tiles; all split their few tiles along the stored rows
    rng = np.random.default_rng(R + C + M + 11 * k)
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, M, R)
    got = h_u16(tq.prefill_axis0(d_codes(codes), d_half(scales), d_bf16(x), k, algo=tq.PREFILL_FUSED))
    want, cond = oracle.prefill_axis0_sums(codes, scales, x, M, R, C, k, L, T, np.arange(M), np.arange(C), with_abs=True)
    tol.assert_bf16_close(got, want, cond, f"fused prefill axis0 R={R} C={C} M={M} k={k}")


@pytest.mark.parametrize("k", [3])
@pytest.mark.parametrize("C,M", [(25600, 300), (38400, 64)])
def test_prefill_axis0_fused_stream_pieces(k, C, M):
    # 200 (M = 300, 512-row tiles) or 300 (M = 64, 128-row tiles) output tiles leave more than half
    # of the workgroup slots busy after the full rounds, so the steps are dealt out in ranges that
    # cross tile boundaries and the fold adds the pieces of the tiles cut between ranges
    R = 640                                      # 20 steps per tile: ranges of 16 or 12 steps
    rng = np.random.default_rng(C + M)
    codes, scales = rand_matrix(rng, R, C, k)
    x = ti.activations(rng, M, R)
    got = tq.prefill_axis0(d_codes(codes), d_half(scales), d_bf16(x), k, algo=tq.PREFILL_FUSED)
    ms = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    cols = np.unique(np.concatenate([[0, 127, 128, C - 1], rng.integers(0, C, 120)]))
    want, cond = oracle.prefill_axis0_sums(codes, scales, x, M, R, C, k, L, T, ms, cols, with_abs=True)
    sub = h_u16(got[torch.as_tensor(ms, device=DEV)][:, torch.as_tensor(cols, device=DEV)])
    tol.assert_bf16_close(sub, want, cond, f"fused prefill axis0 stream C={C} M={M}")


@pytest.mark.parametrize("axis0,R,C,M,chosen", [
    (False, 512, 1024, 40, tq.PREFILL_FUSED), (False, 512, 1024, 200, tq.PREFILL_EXPAND_GEMM),
    (True, 384, 512, 40, tq.PREFILL_FUSED), (True, 300, 512, 40, tq.PREFILL_EXPAND_GEMM)])
def test_prefill_auto_matches_the_chosen_algo(axis0, R, C, M, chosen):
    # AUTO runs exactly one of the two algorithms: its output is bit-identical to that one's
    rng = np.random.default_rng(R + C + M + 5)
    k = 3
    codes, scales = rand_matrix(rng, R, C, k)
    x = d_bf16(ti.activations(rng, M, R if axis0 else C))
    fn = tq.prefill_axis0 if axis0 else tq.prefill
    want = h_u16(fn(d_codes(codes), d_half(scales), x, k, algo=chosen))   # picks the GEMM kernel first
    auto = h_u16(fn(d_codes(codes), d_half(scales), x, k, algo=tq.PREFILL_AUTO))
    np.testing.assert_array_equal(auto, want)


@pytest.mark.parametrize("axis0", [False, True])
def test_prefill_tune_then_calls(axis0):
    # the tune call times the GEMM candidates, writes the result, and later EXPAND_GEMM calls of the
    # shape run the pick: all three outputs meet the oracle, and the calls after tuning agree bit for bit
    rng = np.random.default_rng(77 + axis0)
    R, C, M, k = 640, 1024, 96, 2
    codes, scales = rand_matrix(rng, R, C, k)
    n_in = R if axis0 else C
    x = ti.activations(rng, M, n_in)
    fn = tq.prefill_axis0 if axis0 else tq.prefill
    args = (d_codes(codes), d_half(scales), d_bf16(x), k)
    a = h_u16(fn(*args, tune=True))
    b = h_u16(fn(*args, algo=tq.PREFILL_EXPAND_GEMM))
    c = h_u16(fn(*args, algo=tq.PREFILL_EXPAND_GEMM))
    if axis0:
        want, cond = oracle.prefill_axis0_sums(codes, scales, x, M, R, C, k, L, T, np.arange(M), np.arange(C),
                                               with_abs=True)
    else:
        want, cond = oracle.prefill_sums(codes, scales, x, M, R, C, k, L, T, np.arange(M), np.arange(R),
                                         with_abs=True)
    for got, what in ((a, "tune"), (b, "after tune"), (c, "again")):
        tol.assert_bf16_close(got, want, cond, f"prefill axis0={axis0} {what}")
    np.testing.assert_array_equal(b, c)


@pytest.mark.parametrize("algo,M", [(tq.PREFILL_EXPAND_GEMM, 32), (tq.PREFILL_EXPAND_GEMM, 512),
                                    (tq.PREFILL_FUSED, 32), (tq.PREFILL_FUSED, 512), (tq.PREFILL_FUSED, 2048)])
def test_prefill_axis0_down_17408x5120_k3(axis0_workload, algo, M):
    # the down projection of the MLP prefill: stored W^T 17408 x 5120, k = 3; x [M, 17408]
    w, _ = axis0_workload
    m = w.mats[0]
    rng = np.random.default_rng(M)
    x = ti.activations(rng, M, m.R)
    got = tq.prefill_axis0(d_codes(m.codes), d_half(m.scales), d_bf16(x), m.k, algo=algo)
    ms = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    cols = np.unique(np.concatenate([[0, 255, 256, m.C - 1], rng.integers(0, m.C, 60)]))
    want, cond = oracle.prefill_axis0_sums(m.codes, m.scales, x, M, m.R, m.C, m.k, L, T, ms, cols, with_abs=True)
    sub = h_u16(got[torch.as_tensor(ms, device=DEV)][:, torch.as_tensor(cols, device=DEV)])
    tol.assert_bf16_close(sub, want, cond, f"prefill axis0 down M={M}")


# ------------------------------------------------------------------ bf16-weight matvec contract (variants 0-3)

@pytest.mark.parametrize("algo", ALGOS)
def test_bf16_weight_matvec_17408x5120_k2_m1_to_4(prefill_workload, algo):
    # the pages' decode variants 0-3 round every weight to bf16 before the products (trellis-linear.ts file
    # header, HEADER TRELLIS_ROUND); trellis_prefill computes that contract for any M.  Every output of the
    # gate/up shape at M = 1..4 against the oracle's bf16-weight sums.
    w = prefill_workload
    m = w.mats[0]
    x = w.x[0][:4]
    want, cond = oracle.prefill_sums(m.codes, m.scales, x, 4, m.R, m.C, m.k, L, T, np.arange(4), np.arange(m.R),
                                     with_abs=True)
    dc, ds = d_codes(m.codes), d_half(m.scales)
    for M in (1, 2, 3, 4):
        got = h_u16(tq.prefill(dc, ds, d_bf16(x[:M]), m.k, algo=algo))
        tol.assert_bf16_close(got, want[:M], cond[:M], f"bf16-weight matvec algo={algo} M={M}")


@pytest.mark.parametrize("algo", ALGOS)
def test_bf16_weight_matvec_axis0_17408x5120_k3_m1_to_4(axis0_workload, algo):
    # the same contract for the down projection stored transposed (axis 0), every output
    w, _ = axis0_workload
    m = w.mats[0]
    x = w.x[0][:4]
    want, cond = oracle.prefill_axis0_sums(m.codes, m.scales, x, 4, m.R, m.C, m.k, L, T, np.arange(4),
                                           np.arange(m.C), with_abs=True)
    dc, ds = d_codes(m.codes), d_half(m.scales)
    for M in (1, 2, 3, 4):
        got = h_u16(tq.prefill_axis0(dc, ds, d_bf16(x[:M]), m.k, algo=algo))
        tol.assert_bf16_close(got, want[:M], cond[:M], f"bf16-weight axis0 matvec algo={algo} M={M}")
