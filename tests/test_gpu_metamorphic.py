"""GPU metamorphic and stress parity, through the C ABI.

One-hot activations pin the decoders that feed each path bit for bit:
  * prefill (both axes, every kernel form): an x row that is +-1 at one
    column (axis 1) or one stored row (axis 0) and zero elsewhere has a single
    exact product, so the bf16 output row equals +-the oracle's bf16
    expansion weights exactly (mlx-bun 0.2.0 -> 0.4.0 diff, page 55, EXPAND
    kernel; page 56, trellis-tiled-prefill.ts: bf16 of the precise value
    times the scale).  Calls sweep the columns so that every block position,
    every wrap of the window and every tile form is hit.
  * matvecs: the f32 output is the weight itself up to the rounding of the
    fold of 1/d into the scale (the kernels compute y * RN(scale * RN(1/d))
    or RN(y * scale * RN(1/d)); the oracle RN(RN(y / d) * scale)): at most
    five roundings of 2^-24 apart, checked at 6 * 2^-24 relative.
Doubling the fp16 scales doubles every f32 and bf16 output bit for bit (a
power-of-two factor through exact operations).  Wide-range activations
(N(0, 1) * 2^U(-20, 20), +-1e4 outliers, an all-zero slice) with fp16 scales
at both ends of the range stress the kernels' own rescaling of x, against
the oracle under the criterion of tests/tolerance.py.
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
ONE, NEG_ONE = 0x3F80, 0xBF80          # bf16 +1.0 / -1.0
ONEHOT_REL = 6 * 2.0 ** -24


def d_codes(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(DEV)


def d_half(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.float16)


def d_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def h_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits):
    return tol.bf16_to_f64(bits)


def one_hot(n, idx, signs):
    """bf16 bits [len(idx), n]: row j is signs[j] at idx[j], zero elsewhere."""
    x = np.zeros((len(idx), n), np.uint16)
    x[np.arange(len(idx)), idx] = np.where(np.asarray(signs) > 0, ONE, NEG_ONE)
    return x


def signs_for(n, seed):
    return np.where(np.random.default_rng(seed).integers(0, 2, n) > 0, 1.0, -1.0)


def double_scales(s):
    d = (s.view(np.float16).astype(np.float64) * 2).astype(np.float16)
    assert np.all(np.isfinite(d))
    return d.view(np.uint16)


def report(what, got, want, cond):
    print(f"[parity] {what}: {tol.margin_report(got, want, cond)}", flush=True)


# ------------------------------------------------------------------ one-hot: prefill decoder bits

def column_sweeps(C, M):
    """Column sets of M columns each whose union is every column: consecutive
    windows (the last one wraps)."""
    return [(np.arange(M) + off) % C for off in range(0, C, M)]


SINGLE_COLUMNS = [0, 1, 2, 3, 4, 5, 31, 32, 127, 128, 255, 256, 257, 258, 259, 260, 383, 511]


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("M", [1, 32, 33, 64, 65, 128, 256, 300, 512])
def test_prefill_fused_one_hot_is_expansion(k, M):
    # M = 1 / 32 / 33 / 64: register-direct kernel (one or two x tiles); 65 / 128 / 256: 128-row x tiles;
    # 300 / 512: 512-row x tiles.  R = 1000 leaves ragged 32- and 128-row weight tiles.
    R, C = 1000, 512
    rng = np.random.default_rng(600 + 10 * k + M)
    codes, scales = ti.codes(rng, R, C, k), ti.scales(rng, R)
    Wb = f64(oracle.expand_bf16(codes, scales, R, C, k, L, T))            # [R, C]
    dc, ds = d_codes(codes), d_half(scales)
    sweeps = [np.array([c]) for c in SINGLE_COLUMNS] if M == 1 else column_sweeps(C, M)
    for j, cols in enumerate(sweeps):
        sg = signs_for(M, 1000 * k + j)
        got = f64(h_u16(tq.prefill(dc, ds, d_bf16(one_hot(C, cols, sg)), k, algo=tq.PREFILL_FUSED)))
        want = Wb[:, cols].T * sg[:, None]
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"k={k} M={M} sweep {j}: {len(bad)} outputs differ from the expansion, first "
                               f"(x row, weight row) {bad[0]}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}")


def test_prefill_expand_gemm_one_hot_is_expansion():
    R, C, k = 300, 768, 3
    rng = np.random.default_rng(650)
    codes, scales = ti.codes(rng, R, C, k), ti.scales(rng, R)
    Wb = f64(oracle.expand_bf16(codes, scales, R, C, k, L, T))
    cols = np.arange(C)
    sg = signs_for(C, 651)
    got = f64(h_u16(tq.prefill(d_codes(codes), d_half(scales), d_bf16(one_hot(C, cols, sg)), k,
                               algo=tq.PREFILL_EXPAND_GEMM)))
    np.testing.assert_array_equal(got, Wb.T * sg[:, None])


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("M", [1, 32, 128, 256, 300, 384])
def test_prefill_axis0_fused_one_hot_is_expansion(k, M):
    # stored W^T [384, 512]: x rows one-hot over the stored rows give expansion rows.  M <= 256 runs the
    # 128-row x tiles, above the 512-row tiles.
    R, C = 384, 512
    rng = np.random.default_rng(700 + 10 * k + M)
    codes, scales = ti.codes(rng, R, C, k), ti.scales(rng, R)
    Wb = f64(oracle.expand_bf16(codes, scales, R, C, k, L, T))            # [R_in, C_out]
    dc, ds = d_codes(codes), d_half(scales)
    sweeps = [np.array([r]) for r in (0, 1, 31, 32, 127, 128, 383)] if M == 1 else column_sweeps(R, M)
    for j, rows in enumerate(sweeps):
        sg = signs_for(M, 2000 * k + j)
        got = f64(h_u16(tq.prefill_axis0(dc, ds, d_bf16(one_hot(R, rows, sg)), k, algo=tq.PREFILL_FUSED)))
        want = Wb[rows, :] * sg[:, None]
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"k={k} M={M} sweep {j}: {len(bad)} outputs differ, first (x row, output) "
                               f"{bad[0]}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}")


@pytest.fixture(scope="module")
def prefill_expansion():
    w = ti.prefill(Ms=(1,))
    m = w.mats[0]
    return m, f64(oracle.expand_bf16(m.codes, m.scales, m.R, m.C, m.k, L, T))


@pytest.mark.parametrize("M", [32, 64, 512, 2048])
def test_prefill_one_hot_17408x5120_k2(prefill_expansion, M):
    # the prefill workload's matrix in the launch configurations the benchmark times: every output of
    # M one-hot rows at distinct columns (7m + 3 mod 5120 covers every block position)
    m, Wb = prefill_expansion
    cols = (7 * np.arange(M) + 3) % m.C
    sg = signs_for(M, M)
    got = f64(h_u16(tq.prefill(d_codes(m.codes), d_half(m.scales), d_bf16(one_hot(m.C, cols, sg)), m.k,
                               algo=tq.PREFILL_FUSED)))
    want = Wb[:, cols].T * sg[:, None]
    assert np.array_equal(got, want), f"M={M}: {int((got != want).sum())} outputs differ from the expansion"


@pytest.fixture(scope="module")
def down_expansion():
    m = ti.axis0().mats[0]
    return m, f64(oracle.expand_bf16(m.codes, m.scales, m.R, m.C, m.k, L, T))


@pytest.mark.parametrize("M", [32, 512, 2048])
def test_prefill_axis0_one_hot_17408x5120_k3(down_expansion, M):
    m, Wb = down_expansion
    rows = (7 * np.arange(M) + 5) % m.R
    sg = signs_for(M, M + 1)
    got = f64(h_u16(tq.prefill_axis0(d_codes(m.codes), d_half(m.scales), d_bf16(one_hot(m.R, rows, sg)), m.k,
                                     algo=tq.PREFILL_FUSED)))
    want = Wb[rows, :] * sg[:, None]
    assert np.array_equal(got, want), f"M={M}: {int((got != want).sum())} outputs differ from the expansion"


# ------------------------------------------------------------------ one-hot: matvec weights

def matvec_weights(codes, scales, R, C, k, axis):
    """The oracle's f32 weights, through its own one-hot sums (pinned to the
    dense weights on the CPU): [C, R] for axis 1, [R_in, C_out] for axis 0."""
    n = C if axis == 1 else R
    eye = one_hot(n, np.arange(n), np.ones(n))
    if axis == 1:
        return oracle.matvec_axis1(codes, scales, eye, n, R, C, k, L, T)
    return oracle.matvec_axis0(codes, scales, eye, n, R, C, k, L, T)


def assert_weight_close(got, want, what):
    rel = np.abs(got - want) / np.maximum(np.abs(want), np.finfo(np.float64).tiny)
    rel[(got == want)] = 0.0
    worst = float(rel.max())
    assert worst <= ONEHOT_REL, f"{what}: one-hot output {worst / 2.0 ** -24:.2f} x 2^-24 from the weight"


@pytest.mark.parametrize("k", [2, 3, 4])
def test_axis1_one_hot_is_weight(k):
    R, C = 100, 512
    rng = np.random.default_rng(800 + k)
    codes, scales = ti.codes(rng, R, C, k), ti.scales(rng, R)
    W = matvec_weights(codes, scales, R, C, k, 1)                          # [C, R]
    dc, ds = d_codes(codes), d_half(scales)
    for j, cols in enumerate(column_sweeps(C, 4)):
        sg = signs_for(4, 3000 * k + j)
        got = tq.matvec_axis1(dc, ds, d_bf16(one_hot(C, cols, sg)), k, out_dtype=torch.float32)
        assert_weight_close(got.cpu().numpy().astype(np.float64), W[cols] * sg[:, None], f"axis1 k={k} cols {cols}")


@pytest.mark.parametrize("k", [2, 4])
def test_gateup_one_hot_is_weight(k):
    R, C = 64, 512
    rng = np.random.default_rng(810 + k)
    g = (ti.codes(rng, R, C, k), ti.scales(rng, R))
    u = (ti.codes(rng, R, C, k), ti.scales(rng, R))
    Wg, Wu = matvec_weights(*g, R, C, k, 1), matvec_weights(*u, R, C, k, 1)
    args = (d_codes(g[0]), d_half(g[1]), d_codes(u[0]), d_half(u[1]))
    for j, cols in enumerate(column_sweeps(C, 4)):
        sg = signs_for(4, 4000 * k + j)
        x = one_hot(C, cols, sg)
        gf = torch.empty((4, R), dtype=torch.float32, device=DEV)
        uf = torch.empty((4, R), dtype=torch.float32, device=DEV)
        out = tq.gateup_swiglu(*args, d_bf16(x), k, gate_f32=gf, up_f32=uf)
        wg, wu = Wg[cols] * sg[:, None], Wu[cols] * sg[:, None]
        assert_weight_close(gf.cpu().numpy().astype(np.float64), wg, f"gate k={k}")
        assert_weight_close(uf.cpu().numpy().astype(np.float64), wu, f"up k={k}")
        tol.assert_swiglu_close(h_u16(out), wg, wu, np.abs(wg), np.abs(wu), f"gate/up one-hot k={k}")


@pytest.mark.parametrize("k", [2, 3, 4])
def test_axis0_one_hot_is_weight(k):
    R, C = 512, 768                                                        # stored W^T [R_in, C_out]
    rng = np.random.default_rng(820 + k)
    codes, scales = ti.codes(rng, R, C, k), ti.scales(rng, R)
    W = matvec_weights(codes, scales, R, C, k, 0)                          # [R_in, C_out]
    dc, ds = d_codes(codes), d_half(scales)
    for j, rows in enumerate(column_sweeps(R, 4)):
        sg = signs_for(4, 5000 * k + j)
        got = tq.matvec_axis0(dc, ds, d_bf16(one_hot(R, rows, sg)), k, out_dtype=torch.float32)
        assert_weight_close(got.cpu().numpy().astype(np.float64), W[rows] * sg[:, None], f"axis0 k={k} rows {rows}")


# ------------------------------------------------------------------ scales x 2: outputs x 2 exactly

def assert_doubled(a, b, what):
    a, b = a.cpu(), b.cpu()
    if a.dtype == torch.bfloat16:
        a, b = a.float(), b.float()
    assert torch.equal(b, 2 * a), f"{what}: {int((b != 2 * a).sum())} outputs are not exactly doubled"


def test_scale_doubling_axis1_and_gateup():
    w = ti.gateup()
    g, u = w.mats
    x = d_bf16(w.x[0])
    gc, uc = d_codes(g.codes), d_codes(u.codes)
    s1 = (d_half(g.scales), d_half(u.scales))
    s2 = (d_half(double_scales(g.scales)), d_half(double_scales(u.scales)))
    for M in (1, 4):
        for dt in (torch.float32, torch.bfloat16):
            a = tq.matvec_axis1(gc, s1[0], x[:M], g.k, out_dtype=dt)
            b = tq.matvec_axis1(gc, s2[0], x[:M], g.k, out_dtype=dt)
            assert_doubled(a, b, f"axis1 17408x5120 M={M} {dt}")
        f = [torch.empty((M, g.R), dtype=torch.float32, device=DEV) for _ in range(4)]
        tq.gateup_swiglu(gc, s1[0], uc, s1[1], x[:M], g.k, gate_f32=f[0], up_f32=f[1])
        tq.gateup_swiglu(gc, s2[0], uc, s2[1], x[:M], g.k, gate_f32=f[2], up_f32=f[3])
        assert_doubled(f[0], f[2], f"gate M={M}")
        assert_doubled(f[1], f[3], f"up M={M}")


def test_scale_doubling_axis0():
    w = ti.axis0()
    m = w.mats[0]
    dc, x = d_codes(m.codes), d_bf16(w.x[0])
    s1, s2 = d_half(m.scales), d_half(double_scales(m.scales))
    for M in (1, 4):
        for dt in (torch.float32, torch.bfloat16):
            assert_doubled(tq.matvec_axis0(dc, s1, x[:M], m.k, out_dtype=dt),
                           tq.matvec_axis0(dc, s2, x[:M], m.k, out_dtype=dt), f"axis0 M={M} {dt}")


@pytest.mark.parametrize("algo,M", [(tq.PREFILL_FUSED, 32), (tq.PREFILL_FUSED, 512), (tq.PREFILL_EXPAND_GEMM, 512)])
def test_scale_doubling_prefill(algo, M):
    w = ti.prefill(Ms=(M,))
    m = w.mats[0]
    dc, x = d_codes(m.codes), d_bf16(w.x[0])
    s1, s2 = d_half(m.scales), d_half(double_scales(m.scales))
    assert_doubled(tq.prefill(dc, s1, x, m.k, algo=algo), tq.prefill(dc, s2, x, m.k, algo=algo),
                   f"prefill algo={algo} M={M}")
    if algo == tq.PREFILL_FUSED and M == 32:
        assert_doubled(tq.expand_bf16(dc, s1, m.k), tq.expand_bf16(dc, s2, m.k), "expand")


@pytest.mark.parametrize("M", [64, 512])
def test_scale_doubling_prefill_axis0(M):
    m = ti.axis0().mats[0]
    x = d_bf16(ti.activations(np.random.default_rng(M), M, m.R))
    dc, s1, s2 = d_codes(m.codes), d_half(m.scales), d_half(double_scales(m.scales))
    assert_doubled(tq.prefill_axis0(dc, s1, x, m.k, algo=tq.PREFILL_FUSED),
                   tq.prefill_axis0(dc, s2, x, m.k, algo=tq.PREFILL_FUSED), f"prefill axis0 M={M}")


# ------------------------------------------------------------------ wide-range activations, extreme scales

def test_wide_range_axis1_512x2048_k2():
    rng = np.random.default_rng(900)
    R, C, k = 512, 2048, 2
    codes, scales = ti.codes(rng, R, C, k), ti.extreme_scales(rng, R)
    x = ti.wide_activations(rng, 4, C, zero=slice(256, 512))               # wave slice 1 of 8 all zero
    want, cond = oracle.matvec_axis1(codes, scales, x, 4, R, C, k, L, T, with_abs=True)
    dc, ds = d_codes(codes), d_half(scales)
    for M in (1, 4):
        got = tq.matvec_axis1(dc, ds, d_bf16(x[:M]), k, out_dtype=torch.float32).cpu().numpy()
        report(f"wide axis1 M={M}", got, want[:M], cond[:M])
        tol.assert_f32_close(got, want[:M], cond[:M], f"wide-range axis1 M={M}")
        tol.assert_bf16_close(h_u16(tq.matvec_axis1(dc, ds, d_bf16(x[:M]), k)), want[:M], cond[:M],
                              f"wide-range axis1 bf16 M={M}")


@pytest.fixture(scope="module")
def wide_gateup():
    rng = np.random.default_rng(901)
    R, C, k = 17408, 5120, 2
    g = ti.Matrix(1, R, C, k, ti.codes(rng, R, C, k), ti.extreme_scales(rng, R))
    u = ti.Matrix(1, R, C, k, ti.codes(rng, R, C, k), ti.extreme_scales(rng, R))
    x = ti.wide_activations(rng, 4, C, zero=slice(640, 1280))
    want = oracle.gateup_swiglu(g.codes, g.scales, u.codes, u.scales, x, 4, R, C, k, L, T, with_abs=True)
    return g, u, x, want


@pytest.mark.parametrize("M", [1, 4])
def test_wide_range_gateup_17408x5120_k2(wide_gateup, M):
    g, u, x, (og, ou, _, ga, ua) = wide_gateup
    gf = torch.empty((M, g.R), dtype=torch.float32, device=DEV)
    uf = torch.empty((M, g.R), dtype=torch.float32, device=DEV)
    out = tq.gateup_swiglu(d_codes(g.codes), d_half(g.scales), d_codes(u.codes), d_half(u.scales),
                           d_bf16(x[:M]), g.k, gate_f32=gf, up_f32=uf)
    report(f"wide gate M={M}", gf.cpu().numpy(), og[:M], ga[:M])
    tol.assert_f32_close(gf.cpu().numpy(), og[:M], ga[:M], f"wide-range gate M={M}")
    tol.assert_f32_close(uf.cpu().numpy(), ou[:M], ua[:M], f"wide-range up M={M}")
    tol.assert_swiglu_close(h_u16(out), og[:M], ou[:M], ga[:M], ua[:M], f"wide-range swiglu M={M}")


@pytest.fixture(scope="module")
def wide_axis0():
    rng = np.random.default_rng(902)
    R, C, k = 17408, 5120, 3
    m = ti.Matrix(0, R, C, k, ti.codes(rng, R, C, k), ti.extreme_scales(rng, R))
    x = ti.wide_activations(rng, 4, R, zero=slice(1472, 2944))             # one row split all zero
    return m, x, oracle.matvec_axis0(m.codes, m.scales, x, 4, R, C, k, L, T, with_abs=True)


@pytest.mark.parametrize("M", [1, 4])
def test_wide_range_axis0_17408x5120_k3(wide_axis0, M):
    m, x, (want, cond) = wide_axis0
    dc, ds = d_codes(m.codes), d_half(m.scales)
    got = tq.matvec_axis0(dc, ds, d_bf16(x[:M]), m.k, out_dtype=torch.float32).cpu().numpy()
    report(f"wide axis0 M={M}", got, want[:M], cond[:M])
    tol.assert_f32_close(got, want[:M], cond[:M], f"wide-range axis0 M={M}")
    tol.assert_bf16_close(h_u16(tq.matvec_axis0(dc, ds, d_bf16(x[:M]), m.k)), want[:M], cond[:M],
                          f"wide-range axis0 bf16 M={M}")


def test_wide_range_mlp():
    rng = np.random.default_rng(903)
    R, C, C_out, kg, kd = 2048, 5120, 1280, 2, 3
    g = (ti.codes(rng, R, C, kg), ti.extreme_scales(rng, R))
    u = (ti.codes(rng, R, C, kg), ti.extreme_scales(rng, R))
    d = (ti.codes(rng, R, C_out, kd), ti.extreme_scales(rng, R))
    x = ti.wide_activations(rng, 4, C, zero=slice(0, 640))
    hidden = torch.empty((4, R), dtype=torch.bfloat16, device=DEV)
    out = tq.mlp_decode(d_codes(g[0]), d_half(g[1]), d_codes(u[0]), d_half(u[1]), d_codes(d[0]), d_half(d[1]),
                        d_bf16(x), kg, kd, hidden=hidden)
    og, ou, _, ga, ua = oracle.gateup_swiglu(*g, *u, x, 4, R, C, kg, L, T, with_abs=True)
    h = h_u16(hidden)
    tol.assert_swiglu_close(h, og, ou, ga, ua, "wide-range mlp hidden")
    want, cond = oracle.matvec_axis0(*d, h, 4, R, C_out, kd, L, T, with_abs=True)
    tol.assert_bf16_close(h_u16(out), want, cond, "wide-range mlp out")


@pytest.mark.parametrize("algo", [tq.PREFILL_FUSED, tq.PREFILL_EXPAND_GEMM])
@pytest.mark.parametrize("M", [32, 200, 600])
def test_wide_range_prefill(algo, M):
    rng = np.random.default_rng(904 + M)
    R, C, k = 1000, 1280, 3
    codes, scales = ti.codes(rng, R, C, k), ti.extreme_scales(rng, R)
    x = ti.wide_activations(rng, M, C, zero=slice(256, 512))
    got = h_u16(tq.prefill(d_codes(codes), d_half(scales), d_bf16(x), k, algo=algo))
    want, cond = oracle.prefill_sums(codes, scales, x, M, R, C, k, L, T, np.arange(M), np.arange(R), with_abs=True)
    tol.assert_bf16_close(got, want, cond, f"wide-range prefill algo={algo} M={M}")


@pytest.mark.parametrize("algo", [tq.PREFILL_FUSED, tq.PREFILL_EXPAND_GEMM])
@pytest.mark.parametrize("M", [40, 300])
def test_wide_range_prefill_axis0(algo, M):
    rng = np.random.default_rng(905 + M)
    R, C, k = 640, 768, 2
    codes, scales = ti.codes(rng, R, C, k), ti.extreme_scales(rng, R)
    x = ti.wide_activations(rng, M, R, zero=slice(128, 256))
    got = h_u16(tq.prefill_axis0(d_codes(codes), d_half(scales), d_bf16(x), k, algo=algo))
    want, cond = oracle.prefill_axis0_sums(codes, scales, x, M, R, C, k, L, T, np.arange(M), np.arange(C),
                                           with_abs=True)
    tol.assert_bf16_close(got, want, cond, f"wide-range prefill axis0 algo={algo} M={M}")


@pytest.mark.parametrize("M", [32, 2048])
def test_wide_range_prefill_17408x5120_k2(M):
    rng = np.random.default_rng(906 + M)
    w = ti.prefill(Ms=(1,))
    m = w.mats[0]
    scales = ti.extreme_scales(rng, m.R)
    x = ti.wide_activations(rng, M, m.C, zero=slice(1024, 2048))
    got = tq.prefill(d_codes(m.codes), d_half(scales), d_bf16(x), m.k, algo=tq.PREFILL_FUSED)
    ms = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    rows = np.unique(np.concatenate([[0, 7, 14, m.R - 1], rng.integers(0, m.R, 60)]))
    want, cond = oracle.prefill_sums(m.codes, scales, x, M, m.R, m.C, m.k, L, T, ms, rows, with_abs=True)
    sub = h_u16(got[torch.as_tensor(ms, device=DEV)][:, torch.as_tensor(rows, device=DEV)])
    tol.assert_bf16_close(sub, want, cond, f"wide-range prefill 17408x5120 M={M}")
