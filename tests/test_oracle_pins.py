"""Pins of the CPU oracle against things other than itself (no GPU).

Each test checks the oracle against what the pages print (constants and the
alternative formulas they print for the same quantity), closed forms,
number-theoretic invariants, library routines (numpy, torch, scipy,
fractions) or brute force on tiny inputs.  Page abbreviations: TL = mlx-bun
0.2.0 -> 0.4.0 diff page 55, src/model/trellis-linear.ts; VE = page 56,
src/model/trellis-vector-expand.ts.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))
MUL = GOLD["onemad_multiplier"]["value"]
ADD = GOLD["onemad_addend"]["value"]
OFF = GOLD["onemad_offset"]["value"]
DIV = Fraction(GOLD["divisor"]["value"])      # float literal is exact: 605391 / 4096
L, T = GOLD["state_bits_L"]["value"], GOLD["block_T"]["value"]
KS = GOLD["bits_k"]["value"]


# ---------------------------------------------------------------- helpers

def rn_f32(q: Fraction) -> np.float32:
    """Binary32 nearest to the exact rational q, ties to even (brute search)."""
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def fma_f32(a, b, c) -> np.float32:
    """Exact fused multiply-add of binary32 values, one rounding."""
    return rn_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def torch_bf16_bits(v) -> np.ndarray:
    t = torch.as_tensor(np.asarray(v, dtype=np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def half_bits_to_f64(h) -> np.ndarray:
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def pack_symbols(syms, k):
    """Block words holding symbol t at bits [(T-1-t)*k, (T-t)*k), built with
    Python integers (an independent writer for the tail-biting window)."""
    bits = 0
    for t, s in enumerate(syms):
        bits |= int(s) << ((T - 1 - t) * k)
    wpb = T * k // 32
    return np.array([(bits >> (32 * i)) & 0xFFFFFFFF for i in range(wpb)], dtype=np.uint32)


def rand_bf16(rng, shape):
    return torch_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def rand_scales(rng, n):
    return rng.uniform(0.005, 0.02, n).astype(np.float16).view(np.uint16)


def dense_f32_weights(codes, scales, R, C, k):
    """W[r, c] = f32(value * f32(scale[r])) built with numpy float32 multiply."""
    _, _, vals = oracle.decode(codes, R, C, k, L, T)
    sc = half_bits_to_f64(scales).astype(np.float32)
    return (vals * sc[:, None]).astype(np.float32)


# ---------------------------------------------------------------- scalars

def test_half_to_double_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = half_bits_to_f64(bits)
    got = np.array([oracle.half_to_double(b) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_bf16_rounding_matches_torch_and_page_bit_trick():
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000))).astype(np.float32)
    # exact midpoints between adjacent bf16 values (ties must go to even)
    base = bf16_bits_to_f64(rand_bf16(rng, 5000)).astype(np.float32)
    half_ulp = np.ldexp(np.ones(5000, np.float32), (np.frexp(base)[1] - 9).astype(np.int32))
    ties = (base + half_ulp).astype(np.float32)
    vals = np.concatenate([a, ties, np.float32([0.0, -0.0, 1e-45, -1e-45, 3.0e38])])
    got = oracle.bf16_round_array(vals.astype(np.float64))
    assert np.array_equal(got, torch_bf16_bits(vals))
    # TL HEADER trellis_bf16: add 0x7FFF plus the lowest kept bit, clear the low half
    u = vals.view(np.uint32).astype(np.uint64)
    trick = ((u + GOLD["bf16_round_bias"]["value"] + ((u >> 16) & 1)) & 0xFFFF0000) >> 16
    finite = np.isfinite(vals) & (np.abs(vals) < 3.3e38)
    assert np.array_equal(got[finite], trick[finite].astype(np.uint16))


def test_divisor_is_unit_variance_of_four_uniform_bytes():
    # Closed form: a byte uniform on 0..255 has variance (256^2 - 1) / 12; four
    # independent bytes sum to variance 21845.  The printed divisor is its
    # square root rounded to binary32, so y / d has unit variance.
    assert np.float32(math.sqrt(4 * (256 ** 2 - 1) / 12)) == np.float32(float(DIV))
    assert DIV == Fraction(605391, 4096)


# ---------------------------------------------------------------- 1MAD code

def test_code_y_all_states():
    s = np.arange(1 << L, dtype=np.uint64)
    got = np.array([oracle.code_y(int(v)) for v in s], dtype=np.int64)
    # (1) the byte-pair form printed in TL HEADER trellis_y (uint32 arithmetic)
    x = ((s * MUL + ADD) & 0xFFFFFFFF).astype(np.uint32)
    mask = np.uint32(GOLD["byte_pair_mask"]["value"])
    p = (x & mask) + ((x >> np.uint32(8)) & mask)
    pair_form = (p & np.uint32(0xFFFF)).astype(np.int64) + (p >> np.uint32(16)).astype(np.int64) - OFF
    assert np.array_equal(got, pair_form)
    # (2) Python integers and the library byte split
    ints = [sum(((int(v) * MUL + ADD) % 2 ** 32).to_bytes(4, "little")) - OFF for v in s]
    assert np.array_equal(got, np.array(ints))
    # (3) invariants: range, digit sum in base 256 is congruent mod 255
    lo, hi = GOLD["y_range"]["value"]
    assert got.min() >= lo and got.max() <= hi
    assert np.array_equal((got + OFF) % 255, x.astype(np.int64) % 255)
    # (4) statistics: y / d is close to zero mean, unit variance over all states
    v = got / float(DIV)
    assert abs(v.mean()) < 0.05 and abs(v.var() - 1.0) < 0.05


def test_code_value_correctly_rounded():
    lo, hi = GOLD["y_range"]["value"]
    r = np.float32(1.0) / np.float32(float(DIV))
    d32 = np.float32(float(DIV))
    for y in range(lo, hi + 1):
        exact = rn_f32(Fraction(y) / DIV)
        got = oracle.code_value(y)
        assert got == exact, y
        # TL HEADER trellis_val_rcp: q = y*r, e = fma(-q, d, y), value = fma(e, r, q)
        q = np.float32(np.float32(y) * r)
        e = fma_f32(-q, d32, np.float32(y))
        assert fma_f32(e, r, q) == exact, y
        # unrefined y*(1/d) is within one ulp (TL HEADER, variant 6 note)
        ulps = abs(int(np.array(q, np.float32).view(np.int32)) - int(np.array(exact, np.float32).view(np.int32)))
        assert ulps <= 1, y


# ---------------------------------------------------------------- state

@pytest.mark.parametrize("k", KS)
def test_state_is_shift_register_of_symbols(k):
    """The window at bit (T-1-t)*k holds symbol t in its low k bits and the
    preceding symbols above, cyclically: s_t = sum_j sym[(t-j) mod T] 2^(jk)."""
    rng = np.random.default_rng(100 + k)
    assert L % k == 0
    for _ in range(3):
        syms = rng.integers(0, 1 << k, T)
        blk = pack_symbols(syms, k)
        for t in range(T):
            want = sum(int(syms[(t - j) % T]) << (j * k) for j in range(L // k))
            assert oracle.state(blk, k, L, T, t) == want, (k, t)


@pytest.mark.parametrize("k", KS)
def test_state_matches_page_word_form(k):
    """TL HEADER trellis_state: word wi = p >> 5, offset p & 31, spill into the
    next word (index wrapping to 0 at the block end), mask to L bits."""
    rng = np.random.default_rng(200 + k)
    wpb = T * k // 32
    for _ in range(4):
        blk = rng.integers(0, 2 ** 32, wpb, dtype=np.uint64)
        for t in range(T):
            p = (T - 1 - t) * k
            wi, off = p >> 5, p & 31
            win = int(blk[wi]) >> off
            if off + L > 32:
                win |= (int(blk[0 if wi + 1 == wpb else wi + 1]) << (32 - off)) & 0xFFFFFFFF
            win &= (1 << L) - 1
            assert oracle.state(blk.astype(np.uint32), k, L, T, t) == win


@pytest.mark.parametrize("k", KS)
def test_state_matches_page_four_weight_window(k):
    """VE: four adjacent weights from one 64-bit window starting at the last
    one's offset; weight i of the four sits (3-i)*k bits higher."""
    rng = np.random.default_rng(300 + k)
    wpb = T * k // 32
    blk = rng.integers(0, 2 ** 32, wpb, dtype=np.uint64)
    for t0 in range(0, T, 4):
        pos = (T - 1 - (t0 + 3)) * k
        wi, off = pos >> 5, pos & 31
        window = (int(blk[wi]) | (int(blk[0 if wi + 1 == wpb else wi + 1]) << 32)) >> off
        for i in range(4):
            s = (window >> ((3 - i) * k)) & ((1 << L) - 1)
            assert oracle.state(blk.astype(np.uint32), k, L, T, t0 + i) == s


def test_decode_addresses_rows_and_blocks():
    rng = np.random.default_rng(5)
    R, C, k = 3, 768, 3
    wpb = T * k // 32
    codes = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    st, ys, vals = oracle.decode(codes, R, C, k, L, T)
    for r in range(R):
        for c in range(0, C, 7):
            b = c // T
            blk = codes[r, b * wpb:(b + 1) * wpb]
            assert st[r, c] == oracle.state(blk, k, L, T, c % T)
            assert ys[r, c] == oracle.code_y(int(st[r, c]))
            assert vals[r, c] == oracle.code_value(int(ys[r, c]))


# ---------------------------------------------------------------- layers

CASES = [(1, 256, 1, 2), (5, 768, 3, 3), (8, 512, 4, 4), (3, 1024, 2, 2)]


@pytest.mark.parametrize("R,C,M,k", CASES)
def test_matvec_axis1_dense_and_metamorphic(R, C, M, k):
    rng = np.random.default_rng(R * 1000 + C + k)
    codes = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    sc = rand_scales(rng, R)
    x = rand_bf16(rng, (M, C))
    W = dense_f32_weights(codes, sc, R, C, k).astype(np.float64)
    got = oracle.matvec_axis1(codes, sc, x, M, R, C, k, L, T)
    want = bf16_bits_to_f64(x) @ W.T
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # one-hot input picks one weight exactly
    c = int(rng.integers(0, C))
    e = np.zeros((1, C), np.uint16)
    e[0, c] = torch_bf16_bits(1.0)
    assert np.array_equal(oracle.matvec_axis1(codes, sc, e, 1, R, C, k, L, T)[0], W[:, c])
    # doubling the scales doubles the outputs; negating x negates them
    sc2 = (half_bits_to_f64(sc) * 2).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.matvec_axis1(codes, sc2, x, M, R, C, k, L, T), 2 * got)
    assert np.array_equal(oracle.matvec_axis1(codes, sc, x ^ np.uint16(0x8000), M, R, C, k, L, T), -got)
    # row selection returns the same values
    rows = np.array([R - 1, 0])
    assert np.array_equal(oracle.matvec_axis1(codes, sc, x, M, R, C, k, L, T, rows=rows), got[:, rows])


@pytest.mark.parametrize("R,C,M,k", CASES)
def test_matvec_axis0_dense_and_metamorphic(R, C, M, k):
    rng = np.random.default_rng(R * 2000 + C + k)
    codes = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    sc = rand_scales(rng, R)
    x = rand_bf16(rng, (M, R))
    W = dense_f32_weights(codes, sc, R, C, k).astype(np.float64)   # stored W^T [R_in, C_out]
    got = oracle.matvec_axis0(codes, sc, x, M, R, C, k, L, T)
    np.testing.assert_allclose(got, bf16_bits_to_f64(x) @ W, rtol=1e-12, atol=1e-12)
    r = int(rng.integers(0, R))
    e = np.zeros((1, R), np.uint16)
    e[0, r] = torch_bf16_bits(1.0)
    assert np.array_equal(oracle.matvec_axis0(codes, sc, e, 1, R, C, k, L, T)[0], W[r, :])
    assert np.array_equal(oracle.matvec_axis0(codes, sc, x ^ np.uint16(0x8000), M, R, C, k, L, T), -got)
    cols = np.array([C - 1, 3, 0])
    assert np.array_equal(oracle.matvec_axis0(codes, sc, x, M, R, C, k, L, T, cols=cols), got[:, cols])


def _swiglu_reference(g, u):
    from scipy.special import expit
    gT = bf16_bits_to_f64(torch_bf16_bits(g))
    uT = bf16_bits_to_f64(torch_bf16_bits(u))
    sig = bf16_bits_to_f64(torch_bf16_bits(expit(gT)))
    silu = bf16_bits_to_f64(torch_bf16_bits(gT * sig))
    return torch_bf16_bits(silu * uT)


def test_swiglu_chain():
    rng = np.random.default_rng(11)
    g = np.concatenate([rng.standard_normal(3000) * 3, [0.0, -0.0, 40.0, -40.0, 1e-30]])
    u = np.concatenate([rng.standard_normal(3000) * 3, [1.0, 1.0, 2.0, 2.0, 1.0]])
    got = np.array([oracle.swiglu(a, b) for a, b in zip(g, u)], np.uint16)
    assert np.array_equal(got, _swiglu_reference(g, u))
    assert bf16_bits_to_f64(got[3000]) == 0.0          # silu(0) = 0


def test_gateup_is_swiglu_of_two_matvecs():
    rng = np.random.default_rng(12)
    R, C, M, k = 6, 512, 3, 2
    gc = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    uc = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    gs, us = rand_scales(rng, R), rand_scales(rng, R)
    x = rand_bf16(rng, (M, C))
    g, u, out = oracle.gateup_swiglu(gc, gs, uc, us, x, M, R, C, k, L, T)
    assert np.array_equal(g, oracle.matvec_axis1(gc, gs, x, M, R, C, k, L, T))
    assert np.array_equal(u, oracle.matvec_axis1(uc, us, x, M, R, C, k, L, T))
    assert np.array_equal(out, _swiglu_reference(g.ravel(), u.ravel()).reshape(M, R))


@pytest.mark.parametrize("k", KS)
def test_expand_is_bf16_of_f32_weight(k):
    rng = np.random.default_rng(20 + k)
    R, C = 4, 512
    codes = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    sc = rand_scales(rng, R)
    W = dense_f32_weights(codes, sc, R, C, k)
    got = oracle.expand_bf16(codes, sc, R, C, k, L, T)
    assert np.array_equal(got, torch_bf16_bits(W.astype(np.float64)))
    assert np.array_equal(oracle.expand_bf16(codes, sc, R, C, k, L, T, r0=2, nr=2), got[2:])


def test_prefill_dense():
    rng = np.random.default_rng(31)
    R, C, M, k = 7, 768, 9, 3
    codes = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    sc = rand_scales(rng, R)
    x = rand_bf16(rng, (M, C))
    Wb = bf16_bits_to_f64(oracle.expand_bf16(codes, sc, R, C, k, L, T))
    ms, rows = np.arange(M), np.arange(R)
    got = oracle.prefill_sums(codes, sc, x, M, R, C, k, L, T, ms, rows)
    np.testing.assert_allclose(got, bf16_bits_to_f64(x) @ Wb.T, rtol=1e-12, atol=1e-12)
    sub = oracle.prefill_sums(codes, sc, x, M, R, C, k, L, T, [M - 1, 2], [0, R - 1])
    assert np.array_equal(sub, got[np.ix_([M - 1, 2], [0, R - 1])])


@pytest.mark.parametrize("k", KS)
def test_prefill_axis0_dense_and_one_hot(k):
    # stored W^T [R, C]: sums over the stored rows of the expansion times x; a
    # one-hot x over stored rows picks one expansion row exactly
    rng = np.random.default_rng(41 + k)
    R, C, M = 37, 512, 5
    codes = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    sc = rand_scales(rng, R)
    x = rand_bf16(rng, (M, R))
    Wb = bf16_bits_to_f64(oracle.expand_bf16(codes, sc, R, C, k, L, T))     # [R, C]
    got = oracle.prefill_axis0_sums(codes, sc, x, M, R, C, k, L, T, np.arange(M), np.arange(C))
    np.testing.assert_allclose(got, bf16_bits_to_f64(x) @ Wb, rtol=1e-12, atol=1e-12)
    one = np.zeros((2, R), np.uint16)
    one[0, 3] = 0x3F80                                                      # bf16 1.0
    one[1, R - 1] = 0xBF80                                                  # bf16 -1.0
    e = oracle.prefill_axis0_sums(codes, sc, one, 2, R, C, k, L, T, [0, 1], np.arange(C))
    assert np.array_equal(e[0], Wb[3]) and np.array_equal(e[1], -Wb[R - 1])


# ---------------------------------------------------------------- sums of |term|
# The parity criterion measures rounding error against sum_c |w x|, which the
# oracle returns beside each sum.  Pinned to the dense product of the absolute
# weights and absolute activations, to the sum itself where no term cancels
# (one-hot x), to sign invariance and to the triangle inequality.

@pytest.mark.parametrize("R,C,M,k", CASES)
def test_abs_sums_axis1_and_axis0(R, C, M, k):
    rng = np.random.default_rng(R * 3000 + C + k)
    codes = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    sc = rand_scales(rng, R)
    W = np.abs(dense_f32_weights(codes, sc, R, C, k).astype(np.float64))
    x1 = rand_bf16(rng, (M, C))
    s1, a1 = oracle.matvec_axis1(codes, sc, x1, M, R, C, k, L, T, with_abs=True)
    np.testing.assert_allclose(a1, np.abs(bf16_bits_to_f64(x1)) @ W.T, rtol=1e-12, atol=0)
    assert np.all(a1 >= np.abs(s1))
    assert np.array_equal(oracle.matvec_axis1(codes, sc, x1 ^ np.uint16(0x8000), M, R, C, k, L, T,
                                              with_abs=True)[1], a1)
    x0 = rand_bf16(rng, (M, R))
    s0, a0 = oracle.matvec_axis0(codes, sc, x0, M, R, C, k, L, T, with_abs=True)
    np.testing.assert_allclose(a0, np.abs(bf16_bits_to_f64(x0)) @ W, rtol=1e-12, atol=0)
    assert np.all(a0 >= np.abs(s0))
    # one-hot: one term, nothing cancels
    c = int(rng.integers(0, C))
    e = np.zeros((1, C), np.uint16)
    e[0, c] = torch_bf16_bits(-1.0)
    s, a = oracle.matvec_axis1(codes, sc, e, 1, R, C, k, L, T, with_abs=True)
    assert np.array_equal(a, np.abs(s))


def test_abs_sums_gateup_and_prefill():
    rng = np.random.default_rng(13)
    R, C, M, k = 5, 512, 3, 3
    gc = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    uc = rng.integers(0, 2 ** 32, (R, C * k // 32), dtype=np.uint32)
    gs, us = rand_scales(rng, R), rand_scales(rng, R)
    x = rand_bf16(rng, (M, C))
    g, u, _, ga, ua = oracle.gateup_swiglu(gc, gs, uc, us, x, M, R, C, k, L, T, with_abs=True)
    assert np.array_equal(ga, oracle.matvec_axis1(gc, gs, x, M, R, C, k, L, T, with_abs=True)[1])
    assert np.array_equal(ua, oracle.matvec_axis1(uc, us, x, M, R, C, k, L, T, with_abs=True)[1])
    Wb = np.abs(bf16_bits_to_f64(oracle.expand_bf16(gc, gs, R, C, k, L, T)))
    s, a = oracle.prefill_sums(gc, gs, x, M, R, C, k, L, T, np.arange(M), np.arange(R), with_abs=True)
    np.testing.assert_allclose(a, np.abs(bf16_bits_to_f64(x)) @ Wb.T, rtol=1e-12, atol=0)
    assert np.all(a >= np.abs(s))
    # axis 0: stored [R, C] = gc, x over the stored rows
    xa = rand_bf16(rng, (M, R))
    s0, a0 = oracle.prefill_axis0_sums(gc, gs, xa, M, R, C, k, L, T, np.arange(M), np.arange(C), with_abs=True)
    np.testing.assert_allclose(a0, np.abs(bf16_bits_to_f64(xa)) @ Wb, rtol=1e-12, atol=0)
    assert np.all(a0 >= np.abs(s0))


def test_expansion_size_matches_page():
    # TL file header: the dense bf16 transient at the 5120 -> 17408 shape is ~178 MB
    assert round(17408 * 5120 * 2 / 1e6) == GOLD["expansion_megabytes_17408x5120"]["value"]
