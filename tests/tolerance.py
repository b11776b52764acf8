"""Parity criteria between the GPU library and the oracle.

f32 outputs: relative error with a per-output floor,
    e_i = |g_i - o_i| / max(|o_i|, COND * a_i) <= REL = 1e-5,
where o_i is the oracle's exact (double) sum and a_i = sum_c |w x| is the
sum of the absolute values of its terms (the oracle returns it beside the
sum).  A bare relative error cannot be met by any f32 accumulation when the
terms cancel to almost zero: each rounding contributes up to 2^-24 of the
running magnitude, which is set by the terms, not by the result.  The floor
therefore measures such outputs against their own terms: with COND = 2^-6
the error allowed near cancellation is 1e-5 / 64 * a_i, about 2.6 units of
f32 roundoff (2^-24 a_i).  For scale: on the same inputs, f32 sums taken in
the order of the pages' REDUCE kernel (per-lane partial sums, then a
SIMD-group tree) lose up to 1.2 such units and a plain sequential f32 sum
up to 10.3, so the bound admits a well-ordered f32 reduction and rejects a
careless one.  (For N(0, 1) activations over 5120 inputs, a_i is about 45
times the typical |o_i|, so the floor sits near 0.7 times the rms output;
for a sum dominated by one large term it equals |o_i|.)

bf16 outputs: the stored value must lie within one bf16 ulp of the bf16
rounding of some value inside the f32 band above, i.e. its ordered bit key
lies in [key(RN(o - d)) - 1, key(RN(o + d)) + 1] with d = REL * floor_i.
"""
import numpy as np
import torch

REL = 1e-5
COND = 2.0 ** -6


def floor_of(want, cond) -> np.ndarray:
    """Per-output floor max(|o|, COND * sum|term|)."""
    o = np.asarray(want, np.float64)
    a = np.asarray(cond, np.float64)
    if a.shape != o.shape:
        raise ValueError(f"sum of |term| has shape {a.shape}, the outputs {o.shape}")
    return np.maximum(np.abs(o), COND * a)


def f32_rel_error(got, want, cond) -> np.ndarray:
    g = np.asarray(got, np.float64)
    o = np.asarray(want, np.float64)
    floor = floor_of(o, cond)
    err = np.abs(g - o)
    out = np.zeros_like(err)
    nz = floor > 0
    out[nz] = err[nz] / floor[nz]
    out[~nz] = np.where(err[~nz] == 0, 0.0, np.inf)
    return out


def roundoff_units(got, want, cond) -> float:
    """Largest |g - o| over the outputs in units of 2^-24 * sum|term| (a
    diagnostic: how many f32 roundings of its own terms an output lost)."""
    g = np.asarray(got, np.float64)
    o = np.asarray(want, np.float64)
    a = np.asarray(cond, np.float64)
    err = np.abs(g - o)
    nz = a > 0
    return float((err[nz] / (a[nz] * 2.0 ** -24)).max()) if nz.any() else 0.0


def bf16_bits_from_f64(v) -> np.ndarray:
    t = torch.as_tensor(np.asarray(v, np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_key(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_band_violations(got_bits, want, cond, rel=REL) -> np.ndarray:
    """Boolean mask of bf16 outputs outside the band described above."""
    o = np.asarray(want, np.float64)
    d = rel * floor_of(o, cond)
    lo = bf16_key(bf16_bits_from_f64(o - d)) - 1
    hi = bf16_key(bf16_bits_from_f64(o + d)) + 1
    k = bf16_key(got_bits)
    return (k < lo) | (k > hi)


def margin_report(got, want, cond) -> str:
    """Worst floored relative error and worst error in roundings of sum|term|."""
    e = f32_rel_error(got, want, cond)
    worst = float(e.max()) if e.size else 0.0
    return f"floored rel {worst:.2e} ({worst / REL:.3f} of the bound), {roundoff_units(got, want, cond):.2f} roundings"


def assert_f32_close(got, want, cond, what="", rel=REL):
    e = f32_rel_error(got, want, cond)
    worst = float(e.max()) if e.size else 0.0
    assert worst <= rel, (f"{what}: max floored relative error {worst:.3e} > {rel:.0e} "
                          f"({roundoff_units(got, want, cond):.2f} roundings of sum|term|)")
    return worst


def assert_bf16_close(got_bits, want, cond, what="", rel=REL):
    bad = bf16_band_violations(got_bits, want, cond, rel)
    n = int(bad.sum())
    if n:
        idx = np.argwhere(bad)[:5]
        g = np.asarray(got_bits)
        raise AssertionError(f"{what}: {n} of {bad.size} bf16 outputs outside the band; first "
                             f"{[(tuple(i), float(bf16_to_f64(g[tuple(i)])), float(np.asarray(want)[tuple(i)])) for i in idx]}")


def swiglu_candidates(g, u, gcond, ucond, rel=REL, sig_rel=1e-6):
    """bf16 outputs of the SwiGLU cast chain over every rounding of the gate
    and up sums inside their f32 bands, and of the sigmoid within sig_rel
    (device expf vs double exp).  Returns (lo_key, hi_key) arrays."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    dg = rel * floor_of(g, gcond)
    du = rel * floor_of(u, ucond)
    keys = []
    for gg in (g - dg, g + dg):
        gT = bf16_to_f64(bf16_bits_from_f64(gg))
        with np.errstate(over="ignore"):
            s = 1.0 / (1.0 + np.exp(-gT))
        for ss in (s * (1 - sig_rel), s * (1 + sig_rel)):
            sig = bf16_to_f64(bf16_bits_from_f64(ss))
            silu = bf16_to_f64(bf16_bits_from_f64(gT * sig))
            for uu in (u - du, u + du):
                uT = bf16_to_f64(bf16_bits_from_f64(uu))
                keys.append(bf16_key(bf16_bits_from_f64(silu * uT)))
    keys = np.stack(keys)
    return keys.min(axis=0), keys.max(axis=0)


def assert_swiglu_close(got_bits, g, u, gcond, ucond, what=""):
    lo, hi = swiglu_candidates(g, u, gcond, ucond)
    k = bf16_key(got_bits)
    bad = (k < lo - 1) | (k > hi + 1)
    n = int(bad.sum())
    assert n == 0, f"{what}: {n} of {bad.size} SwiGLU outputs outside the candidate band"
