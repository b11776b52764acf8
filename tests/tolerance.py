"""Parity criteria between the GPU library and the oracle.

f32 outputs: relative error with a floor,
    e_i = |g_i - o_i| / max(|o_i|, rms(o)) <= 1e-5,
where o is the oracle's exact (double) result and rms(o) is taken over the
outputs of the same call.  A pure elementwise relative error cannot be met
by any f32 accumulation near outputs that cancel to almost zero; the floor
measures those against the output scale instead.  The expected worst case
for f32 accumulation of a few thousand terms is about 1e-6.

bf16 outputs: the stored value must lie within one bf16 ulp of the bf16
rounding of some value inside the f32 band above, i.e. its ordered bit key
lies in [key(RN(o - d)) - 1, key(RN(o + d)) + 1] with d = 1e-5 max(|o|, rms).
"""
import numpy as np
import torch

REL = 1e-5


def rms(o: np.ndarray) -> float:
    o = np.asarray(o, np.float64)
    return float(np.sqrt(np.mean(o * o))) if o.size else 0.0


def f32_rel_error(got, want) -> np.ndarray:
    g = np.asarray(got, np.float64)
    o = np.asarray(want, np.float64)
    floor = np.maximum(np.abs(o), rms(o))
    err = np.abs(g - o)
    out = np.zeros_like(err)
    nz = floor > 0
    out[nz] = err[nz] / floor[nz]
    out[~nz] = np.where(err[~nz] == 0, 0.0, np.inf)
    return out


def bf16_bits_from_f64(v) -> np.ndarray:
    t = torch.as_tensor(np.asarray(v, np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_key(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_band_violations(got_bits, want, rel=REL) -> np.ndarray:
    """Boolean mask of bf16 outputs outside the band described above."""
    o = np.asarray(want, np.float64)
    d = rel * np.maximum(np.abs(o), rms(o))
    lo = bf16_key(bf16_bits_from_f64(o - d)) - 1
    hi = bf16_key(bf16_bits_from_f64(o + d)) + 1
    k = bf16_key(got_bits)
    return (k < lo) | (k > hi)


def assert_f32_close(got, want, what="", rel=REL):
    e = f32_rel_error(got, want)
    worst = float(e.max()) if e.size else 0.0
    assert worst <= rel, f"{what}: max floored relative error {worst:.3e} > {rel:.0e}"
    return worst


def assert_bf16_close(got_bits, want, what="", rel=REL):
    bad = bf16_band_violations(got_bits, want, rel)
    n = int(bad.sum())
    if n:
        idx = np.argwhere(bad)[:5]
        g = np.asarray(got_bits)
        raise AssertionError(f"{what}: {n} of {bad.size} bf16 outputs outside the band; first "
                             f"{[(tuple(i), float(bf16_to_f64(g[tuple(i)])), float(np.asarray(want)[tuple(i)])) for i in idx]}")


def swiglu_candidates(g, u, rel=REL, sig_rel=1e-6):
    """bf16 outputs of the SwiGLU cast chain over every rounding of the gate
    and up sums inside their f32 bands, and of the sigmoid within sig_rel
    (device expf vs double exp).  Returns (lo_key, hi_key) arrays."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    dg = rel * np.maximum(np.abs(g), rms(g))
    du = rel * np.maximum(np.abs(u), rms(u))
    keys = []
    for gg in (g - dg, g + dg):
        gT = bf16_to_f64(bf16_bits_from_f64(gg))
        s = 1.0 / (1.0 + np.exp(-gT))
        for ss in (s * (1 - sig_rel), s * (1 + sig_rel)):
            sig = bf16_to_f64(bf16_bits_from_f64(ss))
            silu = bf16_to_f64(bf16_bits_from_f64(gT * sig))
            for uu in (u - du, u + du):
                uT = bf16_to_f64(bf16_bits_from_f64(uu))
                keys.append(bf16_key(bf16_bits_from_f64(silu * uT)))
    keys = np.stack(keys)
    return keys.min(axis=0), keys.max(axis=0)


def assert_swiglu_close(got_bits, g, u, what=""):
    lo, hi = swiglu_candidates(g, u)
    k = bf16_key(got_bits)
    bad = (k < lo - 1) | (k > hi + 1)
    n = int(bad.sum())
    assert n == 0, f"{what}: {n} of {bad.size} SwiGLU outputs outside the candidate band"
