"""Seeded synthetic inputs for the packed trellis-coded linear layer.

Shared by the tests, the benchmark and the oracle checks.  This module holds
none of the layer's arithmetic: it only draws random bits and values and
hands them over as numpy arrays (uint32 code words, fp16 scale bits, bf16
activation bits).

Recipe (the pages publish no dataset; everything is synthetic):
  codes  = uniform random uint32 words, numpy PCG64 ``default_rng(seed)``
  scales = uniform [0.005, 0.02] drawn in float64, cast to float16
  x      = standard normal float32, rounded to bfloat16 (nearest even)
Draws happen in the order the workload lists them, from one generator per
workload.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

L_BITS = 12      # state bits
BLOCK_T = 256    # symbols per block


def codes(rng: np.random.Generator, rows: int, cols: int, k: int) -> np.ndarray:
    """uint32 [rows, cols*k/32] uniform random code words."""
    words = cols * k // 32
    return rng.integers(0, 2 ** 32, size=(rows, words), dtype=np.uint32)


def scales(rng: np.random.Generator, rows: int) -> np.ndarray:
    """fp16 bits [rows], values uniform in [0.005, 0.02]."""
    return rng.uniform(0.005, 0.02, rows).astype(np.float16).view(np.uint16)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even) and return the bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(rng: np.random.Generator, M: int, n: int) -> np.ndarray:
    """bf16 bits [M, n] of N(0, 1) draws."""
    return to_bf16_bits(rng.standard_normal((M, n), dtype=np.float32))


def wide_activations(rng: np.random.Generator, M: int, n: int, zero: slice = None,
                     outliers: int = 3) -> np.ndarray:
    """bf16 bits [M, n] spread over a wide range: N(0, 1) * 2^U(-20, 20) per
    element, `outliers` entries per row at +-1e4, and the columns in `zero`
    (a slice) all zero."""
    v = rng.standard_normal((M, n)) * np.exp2(rng.uniform(-20.0, 20.0, (M, n)))
    for m in range(M):
        idx = rng.choice(n, size=min(outliers, n), replace=False)
        v[m, idx] = rng.choice([-1e4, 1e4], size=idx.size)
    if zero is not None:
        v[:, zero] = 0.0
    return to_bf16_bits(v.astype(np.float32))


def extreme_scales(rng: np.random.Generator, rows: int) -> np.ndarray:
    """fp16 bits [rows]: mostly U[0.005, 0.02], with every 7th row at one of
    the fp16 extremes in turn -- the smallest normal 2^-14, a subnormal 2^-20,
    the largest finite 65504, 1000 -- each but 65504 multiplied by 1 or 1.5
    at random."""
    s = rng.uniform(0.005, 0.02, rows)
    ends = [2.0 ** -14, 2.0 ** -20, 65504.0, 1000.0]
    for j, r in enumerate(range(0, rows, 7)):
        e = ends[j % len(ends)]
        s[r] = e * (1.5 if (e < 60000.0 and rng.integers(0, 2)) else 1.0)
    return s.astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Matrix:
    """One packed matrix: stored [R, C] coded along C."""
    axis: int
    R: int
    C: int
    k: int
    codes: np.ndarray
    scales: np.ndarray
    L: int = L_BITS
    T: int = BLOCK_T


@dataclass
class Workload:
    name: str
    seed: int
    mats: List[Matrix]
    x: List[np.ndarray] = field(default_factory=list)   # bf16 bits, one per matrix or shared
    Ms: Tuple[int, ...] = (1,)
    notes: str = ""


def axis1_m1(seed: int = 1001) -> Workload:
    """Axis-1 matvec, M = 1: R = 512, C = 2048, k = 2."""
    rng = np.random.default_rng(seed)
    m = Matrix(1, 512, 2048, 2, codes(rng, 512, 2048, 2), scales(rng, 512))
    return Workload("axis1_512x2048_k2_m1", seed, [m], [activations(rng, 1, 2048)], (1,))


def gateup(seed: int = 1002, R: int = 17408, C: int = 5120, k: int = 2) -> Workload:
    """Fused gate/up + SwiGLU: two R x C matrices, x bf16 [4, C]."""
    rng = np.random.default_rng(seed)
    g = Matrix(1, R, C, k, codes(rng, R, C, k), scales(rng, R))
    u = Matrix(1, R, C, k, codes(rng, R, C, k), scales(rng, R))
    x = activations(rng, 4, C)
    return Workload(f"gateup_{R}x{C}_k{k}", seed, [g, u], [x], (1, 2, 3, 4))


def axis0(seed: int = 1003, R_in: int = 17408, C_out: int = 5120, k: int = 3) -> Workload:
    """Axis-0 scatter: stored W^T [R_in, C_out] coded along C_out, x [4, R_in]."""
    rng = np.random.default_rng(seed)
    m = Matrix(0, R_in, C_out, k, codes(rng, R_in, C_out, k), scales(rng, R_in))
    x = activations(rng, 4, R_in)
    return Workload(f"axis0_{R_in}x{C_out}_k{k}", seed, [m], [x], (1, 2, 3, 4))


def layer_chain(seed: int = 1004, k: int = 4) -> Workload:
    """One decoder layer's projection set at M = 4: axis-1 10240x5120,
    6144x5120, 64x5120 and axis-0 W [5120 out, 6144 in] stored [6144, 5120]."""
    rng = np.random.default_rng(seed)
    mats, xs = [], []
    for (R, C) in ((10240, 5120), (6144, 5120), (64, 5120)):
        mats.append(Matrix(1, R, C, k, codes(rng, R, C, k), scales(rng, R)))
        xs.append(activations(rng, 4, C))
    mats.append(Matrix(0, 6144, 5120, k, codes(rng, 6144, 5120, k), scales(rng, 6144)))
    xs.append(activations(rng, 4, 6144))
    return Workload(f"layer_chain_k{k}_m4", seed, mats, xs, (4,))


def prefill(seed: int = 1005, R: int = 17408, C: int = 5120, k: int = 2,
            Ms: Tuple[int, ...] = (32, 512, 2048)) -> Workload:
    """Axis-1 prefill: R x C matrix, x bf16 [max(Ms), C]."""
    rng = np.random.default_rng(seed)
    m = Matrix(1, R, C, k, codes(rng, R, C, k), scales(rng, R))
    x = activations(rng, max(Ms), C)
    return Workload(f"prefill_{R}x{C}_k{k}", seed, [m], [x], tuple(Ms))


WORKLOADS: Dict[str, object] = {
    "axis1_m1": axis1_m1,
    "gateup": gateup,
    "axis0": axis0,
    "layer_chain": layer_chain,
    "prefill": prefill,
}
