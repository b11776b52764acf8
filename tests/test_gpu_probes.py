"""The measurement probes behind the bench's bound location, through the C ABI.

The register-only decode probe must decode what the oracle decodes: the
K + 1 words a thread holds are words 0 .. K of a block whose last run
(positions 224 .. 255) they fully determine, so the oracle's codes of those
positions, summed over a wave's lanes and passes, times 16 (the B columns),
are the wave's checksum, exactly.  The decode-free gate/up launch only has
to run (its outputs are meaningless by design).
"""
import numpy as np
import pytest
import torch

import oracle
import trellis_coded_quantized_amd as tq
import trellis_inputs as ti

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
L, T = 12, 256


@pytest.mark.parametrize("k", [2, 3, 4])
def test_decode_only_probe_checksum(k):
    rng = np.random.default_rng(70 + k)
    blocks, iters = 2, 3
    n = blocks * tq.PROBE_THREADS
    runs = rng.integers(0, 2 ** 32, (n, k + 1), dtype=np.uint32)
    got = tq.probe_decode_only(torch.from_numpy(runs.view(np.int32)).to(DEV), k, iters).cpu().numpy()
    wpb = T * k // 32
    want = np.zeros(n // 64)
    for t in range(iters):
        blk = np.zeros((n, wpb), np.uint32)
        blk[:, :k + 1] = runs + np.uint32(t)          # words 0 .. k hold the last run of the block
        _, ys, _ = oracle.decode(blk, n, T, k, L, T)
        want += 16.0 * ys[:, 224:].astype(np.float64).sum(axis=1).reshape(-1, 64).sum(axis=1)
    np.testing.assert_array_equal(got.astype(np.float64), want)


def test_gateup_decode_free_probe_runs():
    rng = np.random.default_rng(80)
    R, C, k, M = 512, 5120, 2, 4
    g = [torch.from_numpy(ti.codes(rng, R, C, k).view(np.int32)).to(DEV),
         torch.from_numpy(ti.scales(rng, R).view(np.int16)).to(DEV).view(torch.float16)]
    u = [torch.from_numpy(ti.codes(rng, R, C, k).view(np.int32)).to(DEV),
         torch.from_numpy(ti.scales(rng, R).view(np.int16)).to(DEV).view(torch.float16)]
    x = torch.from_numpy(ti.activations(rng, M, C).view(np.int16)).to(DEV).view(torch.bfloat16)
    out = tq.probe_gateup_decode_free(g[0], g[1], u[0], u[1], x, k)
    torch.cuda.synchronize()
    assert out.shape == (M, R)
    # rows wider than one launch are refused on the host
    wide = torch.zeros((R, 8192 * k // 32), dtype=torch.int32, device=DEV)
    with pytest.raises(tq.TrellisError):
        tq.probe_gateup_decode_free(wide, g[1], wide, u[1], torch.zeros((M, 8192), dtype=torch.bfloat16,
                                                                          device=DEV), k)
