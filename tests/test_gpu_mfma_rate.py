"""The matrix-pipe rate probe (fo_mfma_rate), a measurement aid for the GEMM's
roofline: it must do exactly the MFMA work its FLOP count claims.

With ternary operands every product and partial sum is a small integer, so
fp32 holds the results exactly.  The sum of a wave's outputs is then fixed by
the operand layout of v_mfma_f32_16x16x32 alone (lane l feeds row or column
l mod 16 and K-quarter l div 16 of both operands), whatever the output layout:
summed over a 16x16x32 product, sum_ij (X Y)_ij = sum_k (sum_i X_ik)(sum_j Y_kj).
Each lane's own sum must also grow linearly with the number of rounds.
"""

import numpy as np
import pytest

from tests.gpu_util import say
from workloads import to_bits

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")

FRAG = 4        # A and B operands per set; two sets per lane
THREADS = 512   # eight waves per workgroup


def _expected_wave_sums(vals: np.ndarray, workgroups: int) -> np.ndarray:
    """vals: [n_vec, 8] operand values; the sum of each wave's outputs for one round."""
    n = len(vals)
    lanes = np.arange(workgroups * THREADS)
    out = np.zeros(workgroups * THREADS // 64)
    for wv in range(len(out)):
        ln = lanes[wv * 64:(wv + 1) * 64]
        tot = 0.0
        for u in range(2):
            for i in range(FRAG):
                a = vals[(ln * 16 + u * 8 + i) % n]                # [64 lanes, 8 values]
                for j in range(FRAG):
                    b = vals[(ln * 16 + u * 8 + FRAG + j) % n]
                    for q in range(4):                              # K = 8 * q + e
                        tot += float(np.dot(b[16 * q:16 * q + 16].sum(0), a[16 * q:16 * q + 16].sum(0)))
        out[wv] = tot
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_mfma_rate_does_the_work_it_counts(dtype):
    rng = np.random.Generator(np.random.PCG64(71))
    n_vec, workgroups = 1000, 2                       # 1024 lanes x 16 vectors wrap around 1000 vectors
    vals = rng.integers(-1, 2, size=(n_vec, 8)).astype(np.float32)
    ops = torch.from_numpy(to_bits(vals.reshape(-1), dtype).view(np.int16).copy()).cuda()
    outs = {}
    for iters in (1, 3):
        out = torch.full((workgroups * THREADS,), float("nan"), dtype=torch.float32, device="cuda")
        say(f"mfma_rate {dtype}: {workgroups} workgroups, {iters} rounds, {n_vec} operand vectors")
        fo.mfma_rate(ops, out, workgroups, iters, dtype=dtype)
        torch.cuda.synchronize()
        outs[iters] = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(outs[3], 3 * outs[1])
    waves = outs[1].reshape(-1, 64).sum(1)
    np.testing.assert_array_equal(waves, _expected_wave_sums(vals, workgroups))
    assert fo.mfma_rate_flops(workgroups, 3) == workgroups * 8 * 3 * 32 * 16384


def test_mfma_rate_with_no_rounds_writes_zeros():
    ops = torch.ones(64, dtype=torch.int16, device="cuda")
    out = torch.full((THREADS,), float("nan"), dtype=torch.float32, device="cuda")
    say("mfma_rate: zero rounds")
    fo.mfma_rate(ops, out, 1, 0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
