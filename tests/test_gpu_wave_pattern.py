"""The wave premise on MI355X (deep-dive 三、Wave Group 划分设计空间 › wave 模式): with the
persistent grid of W workgroups, the tiles of one wave finish together, before
any tile of the next wave.

Statistical, so parity unpinned: device wall-clock stamps of every tile's
signal from fo_gemm_signal's trace, on the profiled shape (2048 x 8192 x 8192,
bf16, 512 tiles in 2 waves of 256) and on the prefill shape (4 waves).
"""

import numpy as np
import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("M,N,K", [(2048, 8192, 8192), (4096, 8192, 3584)])
def test_tiles_complete_in_waves(M, N, K):
    p = fo.Plan([M], N, K, "bf16", BM=256, BN=128, swizzle=4, wave_size=256)
    say(f"wave pattern M={M} N={N} K={K} T={p.T}")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    A = (torch.randn(M * K, device="cuda", generator=g) * 0.02).to(torch.bfloat16).view(torch.int16)
    B = (torch.randn(N * K, device="cuda", generator=g) * 0.02).to(torch.bfloat16).view(torch.int16)
    buf = torch.empty(M * N, dtype=torch.int16, device="cuda")
    sig = p.new_sig()
    trace = torch.zeros(2 * p.NT + p.P, dtype=torch.int64, device="cuda")
    for e in (1, 2):                         # the second, warm launch is the one measured
        trace.zero_()
        p.gemm_signal(A, B, buf, sig, e, trace=trace)
    torch.cuda.synchronize()
    t = trace.cpu().numpy().view(np.uint64)[0:2 * p.NT:2].astype(np.int64)
    t = (t - t.min()) * (1e3 / p.info["clock_khz"])          # microseconds
    waves = [t[w * p.W:(w + 1) * p.W] for w in range(p.T)]
    spans = [float(x.max() - x.min()) for x in waves]
    step = float(np.median(np.diff([np.median(x) for x in waves])))
    say("waves (first, median, last) us: " + "; ".join(f"{x.min():.1f} {np.median(x):.1f} {x.max():.1f}" for x in waves))
    assert step > 0
    for w in range(p.T - 1):
        assert waves[w].max() < waves[w + 1].min(), f"wave {w} overlaps wave {w + 1}"
    # each wave is a cluster: the first one tight; later ones widen, since the workgroups
    # never resynchronise and their timing differences accumulate from wave to wave
    assert spans[0] < 0.25 * step, (spans, step)
    assert max(spans) < 0.5 * step, (spans, step)


def test_waves_hold_with_the_polling_consumer_launched_first():
    """The persistent consumer (one workgroup per CU) is launched before the GEMM on another queue and
    polls until the GEMM signals: the GEMM's W workgroups must still all be resident at once, which shows
    in the signal stamps as the same wave clusters (a workgroup held back until the consumer left would
    finish its wave-0 tile after other workgroups' wave-1 tiles, or the consumer would time out)."""
    M, N, K = 2048, 8192, 8192
    p = fo.Plan([M], N, K, "bf16", BM=256, BN=128, swizzle=4, wave_size=256, composition=(1, 1))
    g = torch.Generator(device="cuda")
    g.manual_seed(8)
    A = (torch.randn(M * K, device="cuda", generator=g) * 0.02).to(torch.bfloat16).view(torch.int16)
    B = (torch.randn(N * K, device="cuda", generator=g) * 0.02).to(torch.bfloat16).view(torch.int16)
    peer = torch.zeros(M * N, dtype=torch.int16, device="cuda")
    buf = torch.empty(M * N, dtype=torch.int16, device="cuda")
    recv = torch.empty_like(buf)
    sig = p.new_sig()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    trace = torch.zeros(2 * p.NT + p.P, dtype=torch.int64, device="cuda")
    sa, sb = fo.stream_create(), fo.stream_create()
    torch.cuda.synchronize()
    for e in (1, 2):
        say(f"consumer first, then GEMM: epoch {e}")
        trace.zero_()
        p.consume_group(buf, peer, recv, sig, e, status, timeout_us=500000, stream=sb)
        p.gemm_signal(A, B, buf, sig, e, trace=trace, stream=sa)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, fo.status_string(int(status.item()))
    fo.stream_destroy(sa)
    fo.stream_destroy(sb)
    t = trace.cpu().numpy().view(np.uint64)[0:2 * p.NT:2].astype(np.int64)
    t = (t - t.min()) * (1e3 / p.info["clock_khz"])
    waves = [t[w * p.W:(w + 1) * p.W] for w in range(p.T)]
    say("waves (first, median, last) us: " + "; ".join(f"{x.min():.1f} {np.median(x):.1f} {x.max():.1f}" for x in waves))
    assert waves[0].max() < waves[1].min()
    step = float(np.median(waves[1]) - np.median(waves[0]))
    assert float(waves[0].max() - waves[0].min()) < 0.25 * step
