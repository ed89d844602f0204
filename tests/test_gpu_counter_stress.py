"""All CUs count into one counter: the counting table and the signal under contention from every XCD.

Deep-dive 一、信号机制 › 实现方法: 组级 Tile 计数 -- every finished tile
increments its group's entry of the counting table, and the group is signalled
when the entry reaches its tile count.  Here a plan has a single group of 64
waves: 16384 tiles of 64x64 with K = 64 finish in about a microsecond each, so
the 256 workgroups, dealt over the 8 XCDs, hit the one counter thousands of
times within tens of microseconds.  Per launch (epoch e) the counter values
the tiles saw (their tickets) must be exactly (e-1)*NT .. e*NT-1, each once;
the counter must end at e*NT, the flag at e, the group must fire once; and the
consumer, released by that one flag, must find every tile's stores (recv equals
the reordered output, peer being zero) and every slot's epoch stamp.
"""

import numpy as np
import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")

M = N = 8192
K = 64


@pytest.mark.parametrize("consumer", ["poll", "gated"])
def test_one_counter_hit_from_every_xcd(consumer):
    p = fo.Plan([M], N, K, "bf16", BM=64, BN=64, swizzle=2, epoch_stamps=True)
    try:
        if p.W * p.T != p.NT or p.T < 2:
            pytest.skip(f"needs whole waves; this device gives W = {p.W}")
        p.close()
        p = fo.Plan([M], N, K, "bf16", BM=64, BN=64, swizzle=2, composition=(p.T,), epoch_stamps=True)
        assert p.P == 1
        say(f"counter stress: {p.NT} tiles of 64x64 in one group, W={p.W}, consumer {consumer}")
        g = torch.Generator(device="cuda")
        g.manual_seed(23)
        A = (torch.randn(M * K, device="cuda", generator=g) * 0.1).to(torch.bfloat16).view(torch.int16)
        B = (torch.randn(N * K, device="cuda", generator=g) * 0.1).to(torch.bfloat16).view(torch.int16)
        peer = torch.zeros(M * N, dtype=torch.int16, device="cuda")
        buf = torch.empty(M * N, dtype=torch.int16, device="cuda")
        recv = torch.empty_like(buf)
        sig = p.new_sig()
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        trace = torch.zeros(2 * p.NT + p.P, dtype=torch.int64, device="cuda")
        sa, sb = fo.stream_create(), fo.stream_create()
        torch.cuda.synchronize()
        try:
            for e in (1, 2, 3):
                trace.zero_()
                recv.fill_(-1)
                torch.cuda.synchronize()
                if consumer == "poll":
                    p.consume_group(buf, peer, recv, sig, e, status, timeout_us=1000000, stream=sb)
                    p.gemm_signal(A, B, buf, sig, e, trace=trace, stream=sa)
                else:
                    p.gemm_signal(A, B, buf, sig, e, trace=trace, stream=sa)
                    p.consume_group_gated(buf, peer, recv, sig, e, status, stream=sb)
                torch.cuda.synchronize()
                assert int(status.item()) == 0, fo.status_string(int(status.item()))
                assert int(p.cnt_of(sig)[0].item()) == e * p.NT
                assert int(p.flag_of(sig)[0].item()) == e
                assert bool((p.stamps_of(sig) == e).all())
                tr = trace.cpu().numpy().view(np.uint64)
                tickets = np.sort((tr[1:2 * p.NT:2] & 0xFFFFFFFF).astype(np.int64))
                assert np.array_equal(tickets, np.arange((e - 1) * p.NT, e * p.NT))
                assert int(tr[2 * p.NT]) == 1                       # the group fired once
                workgroups = (tr[1:2 * p.NT:2] >> 32).astype(np.int64)
                assert len(np.unique(workgroups)) == p.W             # every workgroup counted tiles
                assert torch.equal(recv, buf)                        # every tile visible to the consumer
        finally:
            fo.stream_destroy(sa)
            fo.stream_destroy(sb)
    finally:
        p.close()
