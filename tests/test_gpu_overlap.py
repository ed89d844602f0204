"""The consumer runs beside the GEMM: device timestamps show causality and overlap.

Both kernels stamp the device wall clock: the GEMM when each tile signals,
the consumer when its wait for a group ends (the polling consumer) or when
the group's kernel starts behind its stream wait (the gated consumer).
Causality (a group is consumed only after its last tile signalled) must hold
for every group; overlap (the first group is consumed while the GEMM still
computes the last group) shows that the two streams really run at the same
time.
"""

import numpy as np
import pytest

from oracle.tiles import make_plan
from tests.gpu_util import say, to_dev
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

fo = pytest.importorskip("gemm_tile_signaling_amd")
torch = pytest.importorskip("torch")
from gemm_tile_signaling_amd.pipeline import Pipeline  # noqa: E402


@pytest.mark.parametrize("name,comp", [("profiled", (1, 1)), ("ar_prefill", (1, 1, 1, 1)), ("rs", (2, 2))])
@pytest.mark.parametrize("consumer", ["gated", "poll"])
def test_consumer_overlaps_gemm(name, comp, consumer):
    w = WORKLOADS[name]
    A, B, peer, m_per, row_dest = make_inputs(w)
    o = make_plan(m_per, w.N, BM=w.BM, BN=w.BN, S=w.S, W=w.W, composition=comp, mode=w.mode, ranks=w.ranks)
    p = fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W, composition=comp,
                mode=w.mode, ranks=w.ranks)
    say(f"overlap {name} {comp} consumer={consumer}")
    pipe = Pipeline(p, to_dev(A), to_dev(B[0]), to_dev(peer), consumer=consumer)
    gtrace = torch.zeros(2 * p.NT + p.P, dtype=torch.int64, device="cuda")
    ctrace = torch.zeros(p.P, dtype=torch.int64, device="cuda")
    pipe.step()                                     # warm-up pass
    pipe.step(trace=gtrace, consumer_trace=ctrace)
    pipe.join()
    torch.cuda.synchronize()
    pipe.close()
    assert int(pipe.status.item()) == 0
    g = gtrace.cpu().numpy().view(np.uint64).astype(np.int64)
    c = ctrace.cpu().numpy().view(np.uint64).astype(np.int64)
    t_sig = g[0:2 * p.NT:2]
    grp = np.array(o.group_of_b)
    last = np.array([t_sig[grp == j].max() for j in range(p.P)])
    first = np.array([t_sig[grp == j].min() for j in range(p.P)])
    assert np.all(c >= last), (c - last).tolist()            # never before the group's last tile
    assert c[0] < last[-1], (c[0], last[-1])                 # group 0 consumed while the GEMM still runs
    assert fo.Plan is not None and first[-1] <= last[-1]
