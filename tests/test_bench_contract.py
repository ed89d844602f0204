"""Host-side checks of bench.py's contract that need no GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_is_tied_to_the_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench
    h = bench.kernel_source_hash()
    assert len(h) == 64
    rec = bench.committed_traffic("profiled")
    # either the committed counters match the current GEMM sources, or the bench reports no traffic
    import json
    with open(os.path.join(ROOT, "profiles", "signal_gemm_profiled_traffic.json")) as f:
        stored = json.load(f)
    if stored["kernel_source_sha256"] == h:
        assert rec == stored["hbm_bytes_per_launch"]
    else:
        assert rec is None
    assert bench.committed_traffic("no_such_workload") is None


def test_partition_cut_masks_index_the_searchs_predictions():
    """The MoE search check reads each partition's prediction at its cut mask (bit i: a group ends after wave
    i + 1), the order in which fo_plan_search and the oracle list their candidates."""
    sys.path.insert(0, ROOT)
    import bench
    from oracle import enumerate_compositions
    for T in (1, 2, 5, 9):
        comps = list(enumerate_compositions(T))
        assert len(comps) == 1 << (T - 1)
        for mask, comp in enumerate(comps):
            assert bench._cut_mask(comp) == mask
    assert bench._cut_mask((17,)) == 0 and bench._cut_mask((1,) * 17) == (1 << 16) - 1
    assert bench._cut_mask((8, 8, 1)) == (1 << 7) | (1 << 15)
