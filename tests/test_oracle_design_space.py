"""Pins for the wave-group partition design space and the wave arithmetic."""

import json
import os

import pytest

import oracle
from oracle.tiles import make_plan
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _brute_partitions(T):
    """All ordered tuples of positive ints summing to T (recursive definition)."""
    if T == 0:
        return [()]
    out = []
    for first in range(1, T + 1):
        out += [(first,) + rest for rest in _brute_partitions(T - first)]
    return out


@pytest.mark.parametrize("T", range(1, 11))
def test_design_space_size_and_members(T):
    comps = oracle.enumerate_compositions(T)
    assert len(comps) == 2 ** (T - 1)
    assert sorted(comps) == sorted(_brute_partitions(T))


def test_pages_T5_examples():
    g = _golden("design_space.json")
    for ex in g["examples"]:
        T = ex["T"]
        assert len(oracle.enumerate_compositions(T)) == ex["choices"]
        mask = 0
        for w in ex["communicate_after_waves"]:
            if w < T:                           # the last wave always communicates
                mask |= 1 << (w - 1)
        assert oracle.mask_to_composition(mask, T) == tuple(ex["partition"])
        assert oracle.composition_to_mask(tuple(ex["partition"])) == mask


def test_pages_tuning_example_candidates():
    g = _golden("design_space.json")["tuning_example"]
    assert len(oracle.enumerate_compositions(g["T"])) == g["candidates"]


def test_mask_round_trip():
    for T in range(1, 9):
        for mask in range(2 ** (T - 1)):
            comp = oracle.mask_to_composition(mask, T)
            assert sum(comp) == T and min(comp) >= 1
            assert oracle.composition_to_mask(comp) == mask


def test_pages_wave_arithmetic():
    """512 tiles over 128 processors is 4 waves; the tuning GEMM has 8 waves.

    The tile shape is not printed; 32768-element tiles (128 x 256) reproduce
    both figures.
    """
    g = _golden("wave_pattern.json")
    p = g["profiled_gemm"]
    plan = make_plan(p["M"], p["N"], BM=128, BN=256, S=1, W=p["sms"])
    assert plan.NT == p["tiles"] and plan.T == p["waves"]
    t = g["tuning_gemm"]
    plan = make_plan(t["M"], t["N"], BM=128, BN=256, S=1, W=t["sms"])
    assert plan.T == t["waves"]
    assert len(oracle.enumerate_compositions(plan.T)) == t["candidates"]
