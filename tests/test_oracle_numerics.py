"""Pins for the oracle's rounding, GEMM and consumer add.

Pins: hand-computed bit patterns, exact rational rounding (fractions), the
library conversions of torch and numpy as an independent route, a
pure-Python triple-loop product under Higham's error bound, closed forms
(identity, ternary inputs, all-ones), and non-square shapes that catch a
transposed operand.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.numerics import round_to_dtype, decode_bits, encode_bits, gemm_fp64, consume_add


# --------------------------------------------------------------------------- rounding

@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just past the tie
    (3.0e38, 0x7F62),
    (3.4e38, 0x7F80),                           # rounds past the largest finite -> inf
    (2.0 ** -126, 0x0080),                      # smallest normal
    (2.0 ** -133, 0x0001),                      # smallest subnormal
    (2.0 ** -134, 0x0000),                      # half of it: tie -> even (zero)
    (3 * 2.0 ** -135, 0x0001),
    (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
])
def test_bf16_rounding_hand_values(x, bits):
    assert int(encode_bits(round_to_dtype(np.array([x]), "bf16"), "bf16")[0]) == bits


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3C00), (65504.0, 0x7BFF), (65520.0, 0x7C00), (65519.99, 0x7BFF),
    (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02),
])
def test_fp16_rounding_hand_values(x, bits):
    assert int(encode_bits(round_to_dtype(np.array([x]), "fp16"), "fp16")[0]) == bits


def test_nan_passes_through():
    y = round_to_dtype(np.array([np.nan]), "bf16")
    assert np.isnan(y[0])


def _exact_round(x: float, p: int, emin: int, emax: int) -> float:
    """Round-to-nearest-even with exact rational arithmetic (brute force)."""
    if x == 0 or not math.isfinite(x):
        return x
    q = Fraction(x)
    a = abs(q)
    e = max(math.frexp(abs(x))[1] - 1, emin)     # a in [2^e, 2^(e+1)), or subnormal (e = emin)
    assert a < Fraction(2) ** (e + 1) and (e == emin or Fraction(2) ** e <= a)
    ulp = Fraction(2) ** (e - p + 1)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    y = fl * ulp
    if y > (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax:
        return math.copysign(math.inf, x)
    return math.copysign(float(y), x)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_rounding_matches_exact_rational_rounding(dtype):
    d = oracle.DTYPES[dtype]
    rng = np.random.Generator(np.random.PCG64(5))
    lo = d["emin"] - d["p"] - 2
    x = rng.standard_normal(3000) * np.exp2(rng.integers(lo, d["emax"] + 2, size=3000))
    # values exactly on and next to rounding ties
    ties = (1 + (2 * rng.integers(0, 2 ** (d["p"] - 1), size=200) + 1) * 2.0 ** -d["p"]) \
        * np.exp2(rng.integers(-10, 10, size=200))
    x = np.concatenate([x, ties, np.nextafter(ties, 0), np.nextafter(ties, np.inf)])
    got = round_to_dtype(x, dtype)
    want = np.array([_exact_round(float(v), d["p"], d["emin"], d["emax"]) for v in x])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype,td", [("bf16", torch.bfloat16), ("fp16", torch.float16)])
def test_rounding_matches_library_conversion_from_fp32(dtype, td):
    rng = np.random.Generator(np.random.PCG64(6))
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, size=20000))).astype(np.float32)
    lib = torch.from_numpy(x).to(td).view(torch.int16).numpy().view(np.uint16)
    mine = encode_bits(round_to_dtype(x.astype(np.float64), dtype), dtype)
    assert np.array_equal(lib, mine)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_decode_encode_round_trip_all_finite_patterns(dtype):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = decode_bits(bits, dtype)
    fin = np.isfinite(v)
    assert np.array_equal(encode_bits(v[fin], dtype), bits[fin])
    assert np.array_equal(round_to_dtype(v[fin], dtype), v[fin])    # representable values are fixed points


# --------------------------------------------------------------------------- consumer add

@pytest.mark.parametrize("dtype,td", [("bf16", torch.bfloat16), ("fp16", torch.float16)])
def test_consumer_add_equals_fp32_add_then_round(dtype, td):
    """One rounding of the exact sum equals an fp32 add followed by a 16-bit rounding.

    fp32 carries at least 2p + 2 significand bits for both 16-bit types, so
    rounding twice is innocuous for addition (Figueroa's double-rounding
    condition); the route through torch's fp32 add and conversion is an
    independent check of the oracle's single rounding.
    """
    rng = np.random.Generator(np.random.PCG64(8))
    n = 50000
    span = 20 if dtype == "fp16" else 60
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-span // 2, span // 2, size=n))).astype(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-span // 2, span // 2, size=n))).astype(np.float32)
    ta, tb = torch.from_numpy(a).to(td), torch.from_numpy(b).to(td)
    abits = ta.view(torch.int16).numpy().view(np.uint16)
    bbits = tb.view(torch.int16).numpy().view(np.uint16)
    lib = (ta.float() + tb.float()).to(td).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(consume_add(abits, bbits, dtype), lib)


def test_consumer_add_known_values():
    one, half = 0x3F80, 0x3F00            # bf16 1.0, 0.5
    tiny = 0x3B80                          # bf16 2^-8: 1 + 2^-8 is a tie -> 1.0
    out = consume_add(np.array([one, one, one], np.uint16), np.array([one, half, tiny], np.uint16), "bf16")
    assert out.tolist() == [0x4000, 0x3FC0, 0x3F80]


# --------------------------------------------------------------------------- GEMM

def _triple_loop(A, B):
    M, K = len(A), len(A[0])
    N = len(B[0])
    return [[math.fsum(A[i][k] * B[k][j] for k in range(K)) for j in range(N)] for i in range(M)]


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (8, 2, 16), (1, 9, 4), (6, 6, 33)])
def test_gemm_against_triple_loop_within_higham_bound(M, N, K):
    rng = np.random.Generator(np.random.PCG64(M * 100 + N * 10 + K))
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    ref = np.array(_triple_loop(A.tolist(), B.tolist()))
    got = gemm_fp64(A, B)
    u = 2.0 ** -53
    gamma = K * u / (1 - K * u)
    bound = gamma * (np.abs(A) @ np.abs(B))
    assert np.all(np.abs(got - ref) <= bound + 1e-300)


def test_gemm_rejects_transposed_shapes():
    with pytest.raises(ValueError):
        gemm_fp64(np.ones((3, 4)), np.ones((3, 4)))


def test_gemm_closed_forms():
    rng = np.random.Generator(np.random.PCG64(1))
    A = rng.standard_normal((5, 6))
    assert np.array_equal(gemm_fp64(A, np.eye(6)), A)
    assert np.array_equal(gemm_fp64(np.ones((4, 9)), np.ones((9, 3))), np.full((4, 3), 9.0))
    T1 = rng.integers(-1, 2, size=(7, 256)).astype(np.float64)
    T2 = rng.integers(-1, 2, size=(256, 5)).astype(np.float64)
    exact = np.array([[sum(int(T1[i, k]) * int(T2[k, j]) for k in range(256)) for j in range(5)] for i in range(7)])
    assert np.array_equal(gemm_fp64(T1, T2), exact)
    # ternary products with K <= 256 are integers of magnitude <= 256: exact in bf16 and fp16
    for dt in ("bf16", "fp16"):
        assert np.array_equal(round_to_dtype(exact, dt), exact)
