"""Pins of the fused post-reorder epilogue (deep-dive 五 › Epilogue 集成).

No activation and no bias reduce to the already pinned post-reorder; ReLU is
checked as an invariant against the unactivated result; SiLU against
scipy's logistic function and the identity silu(x) - silu(-x) = x; the bias
against per-problem constants.
"""

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle.epilogue import activation, post_epilogue, row_problems
from oracle.layout import element_offsets
from oracle.tiles import make_plan
from workloads import random_bits, to_bits


def _plan():
    return make_plan([70, 0, 130, 64], 192, BM=128, BN=128, S=2, W=3, mode="subtoken", ranks=4,
                     row_dest=np.random.Generator(np.random.PCG64(5)).integers(0, 4, size=264))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_identity_epilogue_is_the_post_reorder(dtype):
    p = _plan()
    off = element_offsets(p)
    y = random_bits(3, p.M * p.N, dtype)
    np.testing.assert_array_equal(post_epilogue(y, off, dtype), oracle.post_reorder(y, off))


def test_relu_keeps_positives_and_zeroes_the_rest():
    p = _plan()
    off = element_offsets(p)
    y = to_bits(np.random.Generator(np.random.PCG64(4)).normal(0, 1, p.M * p.N), "bf16")
    bias = to_bits(np.random.Generator(np.random.PCG64(6)).normal(0, 1, 4 * p.N), "bf16")
    none = oracle.decode_bits(post_epilogue(y, off, "bf16", "none", bias, row_problems(p)), "bf16")
    relu = oracle.decode_bits(post_epilogue(y, off, "bf16", "relu", bias, row_problems(p)), "bf16")
    assert np.all(relu >= 0)
    np.testing.assert_array_equal(relu[none > 0], none[none > 0])
    assert np.all(relu[none <= 0] == 0)


def test_silu_against_the_logistic_function_and_its_odd_part():
    x = np.linspace(-30, 30, 2001)
    np.testing.assert_allclose(activation(x, "silu"), x * expit(x), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(activation(x, "silu") - activation(-x, "silu"), x, rtol=1e-13, atol=1e-13)
    assert activation(np.array([0.0]), "silu")[0] == 0.0
    assert activation(np.array([-800.0]), "silu")[0] == 0.0          # exp overflow: -0


def test_bias_follows_the_rows_problem():
    p = _plan()
    off = element_offsets(p)
    zero = np.zeros(p.M * p.N, np.uint16)
    consts = [0.5, -1.25, 2.0, 3.5]
    bias = to_bits(np.repeat(consts, p.N), "bf16")
    out = oracle.decode_bits(post_epilogue(zero, off, "bf16", "none", bias, row_problems(p)), "bf16")
    want = np.repeat(np.array(consts)[row_problems(p)][:, None], p.N, axis=1)
    np.testing.assert_array_equal(out, want)
    silu = oracle.decode_bits(post_epilogue(zero, off, "bf16", "silu", bias, row_problems(p)), "bf16")
    np.testing.assert_allclose(silu, want * expit(want), rtol=2 ** -8)
