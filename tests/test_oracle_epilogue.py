"""Pins of the epilogue oracle (oracle/epilogue.py) and its error criterion.

Expected values are written out by hand for tiny integer inputs, or come from
mathematics independent of the oracle's code: the normal distribution's CDF at 1
(a standard table value), the erf form of GELU from a library special function,
and the odd-symmetry identity GELU(x) - GELU(-x) = x that both forms satisfy.
"""
import math

import numpy as np
import pytest

from oracle.check import OUT_UNIT, TOL, epilogue_error
from oracle.epilogue import epilogue_ref, gelu_tanh

C = np.array([[1.0, 2.0], [3.0, 4.0]])
D = np.array([[1.0, 2.0], [3.0, 4.0]])
R = np.array([[1.0, 0.0], [0.0, 1.0]])
BIAS = np.array([10.0, -10.0])


def test_identity_is_the_product():
    x, Dp = epilogue_ref(C, D)
    assert np.array_equal(x, C) and np.array_equal(Dp, D)


def test_linear_terms_by_hand():
    # 2*C - 3*R + bias, worked out entry by entry
    x, Dp = epilogue_ref(C, D, alpha=2.0, beta=-3.0, R=R, bias=BIAS)
    assert np.array_equal(x, [[9.0, -6.0], [16.0, -5.0]])
    # |2| D + |-3| |R| + |bias|
    assert np.array_equal(Dp, [[15.0, 14.0], [16.0, 21.0]])
    # beta = 0 ignores R entirely (even a NaN one)
    x, _ = epilogue_ref(C, D, alpha=-1.0, beta=0.0, R=np.full((2, 2), np.nan))
    assert np.array_equal(x, -C)


def test_relu_by_hand():
    x, _ = epilogue_ref(C, D, alpha=2.0, beta=-3.0, R=R, bias=BIAS, act="relu")
    assert np.array_equal(x, [[9.0, 0.0], [16.0, 0.0]])


def test_gelu_tanh_against_independent_facts():
    # Phi(1) = 0.8413447460685429 (standard normal table); GELU(1) = Phi(1) exactly,
    # and the tanh form is within 2e-4 of it
    assert abs(float(gelu_tanh(1.0)) - 0.8413447460685429) < 2e-4
    assert float(gelu_tanh(0.0)) == 0.0
    xs = np.linspace(-7.0, 7.0, 1401)
    # odd-symmetry identity of both GELU forms: GELU(x) - GELU(-x) = x
    assert np.max(np.abs(gelu_tanh(xs) - gelu_tanh(-xs) - xs)) < 1e-12
    # close to the erf form x * Phi(x) everywhere (the approximation's known accuracy)
    from scipy.special import erf
    exact = 0.5 * xs * (1.0 + erf(xs / math.sqrt(2.0)))
    assert np.max(np.abs(gelu_tanh(xs) - exact)) < 1e-3
    # saturation: x for large x, 0 for large -x
    assert abs(float(gelu_tanh(12.0)) - 12.0) < 1e-12 and abs(float(gelu_tanh(-12.0))) < 1e-12


def test_unknown_activation_rejected():
    with pytest.raises(ValueError):
        epilogue_ref(C, D, act="swish")


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_error_criterion(out):
    ref, Dp = epilogue_ref(C, D, alpha=2.0, beta=-3.0, R=R, bias=BIAS, act="gelu_tanh")
    assert epilogue_error(ref, ref, Dp, "f32", out) == 0.0
    bound = (1.2 * TOL["f32"] + 1e-6) * Dp + OUT_UNIT[out] * np.abs(ref)
    assert epilogue_error(ref + 0.9 * bound, ref, Dp, "f32", out) <= 1.0
    assert epilogue_error(ref + 2.0 * bound, ref, Dp, "f32", out) > 1.0
    bad = ref.copy()
    bad[0, 0] = np.nan
    assert epilogue_error(bad, ref, Dp, "f32", out) == float("inf")
    if out == "f16":
        # the value rounded to fp16 passes
        assert epilogue_error(ref.astype(np.float16).astype(np.float64), ref, Dp, "f32", out) <= 1.0
