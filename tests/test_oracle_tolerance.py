"""Pins of the oracle's tolerance metrics against values worked out by hand.

Every GPU parity verdict rests on rel_frobenius (the layer-output bound of
2e-3, exl3xpu README "Correctness" and "P4-03 prefill is deliberately not in
service", defect 2) and on the per-element bound beside it, so each is
checked here on small arrays whose answers are known without running either
function: a wrong denominator, a missing square root, a max-abs or spectral
norm in place of the Frobenius one, or a mean-abs in place of the rms each
fail one of these cases.
"""
import math

import numpy as np
import pytest

from oracle import exl3_oracle as O


def test_rel_frobenius_vector_known_value():
    # ||[0.3, 0.4]|| = 0.5, ||[3, 4]|| = 5: 0.1.  Dividing by ||a|| instead
    # (||[3.3, 4.4]|| = 5.5) gives 0.0909; no square root 0.01; the largest
    # component 0.08.
    assert O.rel_frobenius([3.3, 4.4], [3.0, 4.0]) == pytest.approx(0.1, rel=1e-14)
    assert O.rel_frobenius([3.0, 4.5], [3.0, 4.0]) == 0.1


def test_rel_frobenius_matrix_is_frobenius_not_spectral():
    # ||diag(0.3, 0)||_F / ||diag(3, 4)||_F = 0.3 / 5 = 0.06; the spectral
    # norm would give 0.3 / 4 = 0.075 and the nuclear one 0.3 / 7.
    ref = np.array([[3.0, 0.0], [0.0, 4.0]])
    a = np.array([[3.3, 0.0], [0.0, 4.0]])
    assert O.rel_frobenius(a, ref) == pytest.approx(0.06, rel=1e-14)


def test_rel_frobenius_higher_rank():
    # all 8 elements 1 (norm sqrt 8), one of them off by 1: 1 / sqrt(8)
    ref = np.ones((2, 2, 2))
    a = ref.copy()
    a[1, 0, 1] = 2.0
    assert O.rel_frobenius(a, ref) == pytest.approx(1.0 / math.sqrt(8.0), rel=1e-15)


def test_rel_frobenius_zero_reference_and_equality():
    assert O.rel_frobenius([[3.0, 4.0]], np.zeros((1, 2))) == 5.0
    assert O.rel_frobenius([1.0, -2.0, 7.5], [1.0, -2.0, 7.5]) == 0.0
    # fp16 inputs are widened exactly: 1 + 2^-10 against 1 is 2^-10 / sqrt(2)
    a = np.array([1.0, 1.0 + 2.0 ** -10], dtype=np.float16)
    assert O.rel_frobenius(a, [1.0, 1.0]) == pytest.approx(2.0 ** -10 / math.sqrt(2.0), rel=1e-15)


def test_rel_frobenius_scale_and_sign():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((7, 9))
    a = ref + 1e-3 * rng.standard_normal((7, 9))
    e = O.rel_frobenius(a, ref)
    assert O.rel_frobenius(8.0 * a, 8.0 * ref) == pytest.approx(e, rel=1e-14)
    assert O.rel_frobenius(-a, -ref) == pytest.approx(e, rel=1e-14)
    # not symmetric in its arguments: the reference sets the scale
    assert O.rel_frobenius(ref, a) != pytest.approx(e, rel=1e-9)


def test_fp16_ulp_against_numpy_spacing():
    # every finite fp16 magnitude below the largest binade: the spacing numpy
    # reports for the fp16 value itself
    vals = np.arange(0, 0x7800, dtype=np.uint16).view(np.float16)
    want = np.spacing(vals).astype(np.float64)
    np.testing.assert_array_equal(O.fp16_ulp(vals.astype(np.float64)), want)
    np.testing.assert_array_equal(O.fp16_ulp(-vals.astype(np.float64)), want)
    # hand values: 1 and 1.5 -> 2^-10, 2 -> 2^-9, 0.75 -> 2^-11, 0 -> 2^-24
    np.testing.assert_array_equal(O.fp16_ulp([1.0, 1.5, 2.0, 0.75, 0.0, 65504.0]),
                                  [2.0 ** -10, 2.0 ** -10, 2.0 ** -9, 2.0 ** -11, 2.0 ** -24, 32.0])


def test_elementwise_excess_known_values():
    ref = np.array([3.0, 0.0, 0.0, 4.0])  # rms 2.5 (mean |.| 1.75, max 4)
    a = ref + np.array([0.0, 0.025, 0.0, 0.0])
    # 0.025 / (0.01 * 2.5) = 1 with no ulp term
    assert O.elementwise_excess(a, ref, 0.01, ulps=0.0) == pytest.approx(1.0, rel=1e-12)
    # one ulp of 0 is 2^-24
    assert O.elementwise_excess(a, ref, 0.01, ulps=1.0) == pytest.approx(0.025 / (0.025 + 2.0 ** -24), rel=1e-12)
    # the largest ratio wins: element 0 is off by 0.05 against 0.025 + ulp(3) = 0.025 + 2^-9
    b = ref + np.array([0.05, 0.025, 0.0, 0.0])
    assert O.elementwise_excess(b, ref, 0.01, ulps=1.0) == pytest.approx(0.05 / (0.025 + 2.0 ** -9), rel=1e-12)
    assert O.elementwise_excess(ref, ref, 0.01) == 0.0
    assert O.elementwise_excess(np.zeros((0, 3)), np.zeros((0, 3)), 0.01) == 0.0


def test_elementwise_excess_catches_one_bad_element_the_norm_misses():
    # one element off by 3 rms in four million stays under the 2e-3 Frobenius
    # bound (3 / 2048) but not under a per-element one of 1e-2 rms
    rng = np.random.default_rng(6)
    ref = rng.standard_normal(1 << 22)
    a = ref.copy()
    a[12345] += 3.0
    assert O.rel_frobenius(a, ref) < 2e-3
    assert O.elementwise_excess(a, ref, 1e-2) > 100.0
