"""Pins for the oracle's blockwise Hadamard transform (CPU only)."""
import math

import numpy as np
import scipy.linalg

from oracle import exl3_oracle as O
from tests._golden import facts


def test_sylvester_matches_library():
    np.testing.assert_array_equal(O.sylvester_hadamard(128), scipy.linalg.hadamard(128))


def test_block_size_is_the_printed_multiple():
    assert O.HADAMARD_BLOCK == int(facts()["hadamard_multiple"][0])


def test_orthonormal_and_involution():
    H = O.sylvester_hadamard(128) / math.sqrt(128)
    np.testing.assert_allclose(H @ H.T, np.eye(128), atol=1e-14)
    np.testing.assert_allclose(H @ H, np.eye(128), atol=1e-14)


def test_butterfly_equals_library_matrix_product():
    g = np.random.default_rng(3)
    x = g.standard_normal((5, 384))
    ref = (x.reshape(5, 3, 128) @ (scipy.linalg.hadamard(128) / math.sqrt(128))).reshape(5, 384)
    np.testing.assert_allclose(O.fwht(x), ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.hadamard_explicit(x), ref, rtol=0, atol=1e-12)


def test_closed_forms():
    e0 = np.zeros(128); e0[0] = 1.0
    np.testing.assert_allclose(O.fwht(e0), np.full(128, 1 / math.sqrt(128)), atol=1e-15)
    ones = np.ones(128)
    out = O.fwht(ones)
    assert abs(out[0] - math.sqrt(128)) < 1e-12 and np.abs(out[1:]).max() < 1e-12
    # e_i maps to row i of the normalised Sylvester matrix
    e5 = np.zeros(128); e5[5] = 1.0
    np.testing.assert_allclose(O.fwht(e5), scipy.linalg.hadamard(128)[5] / math.sqrt(128), atol=1e-15)


def test_blocks_are_independent_and_norm_preserving():
    g = np.random.default_rng(4)
    x = g.standard_normal((2, 512))
    y = O.fwht(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    x2 = x.copy(); x2[:, 128:256] = 0
    y2 = O.fwht(x2)
    np.testing.assert_allclose(y2[:, :128], y[:, :128], atol=1e-13)
    assert np.abs(y2[:, 128:256]).max() == 0


def test_signed_round_trip():
    g = np.random.default_rng(5)
    x = g.standard_normal((3, 256))
    s = (g.integers(0, 2, 256) * 2 - 1).astype(np.float16)
    back = O.hadamard(O.hadamard(x, sign_before=s), sign_after=s)
    np.testing.assert_allclose(back, x, atol=1e-13)
    # sign before and sign after are different operations
    a = O.hadamard(x, sign_before=s)
    b = O.hadamard(x, sign_after=s)
    assert np.abs(a - b).max() > 1e-3
