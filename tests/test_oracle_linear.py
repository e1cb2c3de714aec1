"""Pins for the oracle's EXL3 linear layer (CPU only)."""
import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O


def _inputs(seed, m, k, n, kbits):
    return synth.linear_inputs(seed, m, k, n, kbits)


@pytest.mark.parametrize("k,n,kbits", [(128, 128, 4), (256, 128, 3), (128, 384, 2), (256, 256, 8)])
def test_fast_route_equals_effective_weight_route(k, n, kbits):
    d = _inputs(11, 3, k, n, kbits)
    a = O.linear(d["x"], d["trellis"], d["suh"], d["svh"], kbits)
    b = O.linear_weff(d["x"], d["trellis"], d["suh"], d["svh"], kbits)
    assert O.rel_frobenius(a, b) < 1e-12


@pytest.mark.parametrize("fill", [0x0000, 0xFFFF])
def test_constant_trellis_closed_form(fill):
    # All states equal S => W~ = c * ones, c = v(S).  Then
    #   y[r, 128b'] = c * 128 * (sum_b x[r, 128b] suh[128b]) * svh[128b']
    # and y is exactly zero in every other column.
    k, n, m = 384, 256, 4
    d = _inputs(12, m, k, n, 4)
    t = np.full_like(d["trellis"], fill)
    c = float(O.mul1_value(np.array([fill]))[0])
    y = O.linear(d["x"], t, d["suh"], d["svh"], 4)
    xs = d["x"].astype(np.float64) * d["suh"].astype(np.float64)
    col0 = c * 128.0 * xs[:, ::128].sum(axis=1)
    for b2 in range(n // 128):
        np.testing.assert_allclose(y[:, 128 * b2], col0 * float(d["svh"][128 * b2]), rtol=1e-12)
    mask = np.ones(n, bool); mask[::128] = False
    assert np.abs(y[:, mask]).max() < 1e-9 * np.abs(col0).max()


def test_sign_invariances():
    k, n = 256, 256
    d = _inputs(13, 2, k, n, 4)
    y = O.linear(d["x"], d["trellis"], d["suh"], d["svh"], 4)
    x2 = d["x"].copy(); s2 = d["suh"].copy()
    x2[:, 7] = -x2[:, 7]; s2[7] = -s2[7]
    np.testing.assert_allclose(O.linear(x2, d["trellis"], s2, d["svh"], 4), y, atol=1e-12)
    v2 = d["svh"].copy(); v2[9] = -v2[9]
    y3 = O.linear(d["x"], d["trellis"], d["suh"], v2, 4)
    np.testing.assert_allclose(y3[:, 9], -y[:, 9], atol=1e-12)
    np.testing.assert_allclose(np.delete(y3, 9, axis=1), np.delete(y, 9, axis=1), atol=1e-12)
    np.testing.assert_allclose(O.linear(-d["x"], d["trellis"], d["suh"], d["svh"], 4), -y, atol=1e-12)


def test_rows_independent_and_linear():
    k, n = 256, 128
    d = _inputs(14, 5, k, n, 3)
    y = O.linear(d["x"], d["trellis"], d["suh"], d["svh"], 3)
    for r in range(5):
        yr = O.linear(d["x"][r:r + 1], d["trellis"], d["suh"], d["svh"], 3)
        np.testing.assert_allclose(yr[0], y[r], atol=1e-12)
    y2 = O.linear(2.0 * d["x"].astype(np.float64) + 1.0, d["trellis"], d["suh"], d["svh"], 3)
    y1 = O.linear(np.ones_like(d["x"], dtype=np.float64), d["trellis"], d["suh"], d["svh"], 3)
    np.testing.assert_allclose(y2, 2.0 * y + y1, atol=1e-10)


def test_single_nonzero_state_brute_force():
    # Trellis of zeros except one tile whose words make exactly one state
    # differ: the layer output then differs from the constant-trellis output by
    # the outer product of one Hadamard row and one Hadamard column.
    k, n, kbits = 256, 256, 4
    d = _inputs(15, 1, k, n, kbits)
    t0 = np.zeros_like(d["trellis"])
    t1 = t0.copy()
    # In a K=4 tile only states 0, 253, 254, 255 see bit 0 of word 0 (see the
    # tail-biting pin); use a bit that only state 1 sees: bit 4 of the stream
    # is inside windows 0 (offset 4) and 1 (offset 0); pick instead word 1 bit 0
    # (stream bit 16) seen by states 1, 2, 3, 4.  We compute the expected
    # difference straight from the definition of W~ entries.
    t1[1, 2, 1] = 0x8000
    W0 = O.decode_tensor(t0, kbits).astype(np.float64)
    W1 = O.decode_tensor(t1, kbits).astype(np.float64)
    diff = np.argwhere(W1 != W0)
    # stream bit 16 lies in the windows of states 1..4, i.e. row 0, columns 1..4
    assert sorted(map(tuple, diff)) == [(16, 32 + c) for c in range(1, 5)]
    y0 = O.linear(d["x"], t0, d["suh"], d["svh"], kbits)
    y1 = O.linear(d["x"], t1, d["suh"], d["svh"], kbits)
    H = O.sylvester_hadamard() / np.sqrt(128)
    xs = d["x"][0].astype(np.float64) * d["suh"].astype(np.float64)
    xp = xs[:128] @ H                       # row 16 lives in the first 128-block
    dy = np.zeros(n)
    for (r, c) in diff:
        dW = W1[r, c] - W0[r, c]
        dy[:128] += xp[r] * dW * H[c, :] if c < 128 else 0
    dy *= d["svh"].astype(np.float64)
    np.testing.assert_allclose(y1[0] - y0[0], dy, atol=1e-10)


def test_bias_added_last():
    k, n = 128, 256
    d = _inputs(16, 2, k, n, 4)
    bias = np.linspace(-1, 1, n).astype(np.float16)
    y = O.linear(d["x"], d["trellis"], d["suh"], d["svh"], 4)
    yb = O.linear(d["x"], d["trellis"], d["suh"], d["svh"], 4, bias=bias)
    np.testing.assert_allclose(yb - y, np.broadcast_to(bias.astype(np.float64), y.shape), atol=1e-12)


def test_mixed_layer_generator_order_and_widths():
    # widths come first and do not depend on the activation count; tensors are
    # drawn before activations, so m changes only x
    a = synth.mixed_layer_inputs(synth.SEED_MIXED_LAYER, 1,
                                 shapes=(("q", 256, 128), ("k", 128, 256), ("down", 384, 128)))
    b = synth.mixed_layer_inputs(synth.SEED_MIXED_LAYER, 3,
                                 shapes=(("q", 256, 128), ("k", 128, 256), ("down", 384, 128)))
    _, bits = synth.mixed_layer_bits(synth.SEED_MIXED_LAYER, ("q", "k", "down"))
    for nm in ("q", "k", "down"):
        assert a[nm]["bits"] == b[nm]["bits"] == bits[nm]
        assert 2 <= bits[nm] <= 8
        assert np.array_equal(a[nm]["trellis"], b[nm]["trellis"])
        assert a[nm]["trellis"].shape == (a[nm]["k"] // 16, a[nm]["n"] // 16, 16 * bits[nm])
        assert a[nm]["x"].shape == (1, a[nm]["k"]) and b[nm]["x"].shape == (3, b[nm]["k"])
    # bits-per-weight accounting of the full layer: trellis bytes = sum k n K / 8
    _, full = synth.mixed_layer_bits(synth.SEED_MIXED_LAYER)
    nbytes = sum(k * n * full[nm] // 8 for nm, k, n in synth.MIXED_LAYER_SHAPES)
    assert 93_061_120 <= nbytes <= 372_244_480
