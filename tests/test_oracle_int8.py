"""Pins for the oracle's int8 prefill readings (CPU only).

exl3xpu README, "Prefill: int8 linears and oneDNN fused attention": one int8
scale per activation row after the input transform, one static weight scale
from the codebook bound 3.453125, an int8 product with both scales applied.
Every check below reaches the oracle's result by another route: exact
rational arithmetic, closed forms, invariants, explicit Hadamard matrices.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O


def _round_half_even(f: Fraction) -> int:
    return round(f)  # Python rounds a Fraction to nearest, ties to even


def test_weight_quantizer_equals_exact_rationals():
    # I8W over every byte sum, in exact arithmetic: the bound 3.453125 is
    # 221/64, so the static scale is 127 * 64 / 221.
    scale = Fraction(127 * 64, 221)
    want = [_round_half_even(Fraction((s - 510) * 1775, 1 << 18) * scale) for s in range(1021)]
    got = O.mul1_int8_from_sigma(np.arange(1021)).astype(int).tolist()
    assert got == want


def test_weight_quantizer_has_no_ties_and_endpoints():
    scale = Fraction(127 * 64, 221)
    dist = min(abs(Fraction((s - 510) * 1775, 1 << 18) * scale % 1 - Fraction(1, 2)) for s in range(1021))
    assert dist > Fraction(1, 1000)
    q = O.mul1_int8_from_sigma(np.arange(1021)).astype(int)
    assert q[0] == -127 and q[510] == 0 and q[1020] == 127
    assert (np.diff(q) >= 0).all()
    # the largest codebook value maps to the int8 limit
    assert _round_half_even(Fraction(221, 64) * scale) == 127


def test_weight_quantizer_over_all_states():
    # Every 16-bit state: within half an int8 step of the unrounded codebook
    # value, and within that plus half an fp16 ulp (2**-10 below 4) of the
    # fp16 decoded weight.
    s = np.arange(1 << 16)
    q = O.mul1_int8(s).astype(np.float64)
    sig = O.mul1_sigma(s)
    exact = (sig - 510) * 1775 / 2.0 ** 18
    step = 3.453125 / 127
    assert np.abs(q * step - exact).max() <= step / 2 + 1e-15
    v16 = O.mul1_value(s).astype(np.float64)
    assert np.abs(q * step - v16).max() <= step / 2 + 2.0 ** -10
    assert q.min() == -127 and abs(q).max() <= 127


def test_decode_tensor_int8_placement():
    # Same placement as the fp16 decode: the int8 weight of each position
    # comes from the state that gives that position its fp16 weight.
    d = synth.linear_inputs(30, 1, 64, 48, 3)
    W = O.decode_tensor(d["trellis"], 3).astype(np.float64)
    Q = O.decode_tensor_int8(d["trellis"], 3).astype(np.float64)
    assert Q.shape == W.shape and Q.dtype == np.float64
    assert np.abs(Q * (3.453125 / 127) - W).max() <= 3.453125 / 254 + 2.0 ** -10
    # and the fp16 decode is a function of the int8 one's state: equal states
    # give equal int8 codes
    st = O.tensor_states(d["trellis"], 3).reshape(-1)
    q = O.mul1_int8(st)
    for s_val in np.unique(st)[:50]:
        assert len(np.unique(q[st == s_val])) == 1


def test_quantize_rows_properties():
    g = np.random.default_rng(31)
    xp = g.standard_normal((6, 256))
    xp[3] = 0.0
    q, s = O.quantize_rows(xp)
    assert q.dtype == np.int8
    a = np.abs(xp).max(axis=1)
    for r in range(6):
        if r == 3:
            assert (q[r] == 0).all() and s[r] == 0
            continue
        i = int(np.abs(xp[r]).argmax())
        assert abs(int(q[r, i])) == 127 and np.sign(q[r, i]) == np.sign(xp[r, i])
        assert s[r] == a[r] / 127
        # rounding bound, independent of the implementation
        assert np.abs(q[r] - 127 * xp[r] / a[r]).max() <= 0.5 + 1e-12
    # power-of-two scaling leaves the codes alone and scales the scale
    q2, s2 = O.quantize_rows(4.0 * xp)
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, 4.0 * s)
    # sign symmetry
    qn, sn = O.quantize_rows(-xp)
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(sn, s)


def test_quantize_rows_ties_go_to_even():
    xp = np.array([[127.0, 2.5, -2.5, 3.5, 0.5, -0.5, 1.5]])
    q, s = O.quantize_rows(xp)
    assert q[0].tolist() == [127, 2, -2, 4, 0, 0, 2]
    assert s[0] == 1.0


def _explicit_hadamard(d: int) -> np.ndarray:
    h = np.array([[1.0]])
    while h.shape[0] < 128:
        h = np.block([[h, h], [h, -h]])
    return np.kron(np.eye(d // 128), h / math.sqrt(128))


@pytest.mark.parametrize("k,n,bits,m", [(128, 128, 4, 3), (256, 384, 3, 5), (384, 256, 8, 2)])
def test_linear_int8_equals_dequantized_explicit_route(k, n, bits, m):
    # Second route: explicit Hadamard matrices and the dequantized operands
    # (x_q * scale) and (W_q * 3.453125 / 127) multiplied in float64.
    d = synth.linear_inputs(32 + bits, m, k, n, bits)
    y = O.linear_int8(d["x"], d["trellis"], d["suh"], d["svh"], bits)
    Hk, Hn = _explicit_hadamard(k), _explicit_hadamard(n)
    xp = (d["x"].astype(np.float64) * d["suh"].astype(np.float64)) @ Hk
    xq, sx = O.quantize_rows(xp)
    Wd = O.decode_tensor_int8(d["trellis"], bits).astype(np.float64) * (3.453125 / 127)
    y2 = ((xq.astype(np.float64) * sx[:, None]) @ Wd) @ Hn * d["svh"].astype(np.float64)
    assert O.rel_frobenius(y, y2) < 1e-12


@pytest.mark.parametrize("fill", [0x0000, 0xFFFF])
def test_linear_int8_constant_trellis_closed_form(fill):
    # A trellis of all-zero or all-one words has every state equal to that
    # word (D2), so W_q = q_S everywhere and
    #   y'[r, j] = q_S * (sum_i x_q[r, i]) * scale_r * 3.453125 / 127 for every j,
    # and the output transform puts y'[r] * sqrt(128) * svh at column 128 b,
    # exactly zero elsewhere.
    k, n, m = 256, 384, 4
    d = synth.linear_inputs(33, m, k, n, 4)
    t = np.full_like(d["trellis"], fill)
    qs = int(O.mul1_int8(np.array([fill]))[0])
    assert qs == (-127 if fill == 0 else int(np.rint(float(O.mul1_value(np.array([fill]))[0]) * 127 / 3.453125)))
    y = O.linear_int8(d["x"], t, d["suh"], d["svh"], 4)
    xp = (d["x"].astype(np.float64) * d["suh"].astype(np.float64)) @ _explicit_hadamard(k)
    xq, sx = O.quantize_rows(xp)
    yp = qs * xq.astype(np.float64).sum(axis=1) * sx * 3.453125 / 127
    for b in range(n // 128):
        np.testing.assert_allclose(y[:, 128 * b], yp * math.sqrt(128) * float(d["svh"][128 * b]), rtol=1e-12)
    mask = np.ones(n, bool)
    mask[::128] = False
    assert np.abs(y[:, mask]).max() < 1e-9 * np.abs(yp).max()


def test_linear_int8_zero_rows_give_bias():
    d = synth.linear_inputs(34, 3, 128, 256, 4)
    x = d["x"].copy()
    x[1] = 0
    bias = (np.arange(256) % 7 - 3).astype(np.float16)
    y = O.linear_int8(x, d["trellis"], d["suh"], d["svh"], 4, bias=bias)
    np.testing.assert_array_equal(y[1], bias.astype(np.float64))


def test_linear_int8_error_budget_against_fp16_layer():
    # The int8 tolerance: against the fp16-weight layer, int8 rounding of
    # activations (about max/254 per element) and weights (3.453125/254)
    # costs about 1e-2 of relative Frobenius error on these inputs; the
    # bound 2e-2 separates it from a wrong scale or placement (errors of
    # order 1).
    d = synth.linear_inputs(35, 8, 512, 256, 4)
    y8 = O.linear_int8(d["x"], d["trellis"], d["suh"], d["svh"], 4)
    y16 = O.linear(d["x"], d["trellis"], d["suh"], d["svh"], 4)
    err = O.rel_frobenius(y8, y16)
    assert 1e-3 < err < 2e-2, err
