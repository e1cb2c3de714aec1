"""GPU parity of the mixed-width decoder layer: seven EXL3 projections (q, k,
v, o at 5120 x 5120, gate and up 5120 x 17408, down 17408 x 5120) whose widths
are drawn from 2..8 per tensor (TensorFold issue #832, "Description": widths
are mixed per tensor).  Decoded weights must be bit-identical to the float64
oracle's; outputs must be within 2e-3 relative Frobenius error, at one row
(decode GEMV) and at 4096 rows (prefill GEMM, checked on sampled rows in the
launch configuration the benchmark times)."""
import functools

import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
TOL = 2e-3
NAMES = [nm for nm, _, _ in synth.MIXED_LAYER_SHAPES]


@functools.lru_cache(maxsize=2)
def _layer(m):
    return synth.mixed_layer_inputs(synth.SEED_MIXED_LAYER, m)


@functools.lru_cache(maxsize=8)
def _decoded(nm):
    d = _layer(1)[nm]
    return O.decode_tensor(d["trellis"], d["bits"])


def test_mixed_layer_widths_cover_range():
    bits = {nm: _layer(1)[nm]["bits"] for nm in NAMES}
    assert all(2 <= b <= 8 for b in bits.values())
    assert len(set(bits.values())) >= 3, bits


@pytest.mark.parametrize("nm", NAMES)
def test_mixed_layer_decode_bit_exact(nm):
    import torch
    import gemm_exl3_linear_amd as X
    d = _layer(1)[nm]
    W = X.exl3_reconstruct(G.weight(d))
    torch.cuda.synchronize()
    assert np.array_equal(G.f16_bits(W), _decoded(nm).view(np.uint16))


@pytest.mark.parametrize("nm", NAMES)
def test_mixed_layer_m1(nm):
    import torch
    import gemm_exl3_linear_amd as X
    d = _layer(1)[nm]
    y = X.exl3_linear(G.to_dev(d["x"]), G.weight(d))
    torch.cuda.synchronize()
    ref = O.linear(d["x"], d["trellis"], d["suh"], d["svh"], d["bits"], w_decoded=_decoded(nm))
    err = O.rel_frobenius(y.double().cpu().numpy(), ref)
    assert err < TOL, (nm, d["bits"], err)


@pytest.mark.parametrize("nm", NAMES)
def test_mixed_layer_m4096_sampled_rows(nm):
    import torch
    import gemm_exl3_linear_amd as X
    d4 = _layer(4096)[nm]
    # the tensors are drawn before the activations, so they equal the m = 1 draw
    assert np.array_equal(d4["trellis"], _layer(1)[nm]["trellis"])
    y = X.exl3_linear(G.to_dev(d4["x"]), G.weight(d4))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(4096, 16, replace=False))
    ref = O.linear(d4["x"][rows], d4["trellis"], d4["suh"], d4["svh"], d4["bits"], w_decoded=_decoded(nm))
    err = O.rel_frobenius(y[rows].double().cpu().numpy(), ref)
    assert err < TOL, (nm, d4["bits"], err)
