"""GPU parity of the mixed-width decoder layer: seven EXL3 projections (q, k,
v, o at 5120 x 5120, gate and up 5120 x 17408, down 17408 x 5120) whose widths
are drawn from 2..8 per tensor (TensorFold issue #832, "Description": widths
are mixed per tensor).  Decoded weights must be bit-identical to the float64
oracle's; outputs must be within 2e-3 relative Frobenius error, at one row
(decode GEMV) and at 4096 rows (prefill GEMM, every row, in the launch
configuration the benchmark times, through the fp16 and the int8 paths), with
every element within a per-element bound too."""
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


@functools.lru_cache(maxsize=1)
def _decoded(nm):
    d = _layer(1)[nm]
    return G.decode_par(d["trellis"], d["bits"])


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
    G.assert_parity(y.double().cpu().numpy(), ref, what=f"{nm} K={d['bits']}")


@pytest.mark.parametrize("nm", NAMES)
def test_mixed_layer_m4096_all_rows(nm):
    import torch
    import gemm_exl3_linear_amd as X
    d4 = _layer(4096)[nm]
    # the tensors are drawn before the activations, so they equal the m = 1 draw
    assert np.array_equal(d4["trellis"], _layer(1)[nm]["trellis"])
    w = G.weight(d4)
    x = G.to_dev(d4["x"])
    y = X.exl3_linear(x, w)
    torch.cuda.synchronize()
    G.assert_parity(y.double().cpu().numpy(), G.linear_ref(d4, W=_decoded(nm)), what=f"{nm} K={d4['bits']}")
    del y
    y8 = X.exl3_linear_int8(x, w)
    torch.cuda.synchronize()
    ref8 = G.linear_int8_ref(d4)
    G.assert_parity(y8.double().cpu().numpy(), ref8, tol=1e-3, what=f"int8 {nm} K={d4['bits']}")
