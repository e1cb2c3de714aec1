"""Seeded property sweep over shapes, widths and row counts (hypothesis,
derandomized so every run draws the same cases): exl3_linear against the
float64 oracle (relative Frobenius error and the per-element bound),
exl3_reconstruct bit for bit, and exl3_linear_int8 against the oracle's int8
readings.  k and n are multiples of 128 (exl3xpu README, "Adding a model");
widths 1..8 (TensorFold issue #832); rows from one (decode) through both
GEMV paths, the GEMM's short tiles and a few hundred (prefill)."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

import synth
from oracle import exl3_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu

SWEEP = settings(max_examples=40, derandomize=True, deadline=None, database=None,
                 suppress_health_check=list(HealthCheck))
rows = st.one_of(st.integers(1, 20), st.integers(280, 320))


@SWEEP
@given(kb=st.integers(1, 16), nb=st.integers(1, 12), bits=st.integers(1, 8), m=rows,
       seed=st.integers(0, 1 << 20))
def test_linear_sweep(kb, nb, bits, m, seed):
    import torch
    import gemm_exl3_linear_amd as X
    k, n = 128 * kb, 128 * nb
    d = synth.linear_inputs(seed, m, k, n, bits)
    y = X.exl3_linear(G.to_dev(d["x"]), G.weight(d))
    torch.cuda.synchronize()
    ref = O.linear(d["x"], d["trellis"], d["suh"], d["svh"], bits)
    G.assert_parity(y.double().cpu().numpy(), ref, what=f"k={k} n={n} K={bits} m={m}")


@SWEEP
@given(kt=st.integers(1, 24), nt=st.integers(1, 24), bits=st.integers(1, 8), seed=st.integers(0, 1 << 20))
def test_reconstruct_sweep(kt, nt, bits, seed):
    import torch
    import gemm_exl3_linear_amd as X
    d = synth.linear_inputs(seed, 1, 16 * kt, 16 * nt, bits)
    W = X.exl3_reconstruct(G.weight(d))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(G.f16_bits(W), O.decode_tensor(d["trellis"], bits).view(np.uint16))


@SWEEP
@given(kb=st.integers(1, 12), nb=st.integers(1, 8), bits=st.integers(1, 8), m=rows,
       seed=st.integers(0, 1 << 20))
def test_linear_int8_sweep(kb, nb, bits, m, seed):
    import torch
    import gemm_exl3_linear_amd as X
    k, n = 128 * kb, 128 * nb
    d = synth.linear_inputs(seed, m, k, n, bits)
    y = X.exl3_linear_int8(G.to_dev(d["x"]), G.weight(d))
    torch.cuda.synchronize()
    ref = O.linear_int8(d["x"], d["trellis"], d["suh"], d["svh"], bits)
    G.assert_parity(y.double().cpu().numpy(), ref, tol=1e-3, rel_rms=1e-2, what=f"int8 k={k} n={n} K={bits} m={m}")
