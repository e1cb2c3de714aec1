"""GPU parity of exl3_linear_multi: several EXL3 tensors that read one input
(q, k, v; gate and up), each with its own width, shape, signs and bias,
computed in one launch pair at one row (TensorFold issue #832,
"Description": widths are mixed per tensor).  Every output is checked against
the float64 oracle (relative Frobenius error <= 2e-3); at two or more rows the
call runs the single-tensor path and must equal separate exl3_linear calls
bit for bit."""
import functools

import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _tensors(seed, k, shapes, m):
    """One tensor per (n, bits) in `shapes`, all with in_features k, and one
    shared activation block x [m, k]."""
    g = synth.rng(seed)
    ts = []
    for n, bits in shapes:
        t = synth.trellis(g, k, n, bits)
        ts.append(dict(trellis=t, suh=synth.signs(g, k), svh=synth.signs(g, n), k=k, n=n, bits=bits))
    x = synth.activations(g, m, k)
    return ts, x


def _run_multi(ts, x, out_dtype=None, biases=None):
    import torch
    import gemm_exl3_linear_amd as X
    ws = [G.weight(d, bias=None if biases is None else biases[i]) for i, d in enumerate(ts)]
    ys = X.exl3_linear_multi(G.to_dev(x), ws, out_dtype=out_dtype or torch.float16)
    torch.cuda.synchronize()
    return ys


@pytest.mark.parametrize("m", [1, 3, 40])
def test_multi_mixed_widths(m):
    ts, x = _tensors(1100 + m, 512, [(384, 2), (128, 5), (1024, 8), (256, 1)], m)
    ys = _run_multi(ts, x)
    for d, y in zip(ts, ys):
        ref = O.linear(x, d["trellis"], d["suh"], d["svh"], d["bits"])
        err = O.rel_frobenius(y.double().cpu().numpy(), ref)
        assert err < TOL, (d["n"], d["bits"], err)


def test_multi_fp32_output_and_bias():
    import torch
    ts, x = _tensors(1201, 256, [(512, 4), (128, 6)], 1)
    biases = [np.linspace(-1, 1, d["n"]).astype(np.float16) for d in ts]
    ys = _run_multi(ts, x, out_dtype=torch.float32, biases=biases)
    for d, y, b in zip(ts, ys, biases):
        assert y.dtype == torch.float32
        ref = O.linear(x, d["trellis"], d["suh"], d["svh"], d["bits"], bias=b)
        err = O.rel_frobenius(y.double().cpu().numpy(), ref)
        assert err < TOL, err


def test_multi_single_tensor():
    ts, x = _tensors(1301, 1024, [(1024, 3)], 1)
    (y,) = _run_multi(ts, x)
    d = ts[0]
    err = O.rel_frobenius(y.double().cpu().numpy(), O.linear(x, d["trellis"], d["suh"], d["svh"], d["bits"]))
    assert err < TOL, err


def test_multi_rows_equal_single_calls_bitwise():
    import gemm_exl3_linear_amd as X
    ts, x = _tensors(1401, 512, [(256, 3), (384, 7)], 5)
    ys = _run_multi(ts, x)
    for d, y in zip(ts, ys):
        y1 = X.exl3_linear(G.to_dev(x), G.weight(d))
        np.testing.assert_array_equal(G.f16_bits(y), G.f16_bits(y1))


def test_multi_repeat_and_back_to_back():
    # calls with changing activations share one workspace, back to back with
    # no host sync; each must equal the same call run alone, bit for bit
    import torch
    import gemm_exl3_linear_amd as X
    ts, _ = _tensors(1501, 1024, [(2048, 4), (512, 2), (1024, 6)], 1)
    ws_ = [G.weight(d) for d in ts]
    xs = [G.to_dev(synth.activations(synth.rng(1600 + i), 1, 1024)) for i in range(3)]
    alone = []
    for x in xs:
        alone.append([G.f16_bits(y) for y in X.exl3_linear_multi(x, ws_)])
        torch.cuda.synchronize()
    work = torch.zeros(X.exl3_linear_multi_workspace_size(ws_, 1), dtype=torch.uint8, device=G.dev())
    outs = [[torch.empty((1, d["n"]), dtype=torch.float16, device=G.dev()) for d in ts] for _ in range(12)]
    for c in range(12):
        X.exl3_linear_multi(xs[c % 3], ws_, outs=outs[c], workspace=work)
    torch.cuda.synchronize()
    for c in range(12):
        for i in range(len(ts)):
            np.testing.assert_array_equal(G.f16_bits(outs[c][i]), alone[c % 3][i], err_msg=f"call {c} tensor {i}")


@functools.lru_cache(maxsize=1)
def _layer():
    return synth.mixed_layer_inputs(synth.SEED_MIXED_LAYER, 1)


@pytest.mark.parametrize("group", [("q", "k", "v"), ("gate", "up")])
def test_multi_mixed_layer_groups_m1(group):
    lay = _layer()
    ts = [lay[nm] for nm in group]
    x = lay[group[0]]["x"]  # the projections of a group read one input
    ys = _run_multi(ts, x)
    for nm, d, y in zip(group, ts, ys):
        ref = O.linear(x, d["trellis"], d["suh"], d["svh"], d["bits"])
        err = O.rel_frobenius(y.double().cpu().numpy(), ref)
        assert err < TOL, (nm, d["bits"], err)


def test_multi_negation_bit_exact():
    # The several-tensor call contracts one row on the vector units (v_dot2,
    # fp32 round to nearest even), and every step (input transform, products,
    # the -1534 * sum(x') correction, the fixed-order slot sums, the output
    # transform, svh, the fp16 cast) is symmetric under negation: y(-x) is
    # -y(x) bit for bit.
    ts, x = _tensors(740, 1024, [(640, 3), (384, 5)], 1)
    y = _run_multi(ts, x)
    yn = _run_multi(ts, -x)
    for a, b in zip(y, yn):
        np.testing.assert_array_equal(G.f16_bits(b), G.f16_bits(-a))
