"""GPU parity of the int8 prefill path (exl3_linear_int8, exl3_reconstruct_int8)
against the float64 oracle's int8 readings.

Tolerances: the int8 weights are integers from integers, so they must match
bit for bit.  The layer output differs from the oracle's int8 layer only by
fp32 arithmetic (x' and the scales), the rare activation code that fp32 puts
on the other side of a rounding boundary, and the output cast: relative
Frobenius error <= 1e-3 (TOL8).  Against the fp16-weight layer the int8
rounding itself costs about 1e-2 (the oracle's own pin bounds it by 2e-2).
"""
import functools

import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
TOL8 = 1e-3
TOL_VS_FP16 = 2e-2


def _run8(d, m=None, out_dtype=None, bias=None, x=None):
    import torch
    import gemm_exl3_linear_amd as X
    if x is None:
        x = d["x"] if m is None else d["x"][:m]
    y = X.exl3_linear_int8(G.to_dev(x), G.weight(d, bias=bias), out_dtype=out_dtype or torch.float16)
    torch.cuda.synchronize()
    return y


@functools.lru_cache(maxsize=4)
def _wq(seed, m, k, n, bits):
    d = G.linear_case(seed, m, k, n, bits)
    return O.decode_tensor_int8(d["trellis"], bits)


@pytest.mark.parametrize("bits", range(1, 9))
def test_reconstruct_int8_bit_exact(bits):
    import torch
    import gemm_exl3_linear_amd as X
    d = synth.linear_inputs(800 + bits, 1, 64, 96, bits)
    q = X.exl3_reconstruct_int8(G.weight(d))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), O.decode_tensor_int8(d["trellis"], bits))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("m", [1, 70, 300, 700, 1030])
def test_linear_int8_parity(bits, m):
    # several 128-column blocks, k of several 64-row steps, ragged 64-row
    # tiles (three column tiles make too small a grid for taller ones) and a
    # last 16-row group of the fragment-major activations that is only
    # partly filled
    d = G.linear_case(810 + bits, 1030, 512, 384, bits)
    y = _run8(d, m=m).double().cpu().numpy()
    ref = O.linear_int8(d["x"][:m], d["trellis"], d["suh"], d["svh"], bits, wq=_wq(810 + bits, 1030, 512, 384, bits))
    assert O.rel_frobenius(y, ref) < TOL8
    ref16 = O.linear(d["x"][:m], d["trellis"], d["suh"], d["svh"], bits)
    assert O.rel_frobenius(y, ref16) < TOL_VS_FP16


# 128 column tiles: m = 100 and 300 take 128-row tiles (one or three), m =
# 600 256-row tiles (three, the last ragged); 64-row tiles are the narrow
# tensors' above
@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("m", [100, 300, 600])
def test_linear_int8_each_tile_height(bits, m):
    d = G.linear_case(830 + bits, m, 256, 16384, bits)
    y = _run8(d, m=m).double().cpu().numpy()
    ref = O.linear_int8(d["x"], d["trellis"], d["suh"], d["svh"], bits, wq=_wq(830 + bits, m, 256, 16384, bits))
    assert O.rel_frobenius(y, ref) < TOL8


def test_linear_int8_fp32_output_and_bias():
    import torch
    d = G.linear_case(820, 130, 384, 256, 4)
    bias = (np.arange(256) % 11 - 5).astype(np.float16) * np.float16(0.25)
    y = _run8(d, out_dtype=torch.float32, bias=bias).double().cpu().numpy()
    ref = O.linear_int8(d["x"], d["trellis"], d["suh"], d["svh"], 4, bias=bias)
    assert O.rel_frobenius(y, ref) < TOL8


def test_linear_int8_rows_independent_bit_exact():
    # each row is quantized and contracted on its own: any prefix of the
    # batch gives the same rows, and m = 1 equals the row of a full batch,
    # whichever tile height serves it
    d = G.linear_case(821, 700, 512, 256, 3)
    full = G.f16_bits(_run8(d))
    for m in (1, 20, 129, 300, 512):
        np.testing.assert_array_equal(G.f16_bits(_run8(d, m=m)), full[:m])


@pytest.mark.parametrize("k", [512, 5120, 5248])
def test_linear_int8_quant_shapes_agree(k):
    # from 2048 rows on the activations are quantized by 16-row groups (rows
    # of up to 40 blocks held in registers, one wave per row; longer rows two
    # waves each, eight rows per workgroup), below that one row per
    # workgroup; all do the same arithmetic, so the rows of a short batch
    # equal those of a long one bit for bit, and the long batch (2050 rows:
    # its last group is two rows) matches the oracle.  k = 5120 fills the
    # held rows exactly, 5248 is the first width past them.
    d = G.linear_case(826 + k // 128, 2050, k, 256, 3)
    full = _run8(d)
    np.testing.assert_array_equal(G.f16_bits(_run8(d, m=1000)), G.f16_bits(full)[:1000])
    rows = np.r_[0:8, 1020:1030, 2040:2050]
    y = full.double().cpu().numpy()[rows]
    ref = O.linear_int8(d["x"][rows], d["trellis"], d["suh"], d["svh"], 3)
    assert O.rel_frobenius(y, ref) < TOL8


def test_linear_int8_sign_and_zero_rows():
    import torch
    d = G.linear_case(822, 96, 256, 384, 5)
    x = d["x"].copy()
    x[7] = 0
    y = _run8(d, x=x)
    yn = _run8(d, x=-x)
    # x -> -x negates every code and keeps every scale: y(-x) = -y(x) exactly
    # (compared as values: an exact zero stays +0 on both sides)
    np.testing.assert_array_equal(yn.float().cpu().numpy(), -y.float().cpu().numpy())
    assert (y[7].float() == 0).all()
    # an all-zero row gives exactly the bias
    bias = (np.arange(384) % 5 - 2).astype(np.float16)
    yb = _run8(d, x=x, out_dtype=torch.float32, bias=bias)
    np.testing.assert_array_equal(yb[7].cpu().numpy(), bias.astype(np.float32))


@pytest.mark.parametrize("fill", [0x0000, 0xFFFF])
def test_linear_int8_constant_trellis_exact_zeros(fill):
    # W_q is one value everywhere, so every column of a 128-column block gets
    # the same int32 sum and the output transform leaves exact zeros off the
    # block's first column (closed form of the oracle's pin)
    d = dict(G.linear_case(823, 70, 256, 256, 4))
    d["trellis"] = np.full_like(d["trellis"], fill)
    y = _run8(d).float().cpu().numpy()
    mask = np.ones(256, bool)
    mask[::128] = False
    assert (y[:, mask] == 0).all()
    ref = O.linear_int8(d["x"], d["trellis"], d["suh"], d["svh"], 4)
    assert O.rel_frobenius(y, ref) < TOL8


def test_linear_int8_workspace_reused_across_sizes():
    import torch
    import gemm_exl3_linear_amd as X
    d = G.linear_case(824, 300, 384, 256, 2)
    w = G.weight(d)
    ws = torch.empty(X.exl3_linear_int8_workspace_size(w, 300), dtype=torch.uint8, device=G.dev())
    a = X.exl3_linear_int8(G.to_dev(d["x"]), w, workspace=ws)
    b = X.exl3_linear_int8(G.to_dev(d["x"][:33]), w, workspace=ws)
    c = X.exl3_linear_int8(G.to_dev(d["x"]), w, workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(G.f16_bits(b), G.f16_bits(a)[:33])
    np.testing.assert_array_equal(G.f16_bits(c), G.f16_bits(a))


# --- the full-size prefill workload, in the launch configuration the benchmark times ---
def test_int8_prefill_4096x5120x17408_k4_all_rows():
    d = G.linear_case(synth.SEED_PREFILL_4096x5120x17408, 4096, 5120, 17408, 4)
    y = _run8(d).double().cpu().numpy()
    wq = _wq(synth.SEED_PREFILL_4096x5120x17408, 4096, 5120, 17408, 4)
    G.assert_parity(y, G.linear_int8_ref(d, Wq=wq), tol=TOL8, what="int8 vs int8 oracle")
    W = G.decoded(synth.SEED_PREFILL_4096x5120x17408, 4096, 5120, 17408, 4)
    assert O.rel_frobenius(y, G.linear_ref(d, W=W)) < TOL_VS_FP16
