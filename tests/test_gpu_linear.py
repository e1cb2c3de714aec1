"""GPU parity of exl3_linear against the float64 oracle (relative Frobenius
error <= 2e-3 over the whole output), plus the invariants the arithmetic makes
bit-exact on the GPU."""
import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _run(d, m=None, out_dtype=None, bias=None):
    import torch
    import gemm_exl3_linear_amd as X
    x = d["x"] if m is None else d["x"][:m]
    y = X.exl3_linear(G.to_dev(x), G.weight(d, bias=bias), out_dtype=out_dtype or torch.float16)
    torch.cuda.synchronize()
    return y


def _ref(d, m=None, bias=None, W=None):
    x = d["x"] if m is None else d["x"][:m]
    return O.linear(x, d["trellis"], d["suh"], d["svh"], d["bits"], bias=bias, w_decoded=W)


def test_single_tensor_2048x512_k4_m1():
    d = G.linear_case(synth.SEED_SINGLE_2048x512, 1, 2048, 512, 4)
    y = _run(d)
    err = O.rel_frobenius(y.double().cpu().numpy(), _ref(d, W=G.decoded(synth.SEED_SINGLE_2048x512, 1, 2048, 512, 4)))
    assert err < TOL, err


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 16])
def test_gemv_all_widths(bits, m):
    d = synth.linear_inputs(200 + bits, m, 1024, 384, bits)
    y = _run(d)
    err = O.rel_frobenius(y.double().cpu().numpy(), _ref(d))
    assert err < TOL, err


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("m", [17, 64, 100, 300])
def test_gemm_ragged_rows(bits, m):
    d = synth.linear_inputs(300 + bits, m, 512, 256, bits)
    y = _run(d)
    err = O.rel_frobenius(y.double().cpu().numpy(), _ref(d))
    assert err < TOL, err


@pytest.mark.parametrize("m", [1, 5, 40])
def test_fp32_output_and_bias(m):
    import torch
    d = synth.linear_inputs(400 + m, m, 256, 512, 4)
    bias = np.linspace(-2, 2, 512).astype(np.float16)
    y = _run(d, out_dtype=torch.float32, bias=bias)
    assert y.dtype == torch.float32
    err = O.rel_frobenius(y.double().cpu().numpy(), _ref(d, bias=bias))
    assert err < TOL, err


def test_empty_batch_is_noop():
    import torch
    import gemm_exl3_linear_amd as X
    d = synth.linear_inputs(1, 1, 128, 128, 4)
    y = torch.full((0, 128), 7.0, dtype=torch.float16, device=G.dev())
    X.exl3_linear(G.to_dev(d["x"][:0]), G.weight(d), out=y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("m", [1, 4, 16, 40])
def test_sign_invariances_bit_exact(m):
    import torch
    d = synth.linear_inputs(500 + m, m, 512, 384, 4)
    y = _run(d)
    d2 = dict(d)
    d2["x"] = d["x"].copy(); d2["suh"] = d["suh"].copy()
    d2["x"][:, 11] = -d2["x"][:, 11]; d2["suh"][11] = -d2["suh"][11]
    np.testing.assert_array_equal(G.f16_bits(_run(d2)), G.f16_bits(y))
    d3 = dict(d); d3["svh"] = d["svh"].copy(); d3["svh"][5] = -d3["svh"][5]
    y3 = _run(d3)
    assert torch.equal(y3[:, 5], -y[:, 5])
    keep = [c for c in range(384) if c != 5]
    assert torch.equal(y3[:, keep], y[:, keep])


@pytest.mark.parametrize("m", [1, 2, 4])
def test_negation_bit_exact_dot_path(m):
    # y(-x) = -y(x) bit for bit where the rows contract on the vector units:
    # every step (input transform, v_dot2 with round-to-nearest, the fma with
    # the segment's sum of x', fixed-order slot sums, output transform, svh,
    # fp16 cast) is odd in x.  Compared as values: a zero stays +0.
    d = synth.linear_inputs(510 + m, m, 1024, 640, 3)
    y = _run(d).float().cpu().numpy()
    d4 = dict(d); d4["x"] = -d["x"]
    np.testing.assert_array_equal(_run(d4).float().cpu().numpy(), -y)


@pytest.mark.parametrize("m", [16, 40])
def test_negation_matrix_core_paths(m):
    # On the matrix cores the identity holds to one fp16 ulp, not bit for bit:
    # the fp16 MFMA's internal sum of products does not round symmetrically
    # in sign.
    d = synth.linear_inputs(520 + m, m, 512, 384, 4)
    y = _run(d).double().cpu().numpy()
    d4 = dict(d); d4["x"] = -d["x"]
    yn = _run(d4).double().cpu().numpy()
    assert (np.abs(yn + y) <= O.fp16_ulp(y)).all()


@pytest.mark.parametrize("m", [1, 7, 33])
def test_constant_trellis_exact_zeros(m):
    d = synth.linear_inputs(600 + m, m, 384, 256, 4)
    d = dict(d); d["trellis"] = np.zeros_like(d["trellis"])
    y = _run(d).float().cpu().numpy()
    mask = np.ones(256, bool); mask[::128] = False
    assert (y[:, mask] == 0).all()
    err = O.rel_frobenius(y, _ref(d))
    assert err < TOL, err


def test_row_invariance_gemv():
    # Within each contraction path, v_dot2 (1 <= m <= 4) and the matrix cores
    # (5 <= m <= 16), every row equals the same row of any other call, bit for
    # bit: the plan depends on (k, n) and the path only, and a row's sums on
    # its own activations only.  Across the two paths the fp32 rounding order
    # differs, so there the rows agree to one fp16 ulp.
    d = synth.linear_inputs(700, 16, 1024, 512, 4)
    y16t = _run(d)
    y16 = G.f16_bits(y16t)
    for m in (5, 9):
        np.testing.assert_array_equal(G.f16_bits(_run(d, m=m)), y16[:m])
    y4t = _run(d, m=4)
    y4 = G.f16_bits(y4t)
    for m in (1, 2, 3):
        np.testing.assert_array_equal(G.f16_bits(_run(d, m=m)), y4[:m])
    ref = y16t[:4].float()
    ulp = ref.abs().clamp(min=2.0 ** -14) * 2.0 ** -10
    assert ((y4t.float() - ref).abs() <= ulp).all()


def test_row_invariance_gemm():
    d = synth.linear_inputs(701, 300, 512, 256, 3)
    y = G.f16_bits(_run(d))
    ys = G.f16_bits(_run(d, m=20))
    np.testing.assert_array_equal(ys, y[:20])


def test_repeat_bit_identical():
    d = synth.linear_inputs(702, 4, 2048, 1024, 4)
    a = G.f16_bits(_run(d))
    for _ in range(5):
        np.testing.assert_array_equal(G.f16_bits(_run(d)), a)


# --- full-size workloads, in the launch configuration the benchmark times ---
@pytest.mark.parametrize("m", [1, 4, 16])
def test_dense_decode_5120x17408_k4(m):
    d = G.linear_case(synth.SEED_DENSE_5120x17408, 16, 5120, 17408, 4)
    y = _run(d, m=m)
    W = G.decoded(synth.SEED_DENSE_5120x17408, 16, 5120, 17408, 4)
    G.assert_parity(y.double().cpu().numpy(), _ref(d, m=m, W=W), what=f"m={m}")


# single Hadamard blocks and very uneven shapes: one 128-column block over a
# deep k (every wave of the decode GEMV's plan in one block), one k block
# over a wide n (runs shorter than a block), and a lone 128 x 128 tensor
@pytest.mark.parametrize("k,n", [(128, 128), (128, 17408), (5120, 128), (256, 128), (128, 384)])
@pytest.mark.parametrize("m", [1, 3, 5, 16, 17, 64, 300])
def test_single_block_shapes(k, n, m):
    d = synth.linear_inputs(1000 + k // 128 + n // 128 + m, m, k, n, 3 + (m % 4))
    y = _run(d).double().cpu().numpy()
    G.assert_parity(y, _ref(d), what=f"{k}x{n} m={m}")


@pytest.mark.parametrize("k,n,bits", [(4096, 8192, 3), (3072, 12288, 5)])
def test_single_row_two_tier_runs(k, n, bits):
    # On the v_dot2 path a grid of more than one wave per SIMD gives the
    # first-round waves longer runs than the rest; these shapes put the tier
    # boundary and the run ends at other places in the 128-column blocks than
    # the 5120 x 17408 workload does.  Row 0 of the same call at m == 8 (equal
    # runs, matrix cores) sums the same fp32 products in another order: the
    # two agree to one fp16 ulp of the value plus 2^-11 of the row's rms,
    # while a partial slot lost or counted twice would move a whole 128-column
    # block by several percent of the rms.
    d = synth.linear_inputs(710 + bits, 8, k, n, bits)
    y1 = _run(d, m=1)
    err = O.rel_frobenius(y1.double().cpu().numpy(), _ref(d, m=1))
    assert err < TOL, err
    ref = _run(d)[:1].float()
    rms = ref.pow(2).mean().sqrt()
    tol = ref.abs() * 2.0 ** -10 + rms * 2.0 ** -11
    assert ((y1.float() - ref).abs() <= tol).all()


def test_dense_prefill_4096x5120x17408_k4_all_rows():
    d = G.linear_case(synth.SEED_PREFILL_4096x5120x17408, 4096, 5120, 17408, 4)
    y = _run(d).double().cpu().numpy()
    W = G.decoded(synth.SEED_PREFILL_4096x5120x17408, 4096, 5120, 17408, 4)
    G.assert_parity(y, G.linear_ref(d, W=W), what="4096x5120x17408")


def test_workspace_reused_across_sizes():
    # one zero-filled workspace serves GEMV and GEMM calls in any order: the
    # arrival counters are left at zero by every call
    import torch
    import gemm_exl3_linear_amd as X
    d = synth.linear_inputs(703, 40, 512, 384, 4)
    w = G.weight(d)
    need = max(X.exl3_linear_workspace_size(w, m) for m in (1, 16, 40))
    ws = torch.zeros(need, dtype=torch.uint8, device=G.dev())
    ref = {m: G.f16_bits(_run(d, m=m)) for m in (1, 16, 40)}
    for m in (1, 40, 16, 1, 16, 40, 1):
        y = X.exl3_linear(G.to_dev(d["x"][:m]), w, workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(G.f16_bits(y), ref[m])
    assert X.exl3_linear_workspace_size(w, 1) <= need


@pytest.mark.parametrize("m", [1, 16, 40])
def test_back_to_back_calls_changing_weights(m):
    # Calls share one workspace and run back to back with no host sync while
    # the weights change every call: a result that picked up a partial sum
    # left by the previous call (stale cache line) would differ from the same
    # call run alone.  5120 x 17408 spreads every block over many waves, so
    # the slots of one block come from several XCDs.
    import torch
    import gemm_exl3_linear_amd as X
    k, n, bits, copies, calls = 5120, 17408, 4, 4, 24
    ds = [synth.linear_inputs(900 + c, m, k, n, bits) for c in range(copies)]
    ws_ = [G.weight(d) for d in ds]
    x = G.to_dev(ds[0]["x"])
    alone = []
    for w in ws_:
        alone.append(G.f16_bits(X.exl3_linear(x, w)))
        torch.cuda.synchronize()
    ws = torch.zeros(X.exl3_linear_workspace_size(ws_[0], m), dtype=torch.uint8, device=G.dev())
    ys = torch.empty((calls, m, n), dtype=torch.float16, device=G.dev())
    for i in range(calls):
        X.exl3_linear(x, ws_[i % copies], out=ys[i], workspace=ws)
    torch.cuda.synchronize()
    got = G.f16_bits(ys)
    for i in range(calls):
        np.testing.assert_array_equal(got[i], alone[i % copies], err_msg=f"call {i}")
