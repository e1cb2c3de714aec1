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


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("m", [17, 64, 100, 300])
def test_gemm_ragged_rows(bits, m):
    d = synth.linear_inputs(300 + bits, m, 512, 256, bits)
    y = _run(d)
    err = O.rel_frobenius(y.double().cpu().numpy(), _ref(d))
    assert err < TOL, err


# 128 column tiles: m = 100 and 300 take 128-row tiles (one or three), m =
# 600 256-row tiles (three, the last ragged); 64-row tiles are the narrow
# tensors' above
@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("m", [100, 300, 600])
def test_gemm_each_tile_height(bits, m):
    d = synth.linear_inputs(320 + bits, m, 256, 16384, bits)
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


@pytest.mark.parametrize("m", [1, 2, 4, 5, 16, 40])
def test_negation_within_one_ulp(m):
    # y(-x) = -y(x) to one fp16 ulp.  Every row count contracts on the
    # matrix cores (the decode GEMV for m <= 16, the GEMM above), and the
    # fp16 MFMA's sum of products does not round symmetrically in sign
    # (test_mfma_sum_is_not_sign_symmetric), so the identity is not bit-exact.
    d = synth.linear_inputs(520 + m, m, 512, 384, 4)
    y = _run(d).double().cpu().numpy()
    d4 = dict(d); d4["x"] = -d["x"]
    yn = _run(d4).double().cpu().numpy()
    assert (np.abs(yn + y) <= O.fp16_ulp(y)).all()


def test_mfma_sum_is_not_sign_symmetric():
    # The evidence for the one-ulp allowance above: four chained
    # v_mfma_f32_16x16x16_f16 (each accumulating into the last, as the decode
    # accumulates over k) alone, on random fp16 activations against biased
    # codes 1024..2044 like the decode's, with every A and with every A
    # negated.  Most outputs are exact negations, some differ in their last
    # bits, none by more than a few fp32 ulps.
    import torch
    L = G.bench_lib()
    rng = np.random.default_rng(30)
    P = 2048
    a = (rng.standard_normal((P, 4, 64, 4)) * np.exp2(rng.integers(-4, 4, (P, 4, 64, 4)))).astype(np.float16)
    b = (rng.integers(1024, 2045, (P, 4, 64, 4))).astype(np.float16)
    da, db = G.to_dev(a), G.to_dev(b)
    out = torch.empty((P, 2, 64, 4), dtype=torch.float32, device=G.dev())
    assert L.exl3_bench_mfma_negation(da.data_ptr(), db.data_ptr(), out.data_ptr(), P, 0) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    pos, neg = o[:, 0], o[:, 1]
    differ = int(np.count_nonzero(pos != -neg))
    assert 0 < differ < pos.size // 10, f"{differ} of {pos.size} outputs differ from the exact negation"
    # the differences are rounding-sized: a few fp32 ulps of sum |a| |b|, the
    # magnitude the sum passes through (lane l holds A[l % 16][4 (l / 16) + i]
    # and B[4 (l / 16) + i][l % 16]; D[4 (l / 16) + i][l % 16] comes back in
    # lane l, element i)
    A = np.abs(a.astype(np.float64)).reshape(P, 4, 4, 16, 4).transpose(0, 1, 3, 2, 4).reshape(P, 4, 16, 16)
    B = np.abs(b.astype(np.float64)).reshape(P, 4, 4, 16, 4).transpose(0, 1, 2, 4, 3).reshape(P, 4, 16, 16)
    mag = np.einsum("pcmk,pckn->pmn", A, B)  # [P][m][n]
    mag_lanes = mag.reshape(P, 4, 4, 16).transpose(0, 1, 3, 2).reshape(P, 64, 4)
    assert (np.abs(pos + neg) <= 2.0 ** -20 * mag_lanes).all()


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
    # One contraction for every row count of the decode GEMV (1 <= m <= 16):
    # the plan depends on (k, n) only and a row's MFMA sums on its own
    # activations only, so every row equals the same row of any other call,
    # bit for bit, whether its x' came from the waves' own transform
    # (m <= 4) or from the input-transform launch (m > 4).
    d = synth.linear_inputs(700, 16, 1024, 512, 4)
    y16 = G.f16_bits(_run(d))
    for m in (1, 2, 3, 4, 5, 9, 15):
        np.testing.assert_array_equal(G.f16_bits(_run(d, m=m)), y16[:m], err_msg=f"m={m}")


@pytest.mark.parametrize("k,n,bits", [(5120, 17408, 4), (17408, 5120, 8), (2048, 640, 3)])
def test_row_invariance_gemv_large(k, n, bits):
    # the same at the workload shapes, rows 1, 4, 5 and 16, fp32 output
    import torch
    d = synth.linear_inputs(705 + bits, 16, k, n, bits)
    y16 = _run(d, out_dtype=torch.float32).cpu().numpy().view(np.uint32)
    for m in (1, 4, 5):
        got = _run(d, m=m, out_dtype=torch.float32).cpu().numpy().view(np.uint32)
        np.testing.assert_array_equal(got, y16[:m], err_msg=f"m={m}")


def test_row_invariance_gemm():
    d = synth.linear_inputs(701, 300, 512, 256, 3)
    y = G.f16_bits(_run(d))
    ys = G.f16_bits(_run(d, m=20))
    np.testing.assert_array_equal(ys, y[:20])


def test_input_transform_wide_grid_rows_agree():
    # from 8192 (16-row group, 128-column block) tasks on, the prefill input
    # transform gives each workgroup four blocks of its group; k = 640 has
    # five blocks, so every group's second workgroup holds one, and the last
    # group holds three rows (26243 = 16 x 1640 + 3).  Rows computed that way
    # equal the rows of a short batch (one block per workgroup) bit for bit,
    # and sampled rows match the oracle.
    d = synth.linear_inputs(703, 26243, 640, 128, 3)
    y = G.f16_bits(_run(d))
    np.testing.assert_array_equal(G.f16_bits(_run(d, m=2000)), y[:2000])
    rows = np.r_[0:4, 13107:13111, 26236:26243]
    d2 = dict(d); d2["x"] = d["x"][rows]
    got = y[rows].view(np.float16).astype(np.float64)
    assert O.rel_frobenius(got, _ref(d2)) < TOL


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


@pytest.mark.parametrize("k,n,bits", [(4096, 8192, 3), (3072, 12288, 5), (1024, 640, 2)])
def test_single_row_two_tier_runs(k, n, bits):
    # Runs come in two tiers (the first-round waves take longer ones); these
    # shapes put the tier boundary and the run ends at other places in the
    # 256-column pairs than the 5120 x 17408 workload does, and n = 640 ends
    # in a half pair.  m = 1 against the oracle, and bit for bit against row 0
    # of the same call at m = 8.
    d = synth.linear_inputs(710 + bits, 8, k, n, bits)
    y1 = _run(d, m=1)
    G.assert_parity(y1.double().cpu().numpy(), _ref(d, m=1), what=f"{k}x{n} K={bits}")
    np.testing.assert_array_equal(G.f16_bits(y1), G.f16_bits(_run(d))[:1])


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


def test_workspace_shared_with_multi_and_prefill():
    # one zero-filled workspace serves decode, fused several-tensor decode and
    # prefill calls interleaved, with the same bits as calls on their own
    import torch
    import gemm_exl3_linear_amd as X
    ds = [synth.linear_inputs(720 + i, 40, 1024, n, 3) for i, n in enumerate((17408, 384))]
    ws_ = [G.weight(d) for d in ds]
    x = G.to_dev(ds[0]["x"])
    need = max([X.exl3_linear_workspace_size(w, m) for w in ws_ for m in (1, 16, 40)] +
               [X.exl3_linear_multi_workspace_size(ws_, 1)])
    buf = torch.zeros(need, dtype=torch.uint8, device=G.dev())
    ref = {(i, m): G.f16_bits(X.exl3_linear(x[:m], w)) for i, w in enumerate(ws_) for m in (1, 16, 40)}
    ref_multi = [G.f16_bits(a) for a in X.exl3_linear_multi(x[:1], ws_)]
    torch.cuda.synchronize()
    for i, m in [(0, 1), (1, 40), (0, 16), (1, 1), (0, 40), (0, 1), (1, 16)]:
        y = X.exl3_linear(x[:m], ws_[i], workspace=buf)
        ym = X.exl3_linear_multi(x[:1], ws_, workspace=buf)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(G.f16_bits(y), ref[(i, m)])
        for a, r in zip(ym, ref_multi):
            np.testing.assert_array_equal(G.f16_bits(a), r)


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
