"""GPU: exl3_reconstruct is bit-exact against the oracle's decode (every width),
and exl3_hadamard matches the oracle's transform."""
import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("k,n", [(16, 16), (48, 80), (256, 384)])
def test_reconstruct_bit_exact(bits, k, n):
    import gemm_exl3_linear_amd as X
    d = synth.linear_inputs(1000 + bits, 1, k, n, bits)
    W = X.exl3_reconstruct(G.weight(d))
    ref = O.decode_tensor(d["trellis"], bits)
    np.testing.assert_array_equal(G.f16_bits(W), ref.view(np.uint16))


def test_reconstruct_full_size_single_tensor():
    # 2048 x 512, K=4: the parity tensor, decoded in full
    import gemm_exl3_linear_amd as X
    d = G.linear_case(synth.SEED_SINGLE_2048x512, 1, 2048, 512, 4)
    W = X.exl3_reconstruct(G.weight(d))
    np.testing.assert_array_equal(G.f16_bits(W), G.decoded(synth.SEED_SINGLE_2048x512, 1, 2048, 512, 4).view(np.uint16))


@pytest.mark.parametrize("fill", [0x0000, 0xFFFF, 0x8000])
def test_reconstruct_constant_trellis(fill):
    import gemm_exl3_linear_amd as X
    d = synth.linear_inputs(7, 1, 128, 128, 4)
    d["trellis"] = np.full_like(d["trellis"], fill)
    W = X.exl3_reconstruct(G.weight(d))
    np.testing.assert_array_equal(G.f16_bits(W), O.decode_tensor(d["trellis"], 4).view(np.uint16))


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("rows,dim", [(1, 128), (5, 384), (33, 5120)])
def test_hadamard_matches_oracle(dtype, rows, dim):
    import torch
    import gemm_exl3_linear_amd as X
    g = np.random.default_rng(rows * 7 + dim)
    x = g.standard_normal((rows, dim)).astype(np.float16 if dtype == "f16" else np.float32)
    sb = synth.signs(g, dim)
    sa = synth.signs(g, dim)
    xd = G.to_dev(x)
    for b, a in ((sb, sa), (sb, None), (None, sa), (None, None)):
        out = X.exl3_hadamard(xd, None if b is None else G.to_dev(b), None if a is None else G.to_dev(a))
        ref = O.hadamard(x.astype(np.float64), sign_before=b, sign_after=a)
        err = O.rel_frobenius(out.double().cpu().numpy(), ref)
        assert err < (1e-3 if dtype == "f16" else 1e-6), err


def test_hadamard_strided_in_place_round_trip():
    import torch
    import gemm_exl3_linear_amd as X
    g = np.random.default_rng(3)
    buf = torch.zeros((6, 640), dtype=torch.float32, device=G.dev())
    x = torch.from_numpy(g.standard_normal((6, 512)).astype(np.float32)).to(G.dev())
    buf[:, :512] = x
    view = buf[:, :512]
    s = G.to_dev(synth.signs(g, 512))
    X.exl3_hadamard(view, sign_before=s, out=view)        # in place, ld = 640
    X.exl3_hadamard(view, sign_after=s, out=view)
    torch.cuda.synchronize()
    np.testing.assert_allclose(view.cpu().numpy(), x.cpu().numpy(), atol=2e-6)
    assert (buf[:, 512:] == 0).all()
