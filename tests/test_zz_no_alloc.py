"""exl3_linear_no_workspace (the entry point for callers that cannot
allocate) against exl3_linear with a caller workspace, through the C ABI:
bit-identical outputs, on two calls in a row with the second one smaller,
for the decode GEMV (one row, both contraction paths) and the prefill GEMM,
and the refusal of a call whose workspace exceeds the library's array."""
import numpy as np
import pytest

import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _pair(d, m, out_dtype):
    import torch
    import gemm_exl3_linear_amd as X
    w = G.weight(d)
    x = G.to_dev(d["x"][:m])
    y_ref = X.exl3_linear(x, w, out_dtype=out_dtype)
    y = torch.full((m, d["n"]), float("nan"), dtype=out_dtype, device=G.dev())
    X.exl3_linear_no_workspace(x, w, out=y)
    torch.cuda.synchronize()
    return y, y_ref


@pytest.mark.parametrize("k,n,bits,m1,m2", [
    (5120, 17408, 4, 16, 1),    # decode GEMV: matrix cores, then one row on v_dot2
    (17408, 5120, 8, 4, 2),     # v_dot2 rows, a deep k
    (2048, 512, 3, 300, 40),    # prefill GEMM, then a shorter one
    (1024, 384, 5, 40, 5),      # GEMM, then the GEMV
])
@pytest.mark.parametrize("f32", [False, True])
def test_no_workspace_matches_exl3_linear(k, n, bits, m1, m2, f32):
    import torch
    dt = torch.float32 if f32 else torch.float16
    d = synth.linear_inputs(1300 + bits, m1, k, n, bits)
    for m in (m1, m2):
        y, y_ref = _pair(d, m, dt)
        assert torch.equal(y.view(torch.int16 if not f32 else torch.int32),
                           y_ref.view(torch.int16 if not f32 else torch.int32)), (k, n, bits, m)


def test_no_workspace_refuses_calls_past_its_array():
    import torch
    import gemm_exl3_linear_amd as X
    d = synth.linear_inputs(1310, 4096, 5120, 17408, 1)
    w = G.weight(d)
    assert X.exl3_linear_workspace_size(w, 4096) > X.SCRATCH_BYTES
    x = G.to_dev(d["x"])
    y = torch.zeros((4096, 17408), dtype=torch.float16, device=G.dev())
    with pytest.raises(X.Exl3Error) as ei:
        X.exl3_linear_no_workspace(x, w, out=y)
    assert ei.value.status == X.EXL3_E_WORKSPACE
    torch.cuda.synchronize()
    assert (y == 0).all()
    # a smaller call on the same array right after is unaffected
    y1, y1_ref = _pair(d, 3, torch.float16)
    np.testing.assert_array_equal(G.f16_bits(y1), G.f16_bits(y1_ref))
