"""Graph capture of the library's calls (exl3xpu README, "Layout": the decode
path runs under graph capture, "cudagraph FULL_DECODE_ONLY").

Every entry point only enqueues kernels on the caller's stream (no memset, no
host synchronisation, no allocation), so a call can be captured into a graph
and replayed.  Each case: compute the result eagerly, capture the same call
into a graph, then replay it several times with other eager library calls and
synchronisations in between; before each replay the output is cleared
eagerly, and after it the output must equal the eager result bit for bit (the
kernels' summation order does not depend on timing).  The routed-expert
small-batch path keeps arrival counters in its workspace, which every call
leaves at zero; replays after eager calls on the same workspace check that.
"""
import numpy as np
import pytest

import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu
REPLAYS = 4


def _check_graph(run, outs, interleave):
    """run(): enqueue the call on the current stream, writing the tensors
    `outs`.  interleave(i): eager work between replays."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager reference and warm-up off the default stream
        run()
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o in outs:
            o.zero_()
        interleave(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {i} differs"


def _other_linear():
    """An unrelated eager call of the library, to run between replays."""
    import torch
    import gemm_exl3_linear_amd as X
    d = G.linear_case(900, 20, 512, 256, 5)
    w = G.weight(d)
    x = G.to_dev(d["x"])

    def go(i):
        X.exl3_linear(x[: 1 + (i % 2) * 19], w)
        torch.cuda.synchronize()
    return go


@pytest.mark.parametrize("m", [1, 4, 8, 300])
def test_graph_linear(m):
    # m = 1, 4: the decode GEMV with every wave staging its own x' and the
    # finish forming the workgroup terms; m = 8: the input-transform launch
    # and the workgroup combine in LDS; m = 300: the prefill GEMM
    import torch
    import gemm_exl3_linear_amd as X
    d = G.linear_case(901, 300, 4096, 4096, 4)
    w = G.weight(d)
    x = G.to_dev(d["x"][:m])
    y = torch.empty((m, 4096), dtype=torch.float16, device=G.dev())
    ws = torch.zeros(X.exl3_linear_workspace_size(w, m), dtype=torch.uint8, device=G.dev())
    _check_graph(lambda: X.exl3_linear(x, w, out=y, workspace=ws), [y], _other_linear())


def test_graph_linear_int8():
    import torch
    import gemm_exl3_linear_amd as X
    d = G.linear_case(902, 300, 1024, 512, 3)
    w = G.weight(d)
    x = G.to_dev(d["x"])
    y = torch.empty((300, 512), dtype=torch.float32, device=G.dev())
    ws = torch.empty(X.exl3_linear_int8_workspace_size(w, 300), dtype=torch.uint8, device=G.dev())
    _check_graph(lambda: X.exl3_linear_int8(x, w, out=y, workspace=ws), [y], _other_linear())


def test_graph_linear_multi():
    import torch
    import gemm_exl3_linear_amd as X
    shapes = [(2048, 2048, 5), (2048, 512, 2), (2048, 512, 8)]
    ws_, outs = [], []
    for i, (k, n, bits) in enumerate(shapes):
        d = synth.linear_inputs(903 + i, 1, k, n, bits)
        ws_.append(G.weight(d))
        outs.append(torch.empty((1, n), dtype=torch.float16, device=G.dev()))
    x = G.to_dev(synth.linear_inputs(906, 1, 2048, 128, 2)["x"])
    wsp = torch.zeros(X.exl3_linear_multi_workspace_size(ws_, 1), dtype=torch.uint8, device=G.dev())
    _check_graph(lambda: X.exl3_linear_multi(x, ws_, outs=outs, workspace=wsp), outs, _other_linear())


@pytest.mark.parametrize("tt", [1, 200])
def test_graph_grouped_experts(tt):
    # tt = 1: the per-(token, slot) unit path with its arrival counters;
    # tt = 200 (800 (token, slot) pairs at top-4): the binned grouped GEMM path
    import torch
    import gemm_exl3_linear_amd as X
    m = synth.moe_inputs(907 + tt, tt, experts=16, topk=4, hidden=256, inter=128, bits=3)
    gu = X.Exl3Arena.from_numpy(m["gate_up"], G.dev())
    dn = X.Exl3Arena.from_numpy(m["down"], G.dev())
    x = G.to_dev(m["x"])
    ids = G.to_dev(m["ids"].astype(np.int32))
    wt = G.to_dev(m["weights"].astype(np.float32))
    y = torch.empty((tt, 256), dtype=torch.float32, device=G.dev())
    ws = torch.zeros(X.exl3_grouped_experts_workspace_size(gu, dn, tt, 4), dtype=torch.uint8, device=G.dev())

    def between(i):
        # eager calls on the same workspace, then the next replay
        X.exl3_grouped_experts(x, ids, wt, gu, dn, workspace=ws)
        torch.cuda.synchronize()
    _check_graph(lambda: X.exl3_grouped_experts(x, ids, wt, gu, dn, out=y, workspace=ws), [y], between)


@pytest.mark.parametrize("tt", [1, 200])
def test_graph_grouped_experts_mixed_widths(tt):
    # a width per expert: one launch per width and projection, the token
    # slots of the unit path arriving over several of them
    import torch
    import gemm_exl3_linear_amd as X
    m = synth.moe_mixed_inputs(909 + tt, tt, experts=16, topk=4, hidden=256, inter=128, widths=(2, 3, 5))
    gu = X.Exl3MixedArena.from_numpy(m["gate_up"], G.dev())
    dn = X.Exl3MixedArena.from_numpy(m["down"], G.dev())
    x = G.to_dev(m["x"])
    ids = G.to_dev(m["ids"].astype(np.int32))
    wt = G.to_dev(m["weights"].astype(np.float32))
    y = torch.empty((tt, 256), dtype=torch.float32, device=G.dev())
    ws = torch.zeros(X.exl3_grouped_experts_mixed_workspace_size(gu, dn, tt, 4), dtype=torch.uint8,
                     device=G.dev())

    def between(i):
        X.exl3_grouped_experts_mixed(x, ids, wt, gu, dn, workspace=ws)
        torch.cuda.synchronize()
    _check_graph(lambda: X.exl3_grouped_experts_mixed(x, ids, wt, gu, dn, out=y, workspace=ws), [y], between)
