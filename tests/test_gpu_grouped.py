"""GPU parity of exl3_grouped_experts against the float64 oracle across
routing patterns, both regimes (per-pair units and grouped GEMM)."""
import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _run(m, ids=None, w=None):
    import torch
    import gemm_exl3_linear_amd as X
    ids = m["ids"] if ids is None else ids
    w = m["weights"] if w is None else w
    gu = X.Exl3Arena.from_numpy(m["gate_up"], G.dev())
    dn = X.Exl3Arena.from_numpy(m["down"], G.dev())
    y = X.exl3_grouped_experts(G.to_dev(m["x"]), G.to_dev(ids.astype(np.int32)),
                               G.to_dev(w.astype(np.float32)), gu, dn)
    torch.cuda.synchronize()
    return y.double().cpu().numpy()


def _ref(m, ids=None, w=None, tokens=None):
    ids = m["ids"] if ids is None else ids
    w = m["weights"] if w is None else w
    x = m["x"]
    if tokens is not None:
        x, ids, w = x[tokens], ids[tokens], w[tokens]
    return O.grouped_experts(x, ids, w, m["gate_up"], m["down"])


def _small(t, experts=16, topk=4, hidden=256, inter=128, bits=3, seed=40):
    return synth.moe_inputs(seed + t, t, experts=experts, topk=topk, hidden=hidden, inter=inter, bits=bits)


# The unit path serves t * topk <= 224 (token, slot) pairs, the binned grouped
# GEMM path larger calls; sizes on both sides of the threshold (topk = 4 here).
@pytest.mark.parametrize("t", [1, 2, 4, 16, 56, 57, 64, 96, 128, 300])
def test_random_routing(t):
    m = _small(t)
    err = O.rel_frobenius(_run(m), _ref(m))
    assert err < TOL, err


# 256-row tiles serve calls whose experts average at least 96 rows: one tile
# (t = 200 on 8 experts, ~100 rows each) or several with a short last one
# (t = 700, ~350 rows), so waves run with 1..4 of their four row groups
@pytest.mark.parametrize("t", [200, 700])
def test_random_routing_large_tiles(t):
    m = _small(t, experts=8, seed=47)
    err = O.rel_frobenius(_run(m), _ref(m))
    assert err < TOL, err


# hidden widths past one pass of the gate/up input transform (16 blocks of
# 128): 2176 takes a second pass with a single block, 4096 two full passes;
# both paths (t = 8: unit path, t = 200: binned)
@pytest.mark.parametrize("hidden", [2176, 4096])
@pytest.mark.parametrize("t", [8, 200])
def test_wide_hidden(t, hidden):
    m = _small(t, hidden=hidden, seed=52)
    err = O.rel_frobenius(_run(m), _ref(m))
    assert err < TOL, err


@pytest.mark.parametrize("t", [3, 40, 200, 700])
def test_all_tokens_same_experts(t):
    m = _small(t)
    ids = np.tile(np.array([5, 1, 9, 0], np.int32), (t, 1))
    err = O.rel_frobenius(_run(m, ids=ids), _ref(m, ids=ids))
    assert err < TOL, err


@pytest.mark.parametrize("t", [2, 33, 600])
def test_top1_unit_weight(t):
    m = _small(t, topk=1)
    w = np.ones((t, 1), np.float32)
    err = O.rel_frobenius(_run(m, w=w), _ref(m, w=w))
    assert err < TOL, err


@pytest.mark.parametrize("t", [2, 40, 200])
def test_zero_weights_exact_zero(t):
    m = _small(t)
    w = np.zeros_like(m["weights"])
    assert (_run(m, w=w) == 0).all()


@pytest.mark.parametrize("t", [24, 200])
def test_unused_expert_has_no_effect(t):
    m = _small(t, experts=64) if t > 100 else _small(t)
    used = set(np.unique(m["ids"]).tolist())
    unused = [e for e in range(m["gate_up"]["experts"]) if e not in used]
    y = _run(m)
    if unused:
        m2 = dict(m); m2["gate_up"] = dict(m["gate_up"]); m2["gate_up"]["trellis"] = m["gate_up"]["trellis"].copy()
        m2["gate_up"]["trellis"][unused[0]] ^= 0x3C3C
        np.testing.assert_array_equal(_run(m2), y)


def test_many_experts_binning_passes():
    # the binning keeps at most 8192 expert counters in LDS and takes the
    # experts in several passes beyond that: 8200 experts, with some pairs
    # routed past expert 8191
    m = _small(200, experts=8200, hidden=128, inter=128, bits=2, seed=48)
    ids = m["ids"].copy()
    for i in range(0, 200, 5):  # every fifth token: slot 0 to one of 8192..8199
        e = 8192 + (i // 5) % 8
        if e not in ids[i]:
            ids[i, 0] = e
    assert (ids >= 8192).sum() >= 30
    err = O.rel_frobenius(_run(m, ids=ids), _ref(m, ids=ids))
    assert err < TOL, err


@pytest.mark.parametrize("t", [1, 50])
def test_max_topk(t):
    m = _small(t, experts=32, topk=16)
    err = O.rel_frobenius(_run(m), _ref(m))
    assert err < TOL, err


@pytest.mark.parametrize("t", [1, 4, 64, 65])
def test_moe_256x2048x512_k3_small_t(t):
    m = synth.moe_inputs(synth.SEED_MOE_256x2048x512, t)
    err = O.rel_frobenius(_run(m), _ref(m))
    assert err < TOL, err


def test_moe_256x2048x512_k3_t4096_sampled_tokens():
    # every token on the GPU; the oracle on a seeded sample of 256 of them
    # (tokens are independent), each element within the per-element bound
    m = synth.moe_inputs(synth.SEED_MOE_256x2048x512, 4096)
    y = _run(m)
    tokens = np.sort(np.random.default_rng(1).choice(4096, 256, replace=False))
    G.assert_parity(y[tokens], G.grouped_ref(m, tokens=tokens), what="T=4096")


# Token-parallel path: workgroups planned on one XCD hand partial sums over
# through its L2; any workgroup found elsewhere takes a device-scope
# release/acquire hand-off.  Forcing that hand-off everywhere must give the
# same bits (and it is the path another dispatch order would take).
@pytest.mark.parametrize("t", [1, 4, 28])  # 28 x 8 = 224: the largest unit-path call
def test_forced_device_scope_hand_off_same_bits(t, monkeypatch):
    import gemm_exl3_linear_amd as X
    m = synth.moe_inputs(synth.SEED_MOE_256x2048x512, t)
    monkeypatch.delenv("EXL3_FORCE_DEVICE_SCOPE", raising=False)
    y0 = _run(m)
    monkeypatch.setenv("EXL3_FORCE_DEVICE_SCOPE", "1")
    y1 = _run(m)
    y2 = _run(m)
    np.testing.assert_array_equal(y1, y0)
    np.testing.assert_array_equal(y2, y0)
    monkeypatch.setenv("EXL3_FORCE_DEVICE_SCOPE", "0")
    np.testing.assert_array_equal(_run(m), y0)


# The XCD a group's workgroups are expected on is learned from the previous
# call: its finisher stores 1 + its XCD in bits 28..31 of the group's arrival
# counter (count fields zero).  The counter region starts the workspace: 224
# pairs x (intermediate / 128) gate/up groups, then 224 x (hidden / 128) down
# groups, one uint32 each.  Records that name the wrong XCD (planted here from
# the host), or work run on a second stream (which has been seen to rotate the
# dispatch of later launches by one XCD), change which hand-off the groups
# take, never the bits; after every call the count fields are zero again.
def _counter_words(ws, m):
    n = 224 * (m["gate_up"]["n"] // 128 + m["down"]["n"] // 128)
    return ws[:4 * n].view(dtype=__import__("torch").int32)


@pytest.mark.parametrize("t", [1, 4, 28])
def test_xcd_records_only_change_the_hand_off(t):
    import torch
    import gemm_exl3_linear_amd as X
    m = synth.moe_inputs(synth.SEED_MOE_256x2048x512, t)
    gu = X.Exl3Arena.from_numpy(m["gate_up"], G.dev())
    dn = X.Exl3Arena.from_numpy(m["down"], G.dev())
    x, ids, w = G.to_dev(m["x"]), G.to_dev(m["ids"].astype(np.int32)), G.to_dev(m["weights"].astype(np.float32))
    ws = torch.zeros(X.exl3_grouped_experts_workspace_size(gu, dn, t, 8), dtype=torch.uint8, device=G.dev())

    def call():
        y = X.exl3_grouped_experts(x, ids, w, gu, dn, workspace=ws)
        torch.cuda.synchronize()
        c = _counter_words(ws, m).cpu().numpy().view(np.uint32)
        assert not np.any(c & np.uint32((1 << 28) - 1)), "count fields left nonzero"
        assert np.all((c >> 28) <= 8)
        return G.f32_bits(y), c >> 28

    y0, rec = call()
    gu_used = t * 8 * (512 // 128)
    assert np.all((rec[:gu_used] >= 1) & (rec[:gu_used] <= 8)), "a finished group left no record"
    # records naming other XCDs than the ones found: every group off its expected XCD
    planted = torch.from_numpy(((((rec.astype(np.int64) + 2) % 8) + 1) << 28).astype(np.uint32).view(np.int32))
    _counter_words(ws, m).copy_(planted.to(G.dev()))
    y1, rec1 = call()
    np.testing.assert_array_equal(y1, y0)
    # work on a second stream, then the same call again
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        z = torch.zeros(1000, device=G.dev())
        z.add_(1)
    torch.cuda.synchronize()
    for _ in range(2):
        y2, _ = call()
        np.testing.assert_array_equal(y2, y0)


def test_check_ids_refuses_a_capturing_stream(monkeypatch):
    # EXL3_CHECK_IDS waits for a device count on the host, which a stream in
    # graph capture cannot do: the call returns EXL3_E_INVALID with nothing
    # enqueued and the capture ends valid
    import torch
    import gemm_exl3_linear_amd as X
    m = _small(3, seed=50)
    gu = X.Exl3Arena.from_numpy(m["gate_up"], G.dev())
    dn = X.Exl3Arena.from_numpy(m["down"], G.dev())
    x = G.to_dev(m["x"])
    ids = G.to_dev(m["ids"].astype(np.int32))
    w = G.to_dev(m["weights"].astype(np.float32))
    ws = torch.zeros(X.exl3_grouped_experts_workspace_size(gu, dn, 3, 4), dtype=torch.uint8, device=G.dev())
    y = torch.zeros((3, 256), dtype=torch.float32, device=G.dev())
    monkeypatch.setenv("EXL3_CHECK_IDS", "1")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        g.capture_begin()
        try:
            with pytest.raises(X.Exl3Error) as ei:
                X.exl3_grouped_experts(x, ids, w, gu, dn, out=y, workspace=ws, stream=s)
        finally:
            g.capture_end()
    assert ei.value.status == X.EXL3_E_INVALID
    g.replay()
    torch.cuda.synchronize()
    assert (y == 0).all()
    monkeypatch.setenv("EXL3_CHECK_IDS", "0")
    np.testing.assert_array_equal(_run(m), _run(m))


# EXL3_CHECK_IDS: ids outside [0, experts) are counted on the device before
# any expert kernel runs, and the call fails with EXL3_E_INVALID; valid ids
# give the same result as without the check (both regimes, both entry points)
@pytest.mark.parametrize("t", [5, 200])
def test_check_ids_debug_option(t, monkeypatch):
    import torch
    import gemm_exl3_linear_amd as X
    m = _small(t, seed=49)
    y_off = _run(m)
    monkeypatch.setenv("EXL3_CHECK_IDS", "1")
    np.testing.assert_array_equal(_run(m), y_off)
    gu = X.Exl3Arena.from_numpy(m["gate_up"], G.dev())
    dn = X.Exl3Arena.from_numpy(m["down"], G.dev())
    mg = X.Exl3MixedArena.from_numpy(dict(m["gate_up"], trellis=list(m["gate_up"]["trellis"]),
                                          bits=np.full(16, 3, np.int32)), G.dev())
    md = X.Exl3MixedArena.from_numpy(dict(m["down"], trellis=list(m["down"]["trellis"]),
                                          bits=np.full(16, 3, np.int32)), G.dev())
    x = G.to_dev(m["x"])
    w = G.to_dev(m["weights"].astype(np.float32))
    for bad in (16, -1, 1 << 20):
        ids = m["ids"].copy()
        ids[t // 2, 1] = bad
        for call in (lambda i: X.exl3_grouped_experts(x, i, w, gu, dn),
                     lambda i: X.exl3_grouped_experts_mixed(x, i, w, mg, md)):
            with pytest.raises(X.Exl3Error) as ei:
                call(G.to_dev(ids.astype(np.int32)))
            assert ei.value.status == X.EXL3_E_INVALID
    torch.cuda.synchronize()
    y_mixed = X.exl3_grouped_experts_mixed(x, G.to_dev(m["ids"].astype(np.int32)), w, mg, md)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y_mixed.double().cpu().numpy(), y_off)
