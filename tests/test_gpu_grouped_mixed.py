"""GPU parity of exl3_grouped_experts_mixed (a width per expert, TensorFold
issue #832, "Activity") against the float64 oracle, on both regimes (per-pair
units and grouped GEMM), and bit-identity with exl3_grouped_experts where the
two must agree."""
import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _run_mixed(m, ids=None, w=None):
    import torch
    import gemm_exl3_linear_amd as X
    ids = m["ids"] if ids is None else ids
    w = m["weights"] if w is None else w
    gu = X.Exl3MixedArena.from_numpy(m["gate_up"], G.dev())
    dn = X.Exl3MixedArena.from_numpy(m["down"], G.dev())
    y = X.exl3_grouped_experts_mixed(G.to_dev(m["x"]), G.to_dev(ids.astype(np.int32)),
                                     G.to_dev(w.astype(np.float32)), gu, dn)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _run_uniform(m, ids=None):
    import torch
    import gemm_exl3_linear_amd as X
    ids = m["ids"] if ids is None else ids
    gu = X.Exl3Arena.from_numpy(m["gate_up"], G.dev())
    dn = X.Exl3Arena.from_numpy(m["down"], G.dev())
    y = X.exl3_grouped_experts(G.to_dev(m["x"]), G.to_dev(ids.astype(np.int32)),
                               G.to_dev(m["weights"].astype(np.float32)), gu, dn)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _ref(m, ids=None, tokens=None):
    ids = m["ids"] if ids is None else ids
    x, w = m["x"], m["weights"]
    if tokens is not None:
        x, ids, w = x[tokens], ids[tokens], w[tokens]
    return O.grouped_experts(x, ids, w, m["gate_up"], m["down"])


def _small(t, experts=16, topk=4, hidden=256, inter=128, widths=(2, 3, 5, 8), seed=60):
    return synth.moe_mixed_inputs(seed + t, t, experts=experts, topk=topk, hidden=hidden, inter=inter,
                                  widths=widths)


def _as_mixed(arena):
    """The same tensors as a list with one width per expert."""
    e = arena["experts"]
    return dict(arena, trellis=[arena["trellis"][i] for i in range(e)],
                bits=np.full(e, arena["bits"], np.int32))


# t * topk <= 224 pairs take the unit path (every width's launch adds to the
# same arrival counters), more the binned grouped GEMM; both sides here
@pytest.mark.parametrize("t", [1, 2, 16, 56, 57, 200])
def test_mixed_widths_random_routing(t):
    m = _small(t)
    assert len(set(m["gate_up"]["bits"].tolist())) > 1
    err = O.rel_frobenius(_run_mixed(m), _ref(m))
    assert err < TOL, err


# 256-row tiles (t = 700 on 8 experts) and every width 1..8 in each arena
@pytest.mark.parametrize("t", [3, 700])
def test_mixed_widths_all_widths(t):
    m = _small(t, experts=8, widths=(1, 2, 3, 4, 5, 6, 7, 8), seed=61)
    gu, dn = m["gate_up"], m["down"]
    gu["bits"] = np.arange(1, 9, dtype=np.int32)
    dn["bits"] = np.arange(8, 0, -1, dtype=np.int32)
    g = np.random.default_rng(5)
    gu["trellis"] = [g.integers(0, 65536, size=(2, 16, 8, 16 * b), dtype=np.uint16) for b in gu["bits"]]
    dn["trellis"] = [g.integers(0, 65536, size=(1, 8, 16, 16 * b), dtype=np.uint16) for b in dn["bits"]]
    err = O.rel_frobenius(_run_mixed(m), _ref(m))
    assert err < TOL, err


# one width everywhere: the same launches and sums as the uniform call
@pytest.mark.parametrize("t", [1, 24, 200])
def test_one_width_is_bit_identical_to_uniform(t):
    m = synth.moe_inputs(70 + t, t, experts=16, topk=4, hidden=256, inter=128, bits=3)
    y_u = _run_uniform(m)
    mm = dict(m, gate_up=_as_mixed(m["gate_up"]), down=_as_mixed(m["down"]))
    np.testing.assert_array_equal(_run_mixed(mm), y_u)


# routing that only reaches experts of one width K: bit-identical to a
# uniform arena of width K holding the same tensors for those experts
@pytest.mark.parametrize("t", [2, 200])
def test_experts_of_one_width_match_uniform_arena(t):
    m = _small(t, experts=16, topk=2, widths=(3, 5), seed=62)
    gu, dn = m["gate_up"], m["down"]
    K = 5
    # give gate/up and down the same widths so one id set sees width K in both
    dn["bits"] = gu["bits"].copy()
    g = np.random.default_rng(6)
    dn["trellis"] = [g.integers(0, 65536, size=(1, 8, 16, 16 * b), dtype=np.uint16) for b in dn["bits"]]
    sel = np.flatnonzero(gu["bits"] == K)
    assert len(sel) >= 2
    ids = np.stack([g.choice(sel, 2, replace=False) for _ in range(t)]).astype(np.int32)
    y_m = _run_mixed(m, ids=ids)

    def uniform(arena, slots, k, n):
        tr = g.integers(0, 65536, size=(arena["experts"], slots, k // 16, n // 16, 16 * K), dtype=np.uint16)
        for e in sel:
            tr[e] = arena["trellis"][e]
        return dict(arena, trellis=tr, bits=K)
    mu = dict(m, gate_up=uniform(gu, 2, 256, 128), down=uniform(dn, 1, 128, 256))
    np.testing.assert_array_equal(y_m, _run_uniform(mu, ids=ids))
    err = O.rel_frobenius(y_m, _ref(m, ids=ids))
    assert err < TOL, err


@pytest.mark.parametrize("t", [1, 4])
def test_moe_256x2048x512_mixed_widths_small_t(t):
    m = synth.moe_mixed_inputs(80 + t, t, widths=(2, 3, 4))
    err = O.rel_frobenius(_run_mixed(m), _ref(m))
    assert err < TOL, err


def test_moe_256x2048x512_mixed_widths_t4096_sampled_tokens():
    m = synth.moe_mixed_inputs(84, 4096, widths=(2, 3, 4))
    y = _run_mixed(m)
    tokens = np.sort(np.random.default_rng(2).choice(4096, 256, replace=False))
    G.assert_parity(y[tokens], G.grouped_ref(m, tokens=tokens), what="mixed widths T=4096")


def _pack(arena, order, device):
    """Exl3MixedArena with the experts' tensors laid out in `order` (offsets
    follow), to check that only the offsets place an expert."""
    import ctypes
    import torch
    import gemm_exl3_linear_amd as X
    widths = [int(b) for b in arena["bits"]]
    offsets = np.zeros(len(widths), np.int64)
    pos, parts = 0, []
    for e in order:
        offsets[e] = pos
        flat = np.ascontiguousarray(arena["trellis"][e]).reshape(-1)
        parts.append(flat)
        pos += flat.size
    flat = np.concatenate(parts)
    return X.Exl3MixedArena(torch.from_numpy(flat.view(np.int16).copy()).to(device),
                            torch.from_numpy(arena["suh"].astype(np.float16)).to(device),
                            torch.from_numpy(arena["svh"].astype(np.float16)).to(device),
                            torch.tensor(widths, dtype=torch.int32, device=device),
                            torch.from_numpy(offsets).to(device), (ctypes.c_int32 * len(widths))(*widths))


# experts packed in reverse (and shuffled) order: identical results
@pytest.mark.parametrize("t", [3, 200])
def test_packing_order_only_moves_offsets(t):
    import torch
    import gemm_exl3_linear_amd as X
    m = _small(t, experts=12, seed=63)
    ys = []
    for order in (list(range(12)), list(range(11, -1, -1)), list(np.random.default_rng(7).permutation(12))):
        gu = _pack(m["gate_up"], order, G.dev())
        dn = _pack(m["down"], order, G.dev())
        y = X.exl3_grouped_experts_mixed(G.to_dev(m["x"]), G.to_dev(m["ids"].astype(np.int32)),
                                         G.to_dev(m["weights"].astype(np.float32)), gu, dn)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
    np.testing.assert_array_equal(ys[1], ys[0])
    np.testing.assert_array_equal(ys[2], ys[0])
    err = O.rel_frobenius(ys[0], _ref(m))
    assert err < TOL, err


@pytest.mark.parametrize("t", [1, 50])
def test_mixed_widths_max_topk(t):
    m = _small(t, experts=32, topk=16, seed=64)
    err = O.rel_frobenius(_run_mixed(m), _ref(m))
    assert err < TOL, err


@pytest.mark.parametrize("t", [2, 200])
def test_mixed_widths_zero_weights_exact_zero(t):
    m = _small(t, seed=65)
    y = _run_mixed(m, w=np.zeros_like(m["weights"]))
    assert (y == 0).all()
