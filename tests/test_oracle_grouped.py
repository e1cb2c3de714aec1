"""Pins for the oracle's routed-expert MLP and the harness routing (CPU only)."""
import numpy as np
import scipy.special

import synth
from oracle import exl3_oracle as O


def _small(seed=21, t=3, experts=6, topk=2, hidden=256, inter=128, bits=3):
    return synth.moe_inputs(seed, t, experts=experts, topk=topk, hidden=hidden, inter=inter, bits=bits)


def test_silu_matches_library():
    z = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)


def test_top1_unit_weight_is_dense_swiglu():
    d = _small(topk=1)
    ids = d["ids"]
    w = np.ones_like(d["weights"])
    y = O.grouped_experts(d["x"], ids, w, d["gate_up"], d["down"])
    gu, dn = d["gate_up"], d["down"]
    for t in range(ids.shape[0]):
        e = int(ids[t, 0])
        Wg = O.effective_weight(gu["trellis"][e, 0], gu["suh"][e, 0], gu["svh"][e, 0], gu["bits"])
        Wu = O.effective_weight(gu["trellis"][e, 1], gu["suh"][e, 1], gu["svh"][e, 1], gu["bits"])
        Wd = O.effective_weight(dn["trellis"][e, 0], dn["suh"][e, 0], dn["svh"][e, 0], dn["bits"])
        xt = d["x"][t].astype(np.float64)
        g = xt @ Wg
        u = xt @ Wu
        ref = (g * scipy.special.expit(g) * u) @ Wd
        assert O.rel_frobenius(y[t], ref) < 1e-12


def test_zero_weights_give_zero():
    d = _small()
    y = O.grouped_experts(d["x"], d["ids"], np.zeros_like(d["weights"]), d["gate_up"], d["down"])
    assert (y == 0).all()


def test_weight_on_output_is_linear():
    d = _small()
    w64 = d["weights"].astype(np.float64)
    y1 = O.grouped_experts(d["x"], d["ids"], w64, d["gate_up"], d["down"])
    y3 = O.grouped_experts(d["x"], d["ids"], 3.0 * w64, d["gate_up"], d["down"])
    np.testing.assert_allclose(y3, 3.0 * y1, rtol=1e-12, atol=1e-12)


def test_unused_expert_has_no_effect_and_slots_commute():
    d = _small(experts=8)
    used = set(np.unique(d["ids"]).tolist())
    unused = [e for e in range(8) if e not in used][0]
    y = O.grouped_experts(d["x"], d["ids"], d["weights"], d["gate_up"], d["down"])
    gu = dict(d["gate_up"]); gu["trellis"] = gu["trellis"].copy()
    gu["trellis"][unused] ^= 0x5A5A
    y2 = O.grouped_experts(d["x"], d["ids"], d["weights"], gu, d["down"])
    np.testing.assert_array_equal(y, y2)
    perm = d["ids"][:, ::-1].copy(), d["weights"][:, ::-1].copy()
    y3 = O.grouped_experts(d["x"], perm[0], perm[1], d["gate_up"], d["down"])
    np.testing.assert_allclose(y3, y, rtol=1e-12, atol=1e-12)


def test_tokens_independent():
    d = _small(t=4)
    y = O.grouped_experts(d["x"], d["ids"], d["weights"], d["gate_up"], d["down"])
    for t in range(4):
        yt = O.grouped_experts(d["x"][t:t + 1], d["ids"][t:t + 1], d["weights"][t:t + 1],
                               d["gate_up"], d["down"])
        np.testing.assert_allclose(yt[0], y[t], atol=1e-12)


def _mixed(seed=23, t=4, experts=6, topk=2, hidden=256, inter=128, widths=(2, 3, 5, 8)):
    return synth.moe_mixed_inputs(seed, t, experts=experts, topk=topk, hidden=hidden, inter=inter,
                                  widths=widths)


def test_mixed_widths_top1_is_dense_swiglu_at_each_width():
    # every token's output is its one expert's SwiGLU MLP, each projection
    # decoded at that expert's own width (a wrong width changes the tensor's
    # word count, so decoding it at another width cannot give this result)
    d = _mixed(topk=1, t=6)
    gu, dn = d["gate_up"], d["down"]
    assert len(set(gu["bits"].tolist())) > 1 and len(set(dn["bits"].tolist())) > 1
    w = np.ones_like(d["weights"])
    y = O.grouped_experts(d["x"], d["ids"], w, gu, dn)
    for t in range(d["ids"].shape[0]):
        e = int(d["ids"][t, 0])
        kg, kd = int(gu["bits"][e]), int(dn["bits"][e])
        assert gu["trellis"][e].shape[-1] == 16 * kg and dn["trellis"][e].shape[-1] == 16 * kd
        Wg = O.effective_weight(gu["trellis"][e][0], gu["suh"][e, 0], gu["svh"][e, 0], kg)
        Wu = O.effective_weight(gu["trellis"][e][1], gu["suh"][e, 1], gu["svh"][e, 1], kg)
        Wd = O.effective_weight(dn["trellis"][e][0], dn["suh"][e, 0], dn["svh"][e, 0], kd)
        xt = d["x"][t].astype(np.float64)
        g = xt @ Wg
        u = xt @ Wu
        ref = (g * scipy.special.expit(g) * u) @ Wd
        assert O.rel_frobenius(y[t], ref) < 1e-12


def test_mixed_widths_equal_widths_match_uniform_arena():
    # a per-expert width list with one value is the uniform arena
    d = _small(experts=5)
    gu, dn = d["gate_up"], d["down"]
    y = O.grouped_experts(d["x"], d["ids"], d["weights"], gu, dn)
    gu_m = dict(gu, trellis=[gu["trellis"][e] for e in range(5)], bits=np.full(5, gu["bits"], np.int32))
    dn_m = dict(dn, trellis=[dn["trellis"][e] for e in range(5)], bits=np.full(5, dn["bits"], np.int32))
    np.testing.assert_array_equal(O.grouped_experts(d["x"], d["ids"], d["weights"], gu_m, dn_m), y)


def test_mixed_widths_slots_sum_over_experts_of_other_widths():
    # topk=2: each token's output is the weighted sum of two single-expert
    # outputs, whatever the two experts' widths
    d = _mixed(topk=2, t=3)
    y = O.grouped_experts(d["x"], d["ids"], d["weights"], d["gate_up"], d["down"])
    for s in range(2):
        ids1 = d["ids"][:, s:s + 1].copy()
        w1 = d["weights"][:, s:s + 1].astype(np.float64)
        part = O.grouped_experts(d["x"], ids1, w1, d["gate_up"], d["down"])
        y = y - part
    assert np.abs(y).max() < 1e-12


def test_routing_properties():
    g = np.random.default_rng(9)
    logits = synth.router_logits(g, 64, 256)
    ids, w = synth.topk_routing(logits, 8)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    assert ids.dtype == np.int32 and w.dtype == np.float32
    assert ((ids >= 0) & (ids < 256)).all()
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert (w.sum(axis=1) < 1).all()
    assert (np.diff(w, axis=1) <= 0).all()
    # the chosen ids are the 8 largest probabilities
    for r in range(64):
        kth = np.sort(p[r])[-8]
        assert (p[r, ids[r]] >= kth).all()
        np.testing.assert_allclose(w[r], p[r, ids[r]].astype(np.float32))
