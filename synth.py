"""Seeded synthetic inputs for the EXL3 linear layer and the routed-expert MLP.

This module only draws random numbers in a fixed order.  It holds none of the
method's arithmetic (no decode, no codebook, no Hadamard transform, no
product), so that both the float64 oracle's callers and the GPU path's callers
can feed the very same host arrays to each side.

Shapes follow the per-tensor EXL3 record described on the exl3xpu pages
(README of exl3xpu, section "MoE (routed experts)", and the MoE post, section
2A): a trellis of uint16 words shaped [k/16, n/16, 16*K], fp16 sign vectors
suh (length k) and svh (length n), and for experts packed arenas
[E, slots, k/16, n/16, 16*K].

Draw order for one tensor (numpy PCG64 via ``default_rng(seed)``):
  1. trellis words, uniform over [0, 65535]
  2. suh, then svh, as +-1 with probability 1/2 each, stored as fp16
  3. activations x ~ N(0, 1), rounded to fp16
  4. for the expert MLP, router logits ~ N(0, 1) as float32
"""
from __future__ import annotations

import numpy as np

# Seeds used for the named workloads (one per workload, fixed).
SEED_SINGLE_2048x512 = 0
SEED_DENSE_5120x17408 = 1
SEED_PREFILL_4096x5120x17408 = 2
SEED_MIXED_LAYER = 3
SEED_MOE_256x2048x512 = 4
SEED_MOE_MIXED_WIDTHS = 5  # the same MoE shape, a width per expert from {2, 3, 4}


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def trellis(g: np.random.Generator, k: int, n: int, bits: int) -> np.ndarray:
    """Uniform random trellis words, shape [k/16, n/16, 16*bits], uint16."""
    assert k % 16 == 0 and n % 16 == 0 and 1 <= bits <= 8
    return g.integers(0, 65536, size=(k // 16, n // 16, 16 * bits), dtype=np.uint16)


def signs(g: np.random.Generator, length: int) -> np.ndarray:
    """+-1 vector with p = 1/2, as fp16."""
    return (g.integers(0, 2, size=length, dtype=np.int8) * 2 - 1).astype(np.float16)


def activations(g: np.random.Generator, m: int, k: int) -> np.ndarray:
    """x ~ N(0, 1), rounded to fp16, shape [m, k]."""
    return g.standard_normal((m, k)).astype(np.float16)


def linear_inputs(seed: int, m: int, k: int, n: int, bits: int):
    """One dense tensor plus activations, in the fixed draw order."""
    g = rng(seed)
    t = trellis(g, k, n, bits)
    suh = signs(g, k)
    svh = signs(g, n)
    x = activations(g, m, k)
    return dict(trellis=t, suh=suh, svh=svh, x=x, k=k, n=n, bits=bits)


def mixed_layer_bits(seed: int, names=("q", "k", "v", "o", "gate", "up", "down")):
    """Per-tensor widths drawn from {2..8} in the order q,k,v,o,gate,up,down,
    before any tensor data (so the widths do not depend on the shapes)."""
    g = rng(seed)
    return g, {nm: int(g.integers(2, 9)) for nm in names}


# One decoder layer's seven projections (in_features, out_features): four
# 5120 x 5120 attention projections, then the gated MLP 5120 -> 17408 -> 5120.
MIXED_LAYER_SHAPES = (("q", 5120, 5120), ("k", 5120, 5120), ("v", 5120, 5120), ("o", 5120, 5120),
                      ("gate", 5120, 17408), ("up", 5120, 17408), ("down", 17408, 5120))


def mixed_layer_inputs(seed: int, m: int, shapes=MIXED_LAYER_SHAPES):
    """The mixed-width layer: per-tensor widths first (mixed_layer_bits), then
    each tensor's trellis, suh and svh in the order q, k, v, o, gate, up,
    down, then each projection's activations x ~ N(0, 1) [m, in_features] in
    the same order."""
    g, bits = mixed_layer_bits(seed, tuple(nm for nm, _, _ in shapes))
    out = {}
    for nm, k, n in shapes:
        t = trellis(g, k, n, bits[nm])
        suh = signs(g, k)
        svh = signs(g, n)
        out[nm] = dict(trellis=t, suh=suh, svh=svh, k=k, n=n, bits=bits[nm])
    for nm, k, n in shapes:
        out[nm]["x"] = activations(g, m, k)
    return out


def expert_arena(g: np.random.Generator, experts: int, slots: int, k: int, n: int, bits: int):
    """Packed expert arena: trellis [E, slots, k/16, n/16, 16*bits], suh [E, slots, k],
    svh [E, slots, n]."""
    t = g.integers(0, 65536, size=(experts, slots, k // 16, n // 16, 16 * bits), dtype=np.uint16)
    suh = (g.integers(0, 2, size=(experts, slots, k), dtype=np.int8) * 2 - 1).astype(np.float16)
    svh = (g.integers(0, 2, size=(experts, slots, n), dtype=np.int8) * 2 - 1).astype(np.float16)
    return dict(trellis=t, suh=suh, svh=svh, experts=experts, slots=slots, k=k, n=n, bits=bits)


def mixed_expert_arena(g: np.random.Generator, slots: int, k: int, n: int, widths):
    """Arena with a width per expert: trellis is a list whose entry e is
    [slots, k/16, n/16, 16*widths[e]]; suh [E, slots, k], svh [E, slots, n];
    bits int32 [E]."""
    widths = np.asarray(widths, dtype=np.int32)
    t = [g.integers(0, 65536, size=(slots, k // 16, n // 16, 16 * int(b)), dtype=np.uint16)
         for b in widths]
    e = len(widths)
    suh = (g.integers(0, 2, size=(e, slots, k), dtype=np.int8) * 2 - 1).astype(np.float16)
    svh = (g.integers(0, 2, size=(e, slots, n), dtype=np.int8) * 2 - 1).astype(np.float16)
    return dict(trellis=t, suh=suh, svh=svh, experts=e, slots=slots, k=k, n=n, bits=widths)


def router_logits(g: np.random.Generator, t: int, experts: int) -> np.ndarray:
    return g.standard_normal((t, experts)).astype(np.float32)


def topk_routing(logits: np.ndarray, topk: int):
    """Harness routing: softmax of the logits (float64), then the top-k
    probabilities and their expert ids.  Weights are the softmax
    probabilities themselves, not renormalised; ties go to the lower id.
    This is input synthesis (the router is not part of the layer)."""
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    # stable descending sort: negate, argsort with a stable kind keeps lower id first on ties
    order = np.argsort(-p, axis=1, kind="stable")[:, :topk]
    ids = order.astype(np.int32)
    w = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return ids, w


def moe_inputs(seed: int, t: int, experts: int = 256, topk: int = 8, hidden: int = 2048,
               inter: int = 512, bits: int = 3):
    """Routed-expert workload: gate/up arena (2 slots, hidden -> inter), down arena
    (1 slot, inter -> hidden), activations and routing, in a fixed draw order."""
    g = rng(seed)
    gate_up = expert_arena(g, experts, 2, hidden, inter, bits)
    down = expert_arena(g, experts, 1, inter, hidden, bits)
    x = activations(g, t, hidden)
    logits = router_logits(g, t, experts)
    ids, w = topk_routing(logits, topk)
    return dict(gate_up=gate_up, down=down, x=x, ids=ids, weights=w, topk=topk)


def moe_mixed_inputs(seed: int, t: int, experts: int = 256, topk: int = 8, hidden: int = 2048,
                     inter: int = 512, widths=(2, 3, 4, 5, 6)):
    """Routed-expert workload whose experts each have their own width, drawn
    uniformly from ``widths`` (gate/up widths first, then down), then the
    arenas, activations and routing in the order of ``moe_inputs``."""
    g = rng(seed)
    choices = np.asarray(widths, dtype=np.int32)
    w_gu = choices[g.integers(0, len(choices), size=experts)]
    w_dn = choices[g.integers(0, len(choices), size=experts)]
    gate_up = mixed_expert_arena(g, 2, hidden, inter, w_gu)
    down = mixed_expert_arena(g, 1, inter, hidden, w_dn)
    x = activations(g, t, hidden)
    logits = router_logits(g, t, experts)
    ids, w = topk_routing(logits, topk)
    return dict(gate_up=gate_up, down=down, x=x, ids=ids, weights=w, topk=topk)
