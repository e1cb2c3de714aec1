"""Float64 CPU oracle for the EXL3 quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
``cpu_baseline`` leg of the benchmark may import or call this module.  The
product path (the HIP library and its Python binding) never does, and shares
no code, table or constant generator with it.

What the pages fix, and what this file therefore follows:
  * exl3xpu README, "MoE (routed experts)" and the Arc 140V MoE post, section
    2A: a tensor is a trellis of uint16 words shaped [k/16, n/16, 16*K] plus
    sign vectors suh (length k) and svh (length n); 16x16 weight tiles.
  * TensorFold issue #832, "Description": widths K = 1..8, mixed per tensor;
    the record also carries an optional bias and a codebook marker.
  * exl3xpu README, "Prefill: int8 linears ...": every mul1 codebook value is
    bounded by 3.453125 and the GEMM runs in the Hadamard domain.
  * exl3xpu README, "MoE (routed experts)": the routed contribution is
    computed in fp32, with the routing weight applied to the down-projection
    output, never to its input.
  * exl3xpu README, "Adding a model": all linear dims are multiples of 128.

What the pages leave open, and the reading taken here (each one a named
constant or a single function below):
  D1  tile bitstream: the 16*K words of a tile read in index order, each
      word most-significant bit first.
  D2  trellis state j (0..255): the 16-bit window that starts at bit K*j of
      the tile's cyclic bitstream (tail-biting bitshift trellis).
  D3  mul1 codebook: h = S * MUL1_MULTIPLIER mod 2**32; sigma = sum of the 4
      bytes of h; value = fp16_RN((sigma - 510) * 1775 / 2**18).  The factor
      is exact in float64, so the value carries exactly one rounding.
  D4  placement: state j of tile (a, b) is weight row 16a + j // 16, column
      16b + j % 16 (row-major in the tile, rows along k).
  H   Hadamard: Sylvester H_128 / sqrt(128), applied blockwise on 128
      consecutive elements.
  L   y = ((x * suh) H_k  W  H_n) * svh (+ bias).
  G   grouped experts: for every (token, slot): g = L_gate(x), u = L_up(x),
      a = silu(g) * u, d = L_down(a), Y[token] += w[token, slot] * d.
  I8  int8 prefill (exl3xpu README, "Prefill: int8 linears ..."): activations
      get one int8 scale per row, taken after the input transform; weights
      one static scale, 127 / 3.453125, applied inside the decode.
      I8W: W_q = RNE((sigma - 510) * 1775 / 2**18 * 127 / 3.453125), from the
           codebook value before its fp16 rounding (the static scale joins
           the codebook's own affine step, so the weight is rounded once, to
           int8); |W_q| <= 127 and no value is a tie.
      I8X: per row of x' = (x * suh) H_k: a = max |x'|, x_q = RNE(127 x' / a)
           (|x_q| <= 127), scale a / 127; an all-zero row gives x_q = 0.
      I8L: y' = (x_q W_q) * (a / 127) * (3.453125 / 127), the integer product
           exact; y = (y' H_n) * svh (+ bias).

Parity with real EXL3 checkpoints is not claimed: the pages do not define the
trellis or codebook constants, so D1-D4 define this project's own format.
Every function below is pinned by tests that do not re-derive it from itself
(worked examples, brute force over all states, closed forms, invariants and a
library Hadamard matrix).
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# constants of the readings (one name each)
# ---------------------------------------------------------------------------
TILE = 16                       # 16 x 16 weight tiles
STATE_BITS = 16                 # width of a trellis state
MUL1_MULTIPLIER = 0x9E3779      # floor(2**24 / golden ratio), Knuth's multiplicative hash
MUL1_BIAS = 510                 # centre of the byte sum (4 bytes * 255 / 2)
MUL1_SCALE_NUM = 1775           # value = (sigma - 510) * 1775 / 2**18
MUL1_SCALE_SHIFT = 18
MUL1_BOUND = 3.453125           # printed bound of the mul1 codebook
HADAMARD_BLOCK = 128            # linear dims are multiples of 128
CODEBOOK_MUL1 = 2               # the pages' codebook marker for mul1 ("cb=2")
INT8_MAX = 127                  # symmetric int8 range of the int8 prefill
INT8_WEIGHT_SCALE = INT8_MAX / MUL1_BOUND  # static weight scale, 127 / 3.453125


# ---------------------------------------------------------------------------
# D1 / D2: trellis states of one tile
# ---------------------------------------------------------------------------
def tile_bitstream(words: np.ndarray) -> np.ndarray:
    """D1: the tile's bits in stream order (word index order, MSB first).

    Returns an int array of length 16 * len(words) holding 0/1.
    """
    bits = []
    for w in words.tolist():
        for t in range(16):
            bits.append((w >> (15 - t)) & 1)
    return np.array(bits, dtype=np.int64)


def tile_states_bitlevel(words: np.ndarray, bits: int) -> np.ndarray:
    """D2, written out bit by bit: S_j = sum_t beta[(K j + t) mod L] 2^(15 - t).

    Literal definition; pure Python, for small cases and as the reference the
    word-pair form is checked against.
    """
    assert len(words) == TILE * bits
    beta = tile_bitstream(words)
    L = len(beta)  # 256 * K
    out = np.zeros(TILE * TILE, dtype=np.int64)
    for j in range(TILE * TILE):
        s = 0
        for t in range(STATE_BITS):
            s = (s << 1) | int(beta[(bits * j + t) % L])
        out[j] = s
    return out


def tensor_states(trellis: np.ndarray, bits: int) -> np.ndarray:
    """D2 in its word-pair form, vectorised over every tile of a tensor.

    S_j = ((w_q << 16 | w_{(q+1) mod 16K}) >> (16 - o)) & 0xFFFF with
    q = floor(K j / 16), o = K j mod 16.  Returns int64 [k/16, n/16, 256].
    """
    nw = TILE * bits
    assert trellis.shape[-1] == nw
    j = np.arange(TILE * TILE)
    q = (bits * j) // 16
    o = (bits * j) % 16
    w = trellis.astype(np.int64)
    hi = w[..., q]
    lo = w[..., (q + 1) % nw]
    pair = (hi << 16) | lo
    return (pair >> (16 - o)) & 0xFFFF


# ---------------------------------------------------------------------------
# D3: mul1 codebook
# ---------------------------------------------------------------------------
def mul1_sigma(states: np.ndarray) -> np.ndarray:
    """Byte sum of h = S * MUL1_MULTIPLIER mod 2**32 (vectorised, int64)."""
    h = (np.asarray(states, dtype=np.int64) * MUL1_MULTIPLIER) & 0xFFFFFFFF
    return (h & 0xFF) + ((h >> 8) & 0xFF) + ((h >> 16) & 0xFF) + ((h >> 24) & 0xFF)


def mul1_value(states: np.ndarray) -> np.ndarray:
    """D3: fp16_RN((sigma - 510) * 1775 / 2**18).

    (sigma - 510) * 1775 is an integer below 2**20 in magnitude, so the float64
    product with 2**-18 is exact and numpy's float16 cast (round to nearest,
    ties to even) is the one rounding.
    """
    sig = mul1_sigma(states)
    exact = (sig - MUL1_BIAS).astype(np.float64) * (MUL1_SCALE_NUM / float(1 << MUL1_SCALE_SHIFT))
    return exact.astype(np.float16)


# ---------------------------------------------------------------------------
# D4: decoded tensor
# ---------------------------------------------------------------------------
def decode_tile(words: np.ndarray, bits: int) -> np.ndarray:
    """One 16x16 tile from its 16*K words (bit-level states, pure Python)."""
    s = tile_states_bitlevel(np.asarray(words, dtype=np.uint16), bits)
    return mul1_value(s).reshape(TILE, TILE)


def decode_tensor(trellis: np.ndarray, bits: int) -> np.ndarray:
    """Decoded Hadamard-domain weight W~ (fp16, [k, n]) from a [k/16, n/16, 16K] trellis.

    Tile (a, b) lands at rows 16a.., columns 16b..; inside the tile state j is
    row j // 16, column j % 16 (D4).
    """
    kt, nt, _ = trellis.shape
    v = mul1_value(tensor_states(trellis, bits))            # [kt, nt, 256]
    v = v.reshape(kt, nt, TILE, TILE)                        # [a, b, r, c]
    return v.transpose(0, 2, 1, 3).reshape(kt * TILE, nt * TILE)


def bits_per_weight(k: int, n: int, bits: int) -> float:
    """Storage rate of one tensor: trellis bits plus the two fp16 sign vectors."""
    return (k * n * bits + 16 * (k + n)) / (k * n)


# ---------------------------------------------------------------------------
# H: Hadamard transform
# ---------------------------------------------------------------------------
def sylvester_hadamard(size: int = HADAMARD_BLOCK) -> np.ndarray:
    """H[i][j] = (-1)^popcount(i & j), float64, unnormalised."""
    i = np.arange(size)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(np.bitwise_and.outer(i, i))
    return np.where(pc % 2 == 0, 1.0, -1.0)


def hadamard_explicit(x: np.ndarray) -> np.ndarray:
    """x (..., d) times blockdiag(H_128 / sqrt(128)) by explicit matrix products."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % HADAMARD_BLOCK == 0
    H = sylvester_hadamard() / math.sqrt(HADAMARD_BLOCK)
    xb = x.reshape(*x.shape[:-1], d // HADAMARD_BLOCK, HADAMARD_BLOCK)
    return (xb @ H).reshape(x.shape)


def fwht(x: np.ndarray) -> np.ndarray:
    """Same product by the butterfly (a, b) -> (a + b, a - b) over strides 1..64,
    then the 1/sqrt(128) normalisation."""
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    assert d % HADAMARD_BLOCK == 0
    y = x.reshape(-1, d // HADAMARD_BLOCK, HADAMARD_BLOCK)
    h = 1
    while h < HADAMARD_BLOCK:
        y = y.reshape(y.shape[0], y.shape[1], HADAMARD_BLOCK // (2 * h), 2, h)
        a = y[:, :, :, 0, :].copy()
        b = y[:, :, :, 1, :].copy()
        y[:, :, :, 0, :] = a + b
        y[:, :, :, 1, :] = a - b
        y = y.reshape(y.shape[0], y.shape[1], HADAMARD_BLOCK)
        h *= 2
    return (y / math.sqrt(HADAMARD_BLOCK)).reshape(x.shape)


def hadamard(x: np.ndarray, sign_before=None, sign_after=None) -> np.ndarray:
    """((x * sign_before) Hhat_d) * sign_after, float64 (the standalone transform)."""
    x = np.asarray(x, dtype=np.float64)
    if sign_before is not None:
        x = x * np.asarray(sign_before, dtype=np.float64)
    y = fwht(x)
    if sign_after is not None:
        y = y * np.asarray(sign_after, dtype=np.float64)
    return y


# ---------------------------------------------------------------------------
# L: the EXL3 linear layer
# ---------------------------------------------------------------------------
def linear(x, trellis, suh, svh, bits, bias=None, w_decoded=None) -> np.ndarray:
    """y = ((x * suh) Hhat_k  W~  Hhat_n) * svh (+ bias), all in float64.

    x is [m, k]; the fp16 inputs are widened exactly.  ``w_decoded`` lets a
    caller that already holds decode_tensor(trellis) skip decoding again.
    """
    W = decode_tensor(trellis, bits) if w_decoded is None else w_decoded
    xp = hadamard(np.asarray(x, dtype=np.float64), sign_before=suh)
    yp = xp @ W.astype(np.float64)
    y = hadamard(yp, sign_after=svh)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y


def effective_weight(trellis, suh, svh, bits) -> np.ndarray:
    """W_eff = diag(suh) Hhat_k W~ Hhat_n diag(svh) (explicit Hadamard matrices)."""
    W = decode_tensor(trellis, bits).astype(np.float64)
    k, n = W.shape
    Hk = np.kron(np.eye(k // HADAMARD_BLOCK), sylvester_hadamard() / math.sqrt(HADAMARD_BLOCK))
    Hn = np.kron(np.eye(n // HADAMARD_BLOCK), sylvester_hadamard() / math.sqrt(HADAMARD_BLOCK))
    return (np.asarray(suh, np.float64)[:, None] * (Hk @ W @ Hn)) * np.asarray(svh, np.float64)[None, :]


def linear_weff(x, trellis, suh, svh, bits, bias=None) -> np.ndarray:
    """Second route to the same layer: y = x W_eff (+ bias)."""
    y = np.asarray(x, dtype=np.float64) @ effective_weight(trellis, suh, svh, bits)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y


# ---------------------------------------------------------------------------
# I8: int8 prefill
# ---------------------------------------------------------------------------
def mul1_int8_from_sigma(sig: np.ndarray) -> np.ndarray:
    """I8W on byte sums: RNE((sigma - 510) * 1775 / 2**18 * 127 / 3.453125).

    The codebook value before rounding is exact in float64; the product with
    the static scale is within 1e-14 of exact, far from the nearest tie
    (0.0015 away over sigma in [0, 1020]), so np.rint decides as exact
    arithmetic would.
    """
    exact = (np.asarray(sig, dtype=np.int64) - MUL1_BIAS).astype(np.float64) * (
        MUL1_SCALE_NUM / float(1 << MUL1_SCALE_SHIFT))
    return np.rint(exact * INT8_WEIGHT_SCALE).astype(np.int8)


def mul1_int8(states: np.ndarray) -> np.ndarray:
    """I8W: int8 weight of each trellis state."""
    return mul1_int8_from_sigma(mul1_sigma(states))


def decode_tensor_int8(trellis: np.ndarray, bits: int) -> np.ndarray:
    """int8 weight W_q [k, n], placed as decode_tensor places W~ (D4)."""
    kt, nt, _ = trellis.shape
    q = mul1_int8(tensor_states(trellis, bits)).reshape(kt, nt, TILE, TILE)
    return q.transpose(0, 2, 1, 3).reshape(kt * TILE, nt * TILE)


def quantize_rows(xp: np.ndarray):
    """I8X: per-row symmetric int8 of x' (float64 in): (x_q int8 [m, k], scale [m]).

    scale = max |x'| / 127 and x_q = RNE(127 x' / max |x'|); a row of zeros
    gives x_q = 0 and scale 0.
    """
    xp = np.asarray(xp, dtype=np.float64)
    a = np.abs(xp).max(axis=1)
    safe = np.where(a > 0, a, 1.0)
    q = np.rint(xp * INT8_MAX / safe[:, None])
    q[a == 0] = 0
    return q.astype(np.int8), a / INT8_MAX


def linear_int8(x, trellis, suh, svh, bits, bias=None, wq=None) -> np.ndarray:
    """I8L: the int8 prefill layer in float64.

    The integer product x_q W_q runs as a float64 matrix product, which is
    exact here: every term is an integer of magnitude <= 127**2 and every
    partial sum stays below 2**53 for k < 5e11.  ``wq`` lets a caller that
    holds decode_tensor_int8(trellis) skip decoding.
    """
    Wq = decode_tensor_int8(trellis, bits) if wq is None else wq
    xp = hadamard(np.asarray(x, dtype=np.float64), sign_before=suh)
    xq, sx = quantize_rows(xp)
    acc = xq.astype(np.float64) @ Wq.astype(np.float64)
    yp = acc * sx[:, None] / INT8_WEIGHT_SCALE
    y = hadamard(yp, sign_after=svh)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y


# ---------------------------------------------------------------------------
# G: routed experts
# ---------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def grouped_experts(x, ids, weights, gate_up: dict, down: dict, decoded=None) -> np.ndarray:
    """Routed contribution Y [t, hidden] (float64).

    For each token t and slot s: e = ids[t, s]; g and u are the gate (slot 0)
    and up (slot 1) linears of expert e; a = silu(g) * u; d is the down linear
    of e applied to a; Y[t] += weights[t, s] * d.  Experts are evaluated one
    (token, slot) pair at a time through ``linear``; decoded weights are cached
    per expert only to save time.

    An arena's ``bits`` is one width for every expert, or a sequence with the
    width of each expert (TensorFold issue #832, "Activity": the consolidated
    module keeps a width per expert); ``trellis[e][slot]`` is then expert e's
    tensor at its own width.

    ``decoded`` lets a caller that already holds decode_tensor of some expert
    tensors skip decoding them: a dict from ("gate_up" or "down", e, slot) to
    the decoded fp16 [k, n] weight.
    """
    x = np.asarray(x)
    ids = np.asarray(ids)
    weights = np.asarray(weights, dtype=np.float64)
    t_count, topk = ids.shape
    hidden = down["n"]
    y = np.zeros((t_count, hidden), dtype=np.float64)
    cache = {}

    def width(arena, e):
        b = arena["bits"]
        return int(b[e]) if np.ndim(b) else int(b)

    def dec(arena, e, slot):
        key = (id(arena), e, slot)
        if key not in cache:
            kind = "gate_up" if arena is gate_up else "down"
            if decoded is not None and (kind, e, slot) in decoded:
                cache[key] = decoded[(kind, e, slot)]
            else:
                cache[key] = decode_tensor(arena["trellis"][e][slot], width(arena, e))
        return cache[key]

    for t in range(t_count):
        for s in range(topk):
            e = int(ids[t, s])
            xt = x[t:t + 1]
            g = linear(xt, gate_up["trellis"][e][0], gate_up["suh"][e, 0], gate_up["svh"][e, 0],
                       width(gate_up, e), w_decoded=dec(gate_up, e, 0))
            u = linear(xt, gate_up["trellis"][e][1], gate_up["suh"][e, 1], gate_up["svh"][e, 1],
                       width(gate_up, e), w_decoded=dec(gate_up, e, 1))
            a = silu(g) * u
            d = linear(a, down["trellis"][e][0], down["suh"][e, 0], down["svh"][e, 0],
                       width(down, e), w_decoded=dec(down, e, 0))
            y[t] += weights[t, s] * d[0]
    return y


def rel_frobenius(a, ref) -> float:
    """||a - ref||_F / ||ref||_F in float64 (the layer-output tolerance metric).

    The Frobenius norm is the square root of the sum of squares over every
    element, whatever the array's rank.  A zero reference gives the absolute
    norm ||a||_F instead.
    """
    a = np.asarray(a, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    den = math.sqrt(float(np.dot(ref, ref)))
    diff = a - ref
    num = math.sqrt(float(np.dot(diff, diff)))
    return num / den if den > 0 else num


def fp16_ulp(v) -> np.ndarray:
    """Spacing of the fp16 values at |v|: 2^(e - 10) for 2^e <= |v| < 2^(e+1)
    in the normal range, 2^-24 below it (float64)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.maximum(a, 2.0 ** -14))  # a = f 2^e with f in [0.5, 1)
    return np.ldexp(1.0, e - 11)


def elementwise_excess(a, ref, rel_rms: float, ulps: float = 1.0) -> float:
    """Largest |a - ref| / (rel_rms * rms(ref) + ulps * fp16_ulp(ref)) over the
    elements (float64); the per-element bound holds when this is <= 1.

    rms(ref) is the root mean square over the whole array.  The bound sits
    beside the Frobenius one: a few wrong elements can hide in a norm over
    millions of them, but not here.
    """
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert a.shape == ref.shape
    if ref.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(ref * ref)))
    bound = rel_rms * rms + ulps * fp16_ulp(ref)
    return float(np.max(np.abs(a - ref) / bound))
