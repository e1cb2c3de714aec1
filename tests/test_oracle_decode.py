"""Pins for the oracle's trellis decode and mul1 codebook (CPU only)."""
import numpy as np
import pytest

import synth
from oracle import exl3_oracle as O
from tests._golden import facts, rows


def _tile_words(bits, fn):
    return np.array([fn(i) & 0xFFFF for i in range(16 * bits)], dtype=np.uint16)


def test_worked_states_from_golden():
    for kbits, j, s in rows("trellis_states_worked.txt"):
        kbits, j, s = int(kbits), int(j), int(s, 16)
        w = _tile_words(kbits, lambda i: 0x1234 + 0x1111 * i)
        assert O.tile_states_bitlevel(w, kbits)[j] == s
        assert O.tensor_states(w.reshape(1, 1, -1), kbits)[0, 0, j] == s


@pytest.mark.parametrize("kbits", range(1, 9))
def test_wordpair_form_matches_bitlevel(kbits):
    g = np.random.default_rng(100 + kbits)
    for _ in range(3):
        w = g.integers(0, 65536, size=16 * kbits, dtype=np.uint16)
        a = O.tile_states_bitlevel(w, kbits)
        b = O.tensor_states(w.reshape(1, 1, -1), kbits)[0, 0]
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("kbits", range(1, 9))
def test_constant_tiles(kbits):
    zero = np.zeros(16 * kbits, np.uint16)
    ones = np.full(16 * kbits, 0xFFFF, np.uint16)
    assert (O.tile_states_bitlevel(zero, kbits) == 0).all()
    assert (O.tile_states_bitlevel(ones, kbits) == 0xFFFF).all()


def test_tail_biting_single_bit():
    # K=4, only the first bit of the stream set: the windows that see it are
    # the one starting at bit 0 and the three that wrap around the end.
    w = np.zeros(64, np.uint16)
    w[0] = 0x8000
    s = O.tile_states_bitlevel(w, 4)
    nz = {int(j): int(s[j]) for j in np.nonzero(s)[0]}
    assert nz == {0: 0x8000, 253: 0x0008, 254: 0x0080, 255: 0x0800}


def test_single_bit_every_width():
    # A single set bit at stream position p is seen by exactly the states whose
    # window covers p (cyclically), at weight 2**(15 - offset).
    for kbits in range(1, 9):
        L = 256 * kbits
        for p in (0, 7, 16 * kbits - 1, L - 1):
            w = np.zeros(16 * kbits, np.uint16)
            w[p // 16] = 1 << (15 - p % 16)
            s = O.tensor_states(w.reshape(1, 1, -1), kbits)[0, 0]
            for j in range(256):
                off = (p - kbits * j) % L
                expect = (1 << (15 - off)) if off < 16 else 0
                assert s[j] == expect


def test_codebook_worked_values_from_golden():
    for st, sig, val in rows("mul1_codebook_worked.txt"):
        st = int(st, 16)
        assert int(O.mul1_sigma(np.array([st]))[0]) == int(sig)
        assert float(O.mul1_value(np.array([st]))[0]) == float(val)


def test_codebook_bound_all_states():
    bound = float(facts()["codebook_bound"][0])
    v = O.mul1_value(np.arange(65536)).astype(np.float64)
    assert np.abs(v).max() == bound
    assert v[0] == -bound                     # attained at the all-zero state
    assert v.dtype == np.float64 and (np.abs(v) <= bound).all()


def test_codebook_distribution_all_states():
    # With the byte sum of a multiplicative hash the values are close to a
    # zero-mean, unit-variance distribution; a wrong scale or bias fails this.
    v = O.mul1_value(np.arange(65536)).astype(np.float64)
    sig = O.mul1_sigma(np.arange(65536))
    assert abs(v.mean()) < 5e-3
    assert abs(v.std() - 1.0) < 1e-2
    assert sig.min() == 0 and sig.max() == 998
    assert len(np.unique(v)) == 905


def test_codebook_single_rounding():
    # Each value is the fp16 nearest to the exact rational (sigma-510)*1775/2**18.
    sig = np.arange(0, 1021)
    exact = (sig - 510) * 1775 / 2.0 ** 18
    v16 = ((sig - 510) * 1775 / 2.0 ** 18).astype(np.float16).astype(np.float64)
    nxt = np.nextafter(v16.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    prv = np.nextafter(v16.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    assert (np.abs(v16 - exact) <= np.abs(nxt - exact)).all()
    assert (np.abs(v16 - exact) <= np.abs(prv - exact)).all()


def test_decode_tensor_placement():
    # Every tile decoded on its own by the bit-level route must land at rows
    # 16a.., columns 16b.. with state j at (j // 16, j % 16).
    g = np.random.default_rng(7)
    for kbits in (1, 3, 4, 8):
        t = synth.trellis(g, 48, 32, kbits)   # 3 x 2 tiles, not square
        W = O.decode_tensor(t, kbits)
        assert W.shape == (48, 32) and W.dtype == np.float16
        for a in range(3):
            for b in range(2):
                tile = O.decode_tile(t[a, b], kbits)
                np.testing.assert_array_equal(W[16 * a:16 * a + 16, 16 * b:16 * b + 16], tile)
        s = O.tile_states_bitlevel(t[1, 0], kbits)
        assert W[16 + 2, 0 + 5] == O.mul1_value(np.array([s[2 * 16 + 5]]))[0]


def test_shape_and_storage_accounting():
    f = facts()
    shp = tuple(int(v) for v in f["single_tensor_trellis_shape"])
    d = synth.linear_inputs(synth.SEED_SINGLE_2048x512, 1, 2048, 512, 4)
    assert d["trellis"].shape == shp
    assert d["trellis"].nbytes == int(f["single_tensor_trellis_bytes"][0]) == 2048 * 512 * 4 // 8
    for kbits in range(int(f["widths"][0]), int(f["widths"][1]) + 1):
        t = synth.trellis(np.random.default_rng(0), 128, 256, kbits)
        assert t.nbytes * 8 == 128 * 256 * kbits        # K bits per weight
    assert O.bits_per_weight(2048, 512, 4) == 4.0390625
    assert abs(O.bits_per_weight(5120, 17408, 4) - 4.0040441) < 1e-7
    m = synth.moe_inputs(synth.SEED_MOE_256x2048x512, 1, experts=4)
    assert m["gate_up"]["trellis"].shape[1:] == tuple(int(v) for v in f["moe_arena_gate_up"][1:])
    assert m["down"]["trellis"].shape[1:] == tuple(int(v) for v in f["moe_arena_down"][1:])


def test_planted_mistakes_fail():
    # A decode that reads words least-significant bit first, or that drops the
    # wrap-around, or that places tiles transposed, must disagree with the pins.
    w = _tile_words(4, lambda i: 0x1234 + 0x1111 * i)
    good = O.tile_states_bitlevel(w, 4)
    rev = np.array([int(f"{int(x):016b}"[::-1], 2) for x in w], np.uint16)
    assert O.tile_states_bitlevel(rev, 4)[0] != good[0]
    nowrap = O.tensor_states(np.concatenate([w, [0]]).reshape(1, 1, -1)[..., :64], 4)
    assert nowrap[0, 0, 255] == good[255]       # sanity: same input, same wrap
    assert (good[255] != (int(w[63]) & 0xF) << 12)  # window without wrap would differ
