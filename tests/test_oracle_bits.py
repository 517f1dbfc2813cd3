"""Pins of the oracle's 3- and 4-bit codes (an extension beyond the pages' 2 bits): the grid's closed form, the codes against brute force, the record layout as bit
planes over the pinned 2-bit layout, hand-worked positions of the 1-bit plane, and the
error falling with each extra bit.
"""
import numpy as np
import pytest

from oracle import kvarn_ref as R
from kv_cache_bit_amd import synth


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_grid_levels_and_codes_brute_force(bits):
    """s = (max - min)/(2^bits - 1), z = min; every code is the nearest level (ties to even
    index), found here by scanning all levels."""
    rng = np.random.default_rng(bits)
    y = rng.standard_normal((32, 128)) * rng.uniform(0.5, 3, 128)
    s, z, _ = R.grid(y, bits)
    mx, mn = y.max(axis=0), y.min(axis=0)
    assert np.allclose(s, (mx - mn) / (2 ** bits - 1), rtol=2 ** -10)
    assert np.array_equal(z, R.fp16_round(mn))
    q = R.codes(y, s, z, bits)
    levels = z[None, :, None] + s[None, :, None] * np.arange(2 ** bits)[None, None, :]
    dist = np.abs(y[:, :, None] - levels)
    best = dist.min(axis=-1, keepdims=True)
    ties = np.isclose(dist, best, rtol=0, atol=1e-12)
    for t in range(32):
        for j in range(128):
            cand = np.nonzero(ties[t, j])[0]
            want = cand[0] if len(cand) == 1 else cand[cand % 2 == 0][0]
            assert q[t, j] == want
    assert q.max() <= 2 ** bits - 1


@pytest.mark.parametrize("stream", [0, 1])
def test_four_bit_planes_are_two_bit_layouts(stream):
    """A 4-bit record's codes are two 2-bit planes, each in the pinned 2-bit layout."""
    rng = np.random.default_rng(7)
    q = rng.integers(0, 16, (32, 128)).astype(np.uint8)
    b = R.pack_codes(q, stream, 4)
    n = 32 * 128 // 4
    assert b.size == 2 * n
    assert np.array_equal(b[:n], R.pack_codes(q & 3, stream, 2))
    assert np.array_equal(b[n:], R.pack_codes(q >> 2, stream, 2))
    assert np.array_equal(R.unpack_codes(b, 32, 128, stream, 4), q)


def test_one_bit_plane_positions_by_hand():
    """K: channel j sits in 2-bit word w = (j % 16) // 2 at slot k = 4 (m // 2) + m % 2 + 2 d
    (m = j // 16, d = j % 2); its high bit goes to word w // 2, bit 4 (k // 2) + k % 2 +
    2 (w % 2). Worked: j = 0 (w 0, k 0) -> (0, 0); j = 1 (w 0, k 2) -> (0, 4); j = 16
    (w 0, k 1) -> (0, 1); j = 2 (w 1, k 0) -> (0, 2); j = 127 (m 7, w 7, d 1: k 15)
    -> (3, 4 * 7 + 1 + 2 = 31).
    V: j = 16 blk + c, blk = i + 4 hh, i = 2 ip + ii, t = 8 o + 2 n + par -> word
    (16 ip + c) G/8 + o, bit 4 (n + 4 hh) + par + 2 ii. Worked at G = 32: (t 0, j 0) ->
    (0, 0); (t 1, j 0) -> (0, 1); (t 2, j 0) -> (0, 4); (t 0, j 16) (blk 1: ii 1) -> (0, 2);
    (t 0, j 64) (blk 4: hh 1) -> (0, 16); (t 8, j 0) -> (1, 0); (t 0, j 32) (blk 2: ip 1)
    -> (64, 0); (t 31, j 127) (blk 7: i 3, hh 1, ip 1, ii 1; c 15; o 3, n 3, par 1)
    -> ((16 + 15) * 4 + 3, 4 * 7 + 1 + 2 = 31)."""
    for j, want in [(0, (0, 0)), (1, (0, 4)), (16, (0, 1)), (2, (0, 2)), (127, (3, 31))]:
        assert R.k_bit_position(j) == want, j
    for (t, j), want in [((0, 0), (0, 0)), ((1, 0), (0, 1)), ((2, 0), (0, 4)), ((0, 16), (0, 2)),
                         ((0, 64), (0, 16)), ((8, 0), (1, 0)), ((0, 32), (64, 0)),
                         ((31, 127), (127, 31))]:
        assert R.v_bit_position(t, j, 32) == want, (t, j)


@pytest.mark.parametrize("G", [32, 64])
def test_one_bit_plane_is_a_bijection(G):
    """Every (token, channel) has its own bit, and the G*D bits fill the plane exactly."""
    for stream in (0, 1):
        seen = set()
        for t in range(G):
            for j in range(128):
                if stream == 0:
                    u, p = R.k_bit_position(j)
                    key = (4 * t + u, p)
                else:
                    key = R.v_bit_position(t, j, G)
                assert 0 <= key[1] < 32
                seen.add(key)
        assert len(seen) == G * 128 and max(k[0] for k in seen) == G * 128 // 32 - 1
        rng = np.random.default_rng(G + stream)
        q = rng.integers(0, 8, (G, 128)).astype(np.uint8)
        b = R.pack_codes(q, stream, 3)
        assert b.size == G * 128 * 3 // 8
        assert np.array_equal(b[:G * 32], R.pack_codes(q & 3, stream, 2))
        assert np.array_equal(R.unpack_codes(b, G, 128, stream, 3), q)


def test_record_sizes():
    for bits in (2, 3, 4):
        for G in (32, 64):
            assert R.record_bytes(G, 128, bits) == G * 128 * bits // 8 + 2 * G + 6 * 128
    assert R.record_bytes(32, 128, 3) * 8 / (32 * 128) == 4.625
    assert R.record_bytes(64, 128, 4) * 8 / (64 * 128) == 4.875


def test_error_falls_with_bits():
    """The dequantized tile error stays within half a step per element, and the mean square
    error falls about 4x per extra bit (a uniform quantizer's step halves)."""
    k, v = synth.kv_host(3, 1, 256, 1)
    x = R.canonicalize(k)[0][0, :, 0]
    mse = {}
    for bits in (2, 3, 4):
        c = R.Cache(R.Geom(1, 1, 128, 256, 32, 3, bits), synth.sign_vector(0))
        R.quantize_prefill(c, k, v, 256)
        for tile in range(8):
            u = R.unpack_record(c.record(0, 0, tile, 0), 32, 128, 0, bits)
            w = R.rotate(x[32 * tile:32 * tile + 32], c.sigma)
            y = R.normalize(w, u["r16"], u["c16"])
            yhat = u["z16"][None] + u["s16"][None] * u["q"]
            assert np.all(np.abs(y - yhat) <= u["s16"][None] * 0.5 * 1.01 + 1e-3 * np.abs(y))
        kh, _ = R.dequantize(c, 256)
        mse[bits] = float(np.mean((kh[0, :, 0] - x) ** 2) / np.mean(x * x))
    assert 2.5 < mse[2] / mse[3] < 6 and 2.5 < mse[3] / mse[4] < 6, mse
