"""Pins of the oracle's VarN (ai-paper-analysis page, section 3.2: token-axis then
channel-axis variance normalization, repeated 2-3 times, Sinkhorn-Knopp like).
"""
import numpy as np

from oracle import kvarn_ref as R
from kv_cache_bit_amd import synth


def c1_tiles(seed=0, tokens=256, g=32, law="lognormal", **kw):
    """Rotated G x 128 tiles from the single-head outlier workload (K and V stacked)."""
    k, v = synth.kv_host(seed, 1, tokens, 1, 128, law=law, **kw)
    s = synth.sign_vector(0, 128)
    xs = [R.canonicalize(b[0, :, 0])[0] for b in (k, v)]
    w = np.stack([R.rotate(x, s) for x in xs])                    # [2][T][D]
    return w.reshape(-1, g, 128)


def test_rank_one_closed_form():
    """If W^2 = alpha_t beta_j, one iteration gives r_t = sqrt(alpha_t mean(beta)),
    c_j = sqrt(beta_j / mean(beta)) and |Y| = 1 everywhere (both axes exactly 1)."""
    rng = np.random.default_rng(0)
    alpha = rng.uniform(0.1, 30, 32)
    beta = rng.uniform(0.01, 5, 128)
    sgn = rng.choice([-1.0, 1.0], size=(32, 128))
    w = sgn * np.sqrt(alpha[:, None] * beta[None, :])
    r, c = R.varn(w, 1)
    assert np.allclose(r, np.sqrt(alpha * beta.mean()), rtol=1e-13)
    assert np.allclose(c, np.sqrt(beta / beta.mean()), rtol=1e-13)
    y = w / (r[:, None] * c[None, :])
    assert np.allclose(np.abs(y), 1.0, rtol=1e-13)
    # further iterations are at the fixed point
    r3, c3 = R.varn(w, 3)
    assert np.allclose(r3, r, rtol=1e-13) and np.allclose(c3, c, rtol=1e-13)


def test_token_pass_first_then_channel():
    """One iteration on a 2x2 example, worked by hand:
    W = [[2, 0], [0, 4]] -> token pass r = [sqrt(2), sqrt(8)] (row mean squares 2 and 8),
    then Y = [[sqrt2, 0], [0, sqrt2]], channel mean squares 1 and 1 -> c = [1, 1]."""
    w = np.array([[2.0, 0.0], [0.0, 4.0]])
    r, c = R.varn(w, 1)
    assert np.allclose(r, [np.sqrt(2), np.sqrt(8)], rtol=1e-15)
    assert np.allclose(c, [1.0, 1.0], rtol=1e-15)
    # channel pass uses the token-normalized values: W = [[1, 1], [3, 3]]
    # token pass: ms = [1, 9] -> r = [1, 3]; Y = [[1,1],[1,1]] -> c = [1, 1]
    r, c = R.varn(np.array([[1.0, 1.0], [3.0, 3.0]]), 1)
    assert np.allclose(r, [1, 3]) and np.allclose(c, [1, 1])
    # and a case where the channel pass matters: W = [[1, 3], [1, 3]]
    # token pass: ms = [5, 5] -> r = sqrt5; Y = [[1,3],[1,3]]/sqrt5 -> channel ms = [1/5, 9/5]
    r, c = R.varn(np.array([[1.0, 3.0], [1.0, 3.0]]), 1)
    assert np.allclose(r, [np.sqrt(5)] * 2) and np.allclose(c, [np.sqrt(0.2), np.sqrt(1.8)])


def test_sinkhorn_fixed_point_many_iterations():
    w = c1_tiles()[:4]
    r, c = R.varn(w, 200)
    y = w / (r[..., :, None] * c[..., None, :])
    ms_t, ms_j = R.axis_mean_squares(y)
    assert np.abs(ms_j - 1).max() < 1e-12
    assert np.abs(ms_t - 1).max() < 1e-8


def test_c1_tiles_near_unit_after_three_iterations():
    w = c1_tiles()
    t = R.quantize_tile(w, 3)
    ms_t, ms_j = R.axis_mean_squares(t["y"])
    assert np.abs(ms_j - 1).max() <= 3e-3      # only fp16 scale rounding remains on the last axis
    assert np.abs(ms_t - 1).max() <= 3e-2
    worst = []
    for n_it in range(1, 7):
        r, c = R.varn(w, n_it)
        y = w / (r[..., :, None] * c[..., None, :])
        worst.append(np.abs(R.axis_mean_squares(y)[0] - 1).max())
    assert all(a >= b for a, b in zip(worst, worst[1:]))


def test_g64_two_iterations_spike_law():
    w = c1_tiles(seed=3, tokens=512, g=64, law="spike", p=0.02, factor=50.0)
    t = R.quantize_tile(w, 2)
    ms_t, ms_j = R.axis_mean_squares(t["y"])
    assert np.abs(ms_j - 1).max() <= 3e-3
    assert np.abs(ms_t - 1).max() <= 5e-2


def test_power_of_two_token_equivariance():
    """Scaling one token by 2^k changes only its r (by exactly 2^k); c, s, z, q unchanged."""
    w = c1_tiles()[:3]
    base = R.quantize_tile(w, 3)
    for k in (-5, 3, 9):
        w2 = w.copy()
        w2[:, 7] *= 2.0 ** k
        t = R.quantize_tile(w2, 3)
        assert np.array_equal(t["r16"][:, 7], base["r16"][:, 7] * 2.0 ** k)
        others = np.arange(32) != 7
        assert np.array_equal(t["r16"][:, others], base["r16"][:, others])
        for key in ("c16", "s16", "z16", "q"):
            assert np.array_equal(t[key], base[key]), key


def test_zero_iterations_is_plain_per_channel_minmax():
    w = c1_tiles()[:2]
    t = R.quantize_tile(w, 0)
    assert np.all(t["r16"] == 1) and np.all(t["c16"] == 1)
    assert np.array_equal(t["z16"], R.fp16_round(w.min(axis=-2)))


def test_degenerate_tiles():
    g, d = 32, 128
    z = np.zeros((g, d))
    t = R.quantize_tile(z, 3)
    assert np.all(t["r16"] == 1) and np.all(t["c16"] == 1)
    assert np.all(t["s16"] == 0) and np.all(t["z16"] == 0) and np.all(t["q"] == 0)
    assert np.all(R.dequantize_tile(t["q"], t["r16"], t["c16"], t["s16"], t["z16"]) == 0)
    # one zero row keeps r = 1 and dequantizes to exactly 0
    rng = np.random.default_rng(5)
    w = rng.standard_normal((g, d))
    w[4] = 0
    t = R.quantize_tile(w, 3)
    assert t["r16"][4] == 1.0
    deq = R.dequantize_tile(t["q"], t["r16"], t["c16"], t["s16"], t["z16"])
    # row 4: Y = 0 -> code of 0 on a grid z + s k; it need not be exact, but must be the nearest level
    lv = t["z16"][None, :] + t["s16"][None, :] * np.arange(4)[:, None]
    assert np.all(np.abs(deq[4] / (t["r16"][4] * t["c16"])) <= np.abs(lv).min(axis=0) + 1e-12)
    # a constant column: s = 0, all codes 0, dequantizes to r c z
    w = rng.standard_normal((g, d))
    w[:, 9] = 0.75
    t = R.quantize_tile(w, 0)
    assert t["s16"][9] == 0 and np.all(t["q"][:, 9] == 0)
    assert np.all(R.dequantize_tile(t["q"], t["r16"], t["c16"], t["s16"], t["z16"])[:, 9] == 0.75)


def test_scale_clamp_flag():
    w = np.full((32, 128), 1e-9)
    t = R.quantize_tile(w, 3)
    assert t["flags"] & R.FLAG_SCALE_CLAMPED
    assert np.all(t["r16"] >= R.SCALE_MIN)


def test_rank_one_tile_end_to_end_closed_form():
    """The whole tile quantizer on a rank-one tile W = sgn * sqrt(alpha_t beta_j), with
    both signs in every channel. From the closed form above: r16 = fp16(sqrt(alpha_t mean
    beta)) and c16 = fp16(sqrt(beta_j / mean beta)); Y = W / (r16 c16) is +-1 up to the two
    fp16 roundings, so each channel's grid spans [-1, 1]: z near -1, s near 2/(2^bits - 1),
    and every code is 0 where sgn < 0 and the top level 2^bits - 1 where sgn > 0, far from
    any rounding edge. Dequantization returns W to the grid's resolution."""
    rng = np.random.default_rng(7)
    alpha = rng.uniform(0.25, 40.0, 32)
    beta = rng.uniform(0.05, 6.0, 128)
    sgn = rng.choice([-1.0, 1.0], size=(32, 128))
    sgn[0], sgn[1] = 1.0, -1.0  # both signs in every channel
    w = sgn * np.sqrt(alpha[:, None] * beta[None, :])
    r_cf = np.sqrt(alpha * beta.mean())
    c_cf = np.sqrt(beta / beta.mean())
    for bits in (2, 3, 4):
        top = 2 ** bits - 1
        t = R.quantize_tile(w, 3, 0, bits)
        assert np.array_equal(t["r16"], R.fp16_round(r_cf))
        assert np.array_equal(t["c16"], R.fp16_round(c_cf))
        assert np.array_equal(t["q"], np.where(sgn > 0, top, 0))
        # Y within 2^-9 of +-1 moves min and max by that much: a few fp16 ulps at most
        assert np.all(np.abs(t["z16"] + 1.0) <= 2.0 ** -8)
        assert np.all(np.abs(t["s16"] - 2.0 / top) <= 2.0 ** -8 * (2.0 / top) + 2.0 ** -11)
        assert t["flags"] == 0
        w_hat = R.dequantize_tile(t["q"], t["r16"], t["c16"], t["s16"], t["z16"])
        assert np.all(np.abs(w_hat - w) <= 2.0 ** -7 * np.abs(w))
