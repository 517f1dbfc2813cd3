"""Pins of the oracle's ablation variants (ai-paper-analysis page, section 5, ablations:
Hadamard only, VarN only, VarN along the token axis only, along the channel axis only),
and of the centered-variance reading kept as a further switch.

Each variant is pinned to what it reduces to: a single pass of one axis is a plain
root-mean-square (or standard deviation) of that axis; no rotation with no VarN is the
per-channel 4-level min/max quantizer applied to the tokens themselves, checked through
its invariants (every value on its channel's grid, error at most half a step).
"""
import numpy as np
import pytest

from oracle import kvarn_ref as R
from kv_cache_bit_amd import synth


def tiles(seed=0, tokens=128, g=32):
    k, v = synth.kv_host(seed, 1, tokens, 1, 128)
    s = synth.sign_vector(0, 128)
    xs = [R.canonicalize(b[0, :, 0])[0] for b in (k, v)]
    return np.stack([R.rotate(x, s) for x in xs]).reshape(-1, g, 128)


@pytest.mark.parametrize("n_it", [1, 3])
def test_token_axis_only_is_token_rms(n_it):
    """Without the channel pass the token pass has nothing to react to after the first
    iteration: r_t = |w_t| / sqrt(D) and c = 1, for any number of iterations."""
    w = tiles()
    r, c = R.varn(w, n_it, R.VARIANT_NO_CHANNEL_PASS)
    assert np.allclose(r, np.linalg.norm(w, axis=-1) / np.sqrt(128), rtol=1e-13)
    assert np.all(c == 1.0)


@pytest.mark.parametrize("n_it", [1, 3])
def test_channel_axis_only_is_channel_rms(n_it):
    """Without the token pass: c_j = |w_.j| / sqrt(G) and r = 1."""
    w = tiles()
    r, c = R.varn(w, n_it, R.VARIANT_NO_TOKEN_PASS)
    assert np.allclose(c, np.linalg.norm(w, axis=-2) / np.sqrt(w.shape[-2]), rtol=1e-13)
    assert np.all(r == 1.0)


def test_no_pass_at_all_is_identity_scales():
    w = tiles()[:2]
    r, c = R.varn(w, 3, R.VARIANT_NO_TOKEN_PASS | R.VARIANT_NO_CHANNEL_PASS)
    assert np.all(r == 1.0) and np.all(c == 1.0)


def test_centered_by_hand():
    """W = [[1, 3], [1, 3]]: the centered token pass sees row variance 1 (mean 2) and keeps
    r = 1; the channels are then constant (variance 0) and keep c = 1. The mean-square
    reading gives r = sqrt(5) instead (worked in the VarN pins)."""
    r, c = R.varn(np.array([[1.0, 3.0], [1.0, 3.0]]), 1, R.VARIANT_CENTERED)
    assert np.allclose(r, [1.0, 1.0], rtol=1e-15) and np.allclose(c, [1.0, 1.0], rtol=1e-15)


def test_centered_token_pass_is_std():
    w = tiles()
    r, _ = R.varn(w, 1, R.VARIANT_CENTERED | R.VARIANT_NO_CHANNEL_PASS)
    assert np.allclose(r, np.std(w, axis=-1), rtol=1e-12)


def test_centered_equals_mean_square_on_zero_mean_lines():
    """Rows of a Sylvester Hadamard matrix other than the first have zero mean; scaled
    per row, the centered and mean-square token passes agree (r_t = a_t)."""
    a = np.array([1.0, 2.0, 0.5, 3.0])
    w = np.stack([R.hadamard_sylvester(8)[i, :] for i in (1, 2, 3, 5)]).astype(np.float64) * a[:, None]
    assert np.allclose(w.mean(axis=-1), 0.0)
    r0, _ = R.varn(w, 1, R.VARIANT_NO_CHANNEL_PASS)
    r1, _ = R.varn(w, 1, R.VARIANT_NO_CHANNEL_PASS | R.VARIANT_CENTERED)
    assert np.allclose(r0, r1, rtol=1e-14) and np.allclose(r0, a, rtol=1e-14)


def make_cache(variant, n_it=3, T=96, G=32, seed=3):
    k, v = synth.kv_host(seed, 1, T, 2)
    c = R.Cache(R.Geom(1, 2, 128, 128, G, n_it, 2, variant), synth.sign_vector(5))
    R.quantize_prefill(c, k, v, T)
    return c, k, v


def test_variant_in_header():
    c, _, _ = make_cache(R.VARIANT_NO_ROTATION | R.VARIANT_NO_TOKEN_PASS)
    assert c.buf[R.VARIANT_OFFSET:R.VARIANT_OFFSET + 4].view(np.uint32)[0] == 5
    c0, _, _ = make_cache(0)
    assert c0.buf[R.VARIANT_OFFSET:R.VARIANT_OFFSET + 4].view(np.uint32)[0] == 0


def test_no_rotation_no_varn_is_per_channel_minmax():
    """No rotation and no VarN: every dequantized tile value of channel j lies on that
    channel's 4-level grid {z + s k}, the grid's ends match the channel's min and max to
    fp16 rounding, and the error is at most half a step (plus fp16 rounding of s, z)."""
    c, k, v = make_cache(R.VARIANT_NO_ROTATION, n_it=0, T=96)
    kh, vh = R.dequantize(c, 96)
    for x_bits, xh in ((k, kh), (v, vh)):
        x = R.canonicalize(x_bits)[0]
        for h in range(2):
            for t0 in range(0, 96, 32):
                xt, ht = x[0, t0:t0 + 32, h], xh[0, t0:t0 + 32, h]
                mn, mx = xt.min(axis=0), xt.max(axis=0)
                step = (mx - mn) / 3
                lv = (ht - mn) / np.where(step > 0, step, 1)
                assert np.all(np.abs(lv - np.rint(lv)) < 2e-3), "value off its channel's grid"
                assert np.all(np.abs(ht - xt) <= step / 2 + 1e-3 * (np.abs(mn) + np.abs(mx)) + 1e-12)
                assert np.allclose(ht.min(axis=0), mn, rtol=2e-3, atol=1e-6)
                assert np.allclose(ht.max(axis=0), mx, rtol=2e-3, atol=1e-6)


def test_no_rotation_attention_ignores_prerotated_flag():
    """With the identity in place of H_D the rotated and original spaces coincide, so the
    Q_PREROTATED flag changes nothing; the result is softmax attention over the
    dequantized cache computed by its definition."""
    c, _, _ = make_cache(R.VARIANT_NO_ROTATION, T=80)
    qb = synth.q_host(9, 1, 4)
    a = R.attn_decode(c, qb, 4)
    b = R.attn_decode(c, qb, 4, flags=R.Q_PREROTATED)
    assert np.array_equal(a, b)
    kh, vh = R.dequantize(c, 80)
    q = R.bf16_to_f64(qb)
    for gi in range(4):
        h = gi // 2
        lg = kh[0, :, h] @ q[0, gi] / np.sqrt(128)
        p = np.exp(lg - lg.max())
        assert np.allclose(a[0, gi], (p / p.sum()) @ vh[0, :, h], rtol=1e-12, atol=1e-12)


def test_channel_only_matches_hadamard_only_up_to_fp16():
    """With the grid per channel over the tile's tokens, a per-channel scale is absorbed
    by the grid's (s, z): channel-axis-only VarN reconstructs what no VarN does, except
    where the fp16 rounding of c, s and z moves a value across a rounding boundary."""
    a, _, _ = make_cache(R.VARIANT_NO_TOKEN_PASS, n_it=2)
    b, _, _ = make_cache(0, n_it=0)
    for h in range(2):
        for s in range(2):  # compared in the rotated basis, where one code is one value
            xa = R.stream_values(a, 0, h, s, rotated=True)
            xb = R.stream_values(b, 0, h, s, rotated=True)
            close = np.isclose(xa, xb, rtol=5e-3, atol=1e-3 * np.abs(xb).max())
            assert close.mean() > 0.99


def test_ablation_error_order_on_outlier_tokens():
    """On the outlier-token workload (lognormal token norms), full KVarN reconstructs
    tokens far better than Hadamard only, than VarN without the rotation and than VarN
    along the channel axis only (section 5 reports the ablations as accuracy, here they
    are error). Token-axis-only VarN comes within a few percent of the full method: with
    the grid per channel, the channel scales act only through their effect on r."""
    T = 512
    k, v = synth.kv_host(11, 1, T, 1, law="lognormal", p=0.1, sigma=1.5)
    x = R.canonicalize(k)[0][0, :, 0]

    def err(variant, n_it):
        c = R.Cache(R.Geom(1, 1, 128, T, 32, n_it, 2, variant), synth.sign_vector(2))
        R.quantize_prefill(c, k, v, T)
        kh, _ = R.dequantize(c, T)
        return float(np.mean(R.relative_token_error(x, kh[0, :, 0])))

    full = err(0, 3)
    assert 2 * full < err(0, 0)
    assert 2 * full < err(R.VARIANT_NO_TOKEN_PASS, 3)
    assert 1.5 * full < err(R.VARIANT_NO_ROTATION, 3)
    assert abs(err(R.VARIANT_NO_CHANNEL_PASS, 3) / full - 1) < 0.05
