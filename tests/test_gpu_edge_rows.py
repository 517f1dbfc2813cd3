"""GPU parity on token rows at the edges of the input range, inside tiles of ordinary
outlier-bearing rows: all-zero rows, small rows (1e-6, 2^-22), and rows whose squares
would underflow fp32 (1e-30, and bf16 subnormals around 2^-128), which the kernels route
through the checked rotation with a per-token power-of-two scale; prefill, single-token
appends and multi-token appends in uneven chunks write the same bytes. The first token-axis
pass of VarN takes its sums from the Gram diagonal (exact products of the inputs on the
matrix cores); with one iteration those sums fix the token scale r directly. Run on an
MI355X: pytest -m gpu.
"""
import numpy as np
import pytest

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth

from parity import GpuCache, check_prefill, from_u16, gpu_prefill

pytestmark = pytest.mark.gpu


def chunked_appends(gc, kd, vd, T, G):
    """The T tokens through kvarn_append_tokens in uneven chunks from an emptied cache, so
    that completed groups mix tokens stored in the tail with new input rows."""
    t = 0
    for n in (5, G - 2, T):
        n = min(n, T - t)
        if n == 0:
            break
        K.kvarn_append_tokens(gc.g, gc.buf, kd[:, t:t + n].contiguous(), vd[:, t:t + n].contiguous(), n)
        t += n


def edge_rows_kv(seed, B, T, H, span):
    k, v = synth.kv_host(seed, B, T, H)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    for arr in (k, v):
        rows = rng.choice(span, size=10, replace=False)
        tiny = rng.standard_normal((2, B, H, 128)).astype(np.float32)
        for j in range(2):
            arr[:, rows[j]] = 0                                                         # all zero
            arr[:, rows[2 + j]] = synth.f32_to_bf16_bits(tiny[j] * 1e-6)
            arr[:, rows[4 + j]] = synth.f32_to_bf16_bits(tiny[j] * 2.0 ** -22)
            arr[:, rows[6 + j]] = synth.f32_to_bf16_bits(tiny[j] * 1e-30)                # squares below fp32
            arr[:, rows[8 + j]] = synth.f32_to_bf16_bits(tiny[j] * np.float32(2.0 ** -128))  # bf16 subnormals
    return k, v


@pytest.mark.parametrize("G,n_it", [(32, 1), (32, 3), (64, 2)])
def test_prefill_zero_and_tiny_token_rows(G, n_it):
    print("[case] zero/tiny token rows", G, n_it, flush=True)
    B, H = 1, 2
    T = 2 * G + 5
    k, v = edge_rows_kv(11, B, T, H, 2 * G)
    cap = (T // G + 1) * G
    gc = GpuCache(B, H, cap, G, n_it)
    gpu_prefill(gc, k, v, T)
    check_prefill(gc, k, v, T)
    # the same tokens through single-token appends give the same bytes
    ap = GpuCache(B, H, cap, G, n_it)
    gpu_prefill(ap, k, v, 0)
    kd, vd = from_u16(k), from_u16(v)
    for t in range(T):
        K.kvarn_append_decode(ap.g, ap.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
    ha, hb = gc.host_cache(), ap.host_cache()
    m = ha.defined_mask()
    assert np.array_equal(ha.buf[m], hb.buf[m])
    # and through multi-token appends in uneven chunks
    ch = GpuCache(B, H, cap, G, n_it)
    gpu_prefill(ch, k, v, 0)
    chunked_appends(ch, kd, vd, T, G)
    assert np.array_equal(ha.buf[m], ch.host_cache().buf[m])
    assert K.kvarn_cache_flags(ch.buf) == K.kvarn_cache_flags(gc.buf)


@pytest.mark.parametrize("G", [32, 64])
def test_non_finite_inputs(G):
    """NaN inputs are stored as 0 and raise KVARN_FLAG_NAN; infinities saturate at +-2^16
    (KVARN_FLAG_SATURATED). Checked through the parity chain (a full tile and the tail) and
    through single-token appends, which must give the same bytes and flags."""
    print("[case] non-finite inputs", G, flush=True)
    B, H = 1, 2
    T = 2 * G + 3
    k, v = synth.kv_host(21, B, T, H)
    k[0, 3, 0, 9] = 0x7FC0            # NaN in the first tile
    v[0, G + 1, 1, 100] = 0xFFC1      # -NaN in the second tile
    k[0, 2 * G + 1, 1, 0] = 0x7FC0    # NaN in the tail
    v[0, 7, 0, 50] = 0x7F80           # +inf in a tile
    cap = (T // G + 1) * G
    gc = GpuCache(B, H, cap, G, 3)
    gpu_prefill(gc, k, v, T)
    check_prefill(gc, k, v, T)
    want = K.KVARN_FLAG_NAN | K.KVARN_FLAG_SATURATED
    assert K.kvarn_cache_flags(gc.buf) == want
    ap = GpuCache(B, H, cap, G, 3)
    gpu_prefill(ap, k, v, 0)
    kd, vd = from_u16(k), from_u16(v)
    for t in range(T):
        K.kvarn_append_decode(ap.g, ap.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
    assert K.kvarn_cache_flags(ap.buf) == want
    ha, hb = gc.host_cache(), ap.host_cache()
    m = ha.defined_mask()
    assert np.array_equal(ha.buf[m], hb.buf[m])
    # and through multi-token appends in uneven chunks
    ch = GpuCache(B, H, cap, G, 3)
    gpu_prefill(ch, k, v, 0)
    chunked_appends(ch, kd, vd, T, G)
    assert K.kvarn_cache_flags(ch.buf) == want
    assert np.array_equal(ha.buf[m], ch.host_cache().buf[m])
