"""Pins of the oracle's cache semantics, decode attention and error split.

Attention is checked against torch's scaled_dot_product_attention (a library
routine) in float64 on the oracle's own dequantized K, V; the error split against
the identity and sign facts that follow from the ai-paper-analysis page's
section-2 equation.
"""
import numpy as np
import pytest
import torch

from oracle import kvarn_ref as R
from kv_cache_bit_amd import synth


def make_cache(B=1, H=1, T=256, cap=None, g=32, n_it=3, seed=0):
    cap = cap if cap is not None else ((T + g - 1) // g + 1) * g
    geom = R.Geom(B, H, 128, cap, g, n_it, 2)
    c = R.Cache(geom, synth.sign_vector(0))
    k, v = synth.kv_host(seed, B, T, H)
    R.quantize_prefill(c, k, v, T)
    return c, k, v


def sdpa(q, k, v, scale):
    """torch SDPA in float64; q [Hq][D], k, v [T][D] (one KV head)."""
    qt = torch.from_numpy(q)[None, :, None, :]                       # [1][Hq][1][D]
    kt = torch.from_numpy(k)[None, None].expand(1, q.shape[0], -1, -1).contiguous()
    vt = torch.from_numpy(v)[None, None].expand(1, q.shape[0], -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, :, 0].numpy()


def test_header_fields():
    c, _, _ = make_cache(B=2, H=3, T=70)
    assert c.buf[0:4].view(np.uint32)[0] == R.MAGIC
    assert c.buf[4:8].view(np.uint32)[0] == 3
    assert c.buf[8:36].view(np.int32).tolist() == [2, 3, 128, 128, 32, 3, 2]
    assert np.all(c.lens == 70)
    assert c.g.header == 768 and c.g.total % 256 == 0


def test_header_sign_words():
    """Bytes 192..447 restate sigma as the sign bits of packed 16-bit pairs: word d has bit 15
    set iff sigma[2d] = -1 and bit 31 set iff sigma[2d + 1] = -1 (values worked by hand)."""
    sigma = np.ones(128)
    sigma[[1, 2, 4, 5, 127]] = -1
    c = R.Cache(R.Geom(1, 1, 128, 32, 32, 3, 2), sigma)
    words = c.buf[192:448].view(np.uint32)
    assert words[0] == 0x80000000            # (+1, -1)
    assert words[1] == 0x00008000            # (-1, +1)
    assert words[2] == 0x80008000            # (-1, -1)
    assert words[3] == 0                     # (+1, +1)
    assert words[63] == 0x80000000           # (+1, -1): channels 126, 127
    assert np.count_nonzero(words[4:63]) == 0
    # and XORed into a packed pair of fp16 or bf16 values it flips exactly those signs
    pair = np.array([1.5, -2.25], dtype=np.float16).view(np.uint32)[0]
    flipped = np.array([pair ^ words[2]], dtype=np.uint32).view(np.float16)
    assert flipped.tolist() == [-1.5, 2.25]
    pair = np.array([0xC010, 0x3FC0], dtype=np.uint16).view(np.uint32)[0]      # bf16 (-2.25, 1.5)
    flipped = R.bf16_to_f64(np.array([pair ^ words[1]], dtype=np.uint32).view(np.uint16))
    assert flipped.tolist() == [2.25, 1.5]


@pytest.mark.parametrize("T", [0, 5, 31, 32, 33, 100])
def test_prefill_equals_appends(T):
    """prefill(T) and T single-token appends from empty give the same bytes."""
    B, H = 2, 2
    geom = R.Geom(B, H, 128, 128, 32, 3, 2)
    k, v = synth.kv_host(4, B, T, H)
    a = R.Cache(geom, synth.sign_vector(0))
    R.quantize_prefill(a, k, v, T)
    b = R.Cache(geom, synth.sign_vector(0))
    R.quantize_prefill(b, k, v, 0)
    for t in range(T):
        R.append_decode(b, k[:, t], v[:, t])
    m = a.defined_mask()
    assert np.array_equal(m, b.defined_mask())
    assert np.array_equal(a.buf[m], b.buf[m])


def test_capacity_and_saturation_flags():
    geom = R.Geom(1, 1, 128, 32, 32, 3, 2)
    k, v = synth.kv_host(1, 1, 33, 1)
    c = R.Cache(geom, synth.sign_vector(0))
    R.quantize_prefill(c, k, v, 32)
    assert c.flags == 0
    R.append_decode(c, k[:, 32], v[:, 32])
    assert c.flags & R.FLAG_CAPACITY and np.all(c.lens == 32)
    k2 = k.copy()
    k2[0, 3, 0, 5] = 0x4780                                          # 65536 = 2^16: kept
    c2 = R.Cache(geom, synth.sign_vector(0))
    R.quantize_prefill(c2, k2, v, 10)
    assert c2.flags == 0 and c2.tail(0, 0, 0)[3, 5] == 0x4780
    k2[0, 3, 0, 5] = 0xC781                                          # -65792: beyond 2^16
    c3 = R.Cache(geom, synth.sign_vector(0))
    R.quantize_prefill(c3, k2, v, 10)
    assert c3.flags == R.FLAG_SATURATED
    assert c3.tail(0, 0, 0)[3, 5] == 0xC780 and c3.tail_values(0, 0, 0)[3, 5] == -65536.0


def test_dequantize_tail_exact_and_rows_past_length_zero():
    c, k, v = make_cache(T=70)
    kh, vh = R.dequantize(c, 80)
    assert np.array_equal(kh[0, 64:70, 0], R.canonicalize(k[0, 64:70, 0])[0])
    assert np.array_equal(vh[0, 64:70, 0], R.canonicalize(v[0, 64:70, 0])[0])
    assert np.all(kh[0, 70:] == 0) and np.all(vh[0, 70:] == 0)


def test_tail_only_attention_is_textbook_softmax():
    c, k, v = make_cache(T=20)
    q = synth.q_host(3, 1, 4)
    out = R.attn_decode(c, q, 4)
    kk = R.canonicalize(k[0, :, 0])[0]
    vv = R.canonicalize(v[0, :, 0])[0]
    ref = sdpa(R.bf16_to_f64(q[0]), kk, vv, 1 / np.sqrt(128))
    assert np.abs(out[0] - ref).max() < 1e-12


@pytest.mark.parametrize("T,Hq", [(256, 4), (250, 8), (70, 2)])
def test_attention_matches_library_on_dequantized_cache(T, Hq):
    B, H = 2, 2
    c, k, v = make_cache(B=B, H=H, T=T)
    q = synth.q_host(9, B, Hq)
    out = R.attn_decode(c, q, Hq)
    kh, vh = R.dequantize(c, T)
    grp = Hq // H
    for b in range(B):
        for h in range(H):
            ref = sdpa(R.bf16_to_f64(q[b, h * grp:(h + 1) * grp]), kh[b, :, h], vh[b, :, h], 1 / np.sqrt(128))
            assert np.abs(out[b, h * grp:(h + 1) * grp] - ref).max() < 1e-12


def test_attention_special_cases():
    c, k, v = make_cache(T=1)
    q = synth.q_host(1, 1, 1)
    assert np.array_equal(R.attn_decode(c, q, 1)[0, 0], R.canonicalize(v[0, 0, 0])[0])
    c, k, v = make_cache(T=100)
    zero_q = np.zeros((1, 1, 128), dtype=np.uint16)
    _, vh = R.dequantize(c, 100)
    assert np.allclose(R.attn_decode(c, zero_q, 1)[0, 0], vh[0, :, 0].mean(axis=0), rtol=0, atol=1e-12)
    empty = R.Cache(R.Geom(1, 1, 128, 64, 32, 3, 2), synth.sign_vector(0))
    assert np.all(R.attn_decode(empty, q, 1) == 0)


def test_prerotated_query_flag():
    c, _, _ = make_cache(T=100)
    qr_bits = synth.q_host(5, 1, 2)                                  # taken as q H_D, exact bf16
    out = R.attn_decode(c, qr_bits, 2, flags=R.Q_PREROTATED)
    q = R.unrotate(R.bf16_to_f64(qr_bits), c.sigma)
    kh, vh = R.dequantize(c, 100)
    ref = sdpa(q[0], kh[0, :, 0], vh[0, :, 0], 1 / np.sqrt(128))
    assert np.abs(out[0] - ref).max() < 1e-12


def test_scores_invariant_under_joint_rotation():
    c, _, _ = make_cache(T=96)
    q = R.bf16_to_f64(synth.q_host(2, 1, 1))[0, 0]
    k_orig = R.stream_values(c, 0, 0, 0)
    k_rot = R.stream_values(c, 0, 0, 0, rotated=True)
    assert np.abs(k_orig @ q - k_rot @ R.rotate(q, c.sigma)).max() < 1e-11


def test_error_split_identity_and_signs():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((200, 128))
    xh = x + 0.3 * rng.standard_normal((200, 128))
    em, ed = R.error_split(x, xh)
    assert np.abs(em + ed - (xh - x)).max() < 1e-12
    # E_M is parallel to x; E_D . x <= 0 (equality only when xhat is parallel to x)
    ux = x / np.linalg.norm(x, axis=-1, keepdims=True)
    assert np.abs(em - np.sum(em * ux, axis=-1, keepdims=True) * ux).max() < 1e-12
    assert np.all(np.sum(ed * x, axis=-1) <= 1e-12)
    # pure scaling: no direction error; pure rotation: no magnitude error
    em, ed = R.error_split(x, 2 * x)
    assert np.abs(ed).max() < 1e-12 and np.abs(em - x).max() < 1e-12
    s = synth.sign_vector(3)
    em, ed = R.error_split(x, R.rotate(x, s))
    assert np.abs(em).max() < 1e-12
    # zero-norm conventions
    em, ed = R.error_split(np.zeros(4), np.ones(4))
    assert np.all(em == 0) and np.all(ed == 1)
    em, ed = R.error_split(np.ones(4), np.zeros(4))
    assert np.all(ed == 0) and np.all(em == -1)


def test_quality_guard_varn_beats_hadamard_only():
    """Synthetic face of the pages' claim (researchpapers page; ai-paper-analysis
    sections 2 and 5 ablation): with outlier tokens, H + VarN has a far smaller
    per-token relative error than H alone (n_it = 0)."""
    errs = {}
    for n_it in (0, 3):
        geom = R.Geom(1, 1, 128, 256, 32, n_it, 2)
        c = R.Cache(geom, synth.sign_vector(0))
        k, v = synth.kv_host(0, 1, 256, 1)
        R.quantize_prefill(c, k, v, 256)
        kh, vh = R.dequantize(c, 256)
        e = [R.relative_token_error(R.canonicalize(b[0, :, 0])[0], h[0, :, 0]).mean()
             for b, h in ((k, kh), (v, vh))]
        errs[n_it] = np.mean(e)
    assert errs[3] < 0.2
    assert errs[3] < 0.1 * errs[0]


def _fresh(T, G=32, cap=96, B=2, H=2, seed=31):
    k, v = synth.kv_host(seed, B, T + 1, H)
    c = R.Cache(R.Geom(B, H, 128, cap, G, 3, 2), synth.sign_vector(4))
    R.quantize_prefill(c, k, v, T)
    return c, k, v


@pytest.mark.parametrize("T", [40, 0, 17])
def test_append_attn_step_equals_append_then_attend(T):
    """A step whose token does not complete a group: the fused step is the append
    followed by the attention, on the same bytes."""
    a, k, v = _fresh(T)
    b, _, _ = _fresh(T)
    q = synth.q_host(5, 2, 4)
    fused = R.append_attn_decode(a, k[:, T], v[:, T], q, 4)
    R.append_decode(b, k[:, T], v[:, T])
    assert np.array_equal(fused, R.attn_decode(b, q, 4))
    assert np.array_equal(a.buf, b.buf)


def test_append_attn_step_completing_a_group_reads_it_unquantized():
    """A step whose token completes a group (T = 63, G = 32): the attention reads tile 0
    from its record and the 32 tokens of the completed group as given (the 31 bf16 tail
    tokens, then the new token); afterwards the cache equals the plain append's, and
    attending again reads the group quantized, which differs."""
    T = 63
    a, k, v = _fresh(T)
    before, _, _ = _fresh(T)
    b, _, _ = _fresh(T)
    q = synth.q_host(6, 2, 4)
    fused = R.append_attn_decode(a, k[:, T], v[:, T], q, 4)
    qq = R.bf16_to_f64(q)
    for bb in range(2):
        for h in range(2):
            kv = []
            for s, bits in ((0, k), (1, v)):
                rec = R.unpack_record(before.record(bb, h, 0, s), 32, 128, s)
                tile0 = R.unrotate(R.dequantize_tile(rec["q"], rec["r16"], rec["c16"], rec["s16"], rec["z16"]),
                                   before.sigma)
                tail = before.tail_values(bb, h, s)[:31]
                new = R.bf16_to_f64(bits[bb, T, h])
                kv.append(np.vstack([tile0, tail, new[None]]))
            for gi in range(2 * h, 2 * h + 2):
                lg = kv[0] @ qq[bb, gi] / np.sqrt(128)
                p = np.exp(lg - lg.max())
                assert np.allclose(fused[bb, gi], (p / p.sum()) @ kv[1], rtol=1e-12, atol=1e-12)
    R.append_decode(b, k[:, T], v[:, T])
    assert np.array_equal(a.buf, b.buf)
    assert not np.allclose(fused, R.attn_decode(b, q, 4), rtol=1e-6)


def test_append_attn_step_on_full_sequence():
    a, k, v = _fresh(96, cap=96)
    q = synth.q_host(7, 2, 4)
    b, _, _ = _fresh(96, cap=96)
    fused = R.append_attn_decode(a, k[:, 95], v[:, 95], q, 4)
    assert np.array_equal(fused, R.attn_decode(b, q, 4))
    assert a.flags & R.FLAG_CAPACITY and np.all(a.lens == 96)
