"""3- and 4-bit codes on the GPU against the oracle, through the C ABI: the prefill parity
chain with the fp32 intermediates, append equal to prefill, the multi-layer call equal to
per-layer calls, dequantization, decode
attention (plain and fused), a paged cache, and the reconstruction error falling with the
width.
"""
import numpy as np
import pytest
import torch

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth
from oracle import kvarn_ref as R

from parity import GpuCache, check_attention, check_prefill, from_u16, gpu_prefill

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("G,n_it,T,variant", [(32, 3, 250, 0), (64, 2, 300, 0), (32, 2, 96, 1)])
def test_prefill_bits_parity(bits, G, n_it, T, variant):
    say("prefill bits", bits, G, n_it, T, variant)
    B, H = 2, 2
    k, v = synth.kv_host(90 + bits, B, T, H)
    gc = GpuCache(B, H, 320, G, n_it, variant=variant, bits=bits)
    w, y = gpu_prefill(gc, k, v, T, debug=True)
    say("stats", check_prefill(gc, k, v, T, w=w, y=y))


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("G", [32, 64])
def test_append_equals_prefill_bits(bits, G):
    T = 2 * G + 7
    say("append==prefill bits", bits, G, T)
    B, H = 2, 2
    k, v = synth.kv_host(95, B, T, H)
    a = GpuCache(B, H, 4 * G, G, 3, bits=bits)
    b = GpuCache(B, H, 4 * G, G, 3, bits=bits)
    gpu_prefill(a, k, v, T)
    kd, vd = from_u16(k), from_u16(v)
    K.kvarn_append_tokens(b.g, b.buf, kd[:, :G + 3].contiguous(), vd[:, :G + 3].contiguous(), G + 3)
    for t in range(G + 3, T):
        K.kvarn_append_decode(b.g, b.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
    ha, hb = a.host_cache(), b.host_cache()
    m = ha.defined_mask()
    assert np.array_equal(m, hb.defined_mask()) and np.array_equal(ha.buf[m], hb.buf[m])


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("G", [32, 64])
def test_prefill_layers_bits(bits, G):
    """kvarn_quantize_prefill_layers over 3 caches of 3- or 4-bit codes writes the bytes and
    flags of 3 kvarn_quantize_prefill calls; the first layer also goes through the chain."""
    T, n = 2 * G + 9, 3
    say("prefill layers bits", bits, G, T)
    B, H = 2, 2
    ins = [synth.kv_host(60 + i, B, T, H) for i in range(n)]
    a = [GpuCache(B, H, 4 * G, G, 3, seed_sigma=i, bits=bits) for i in range(n)]
    b = [GpuCache(B, H, 4 * G, G, 3, seed_sigma=i, bits=bits) for i in range(n)]
    for i in range(n):
        gpu_prefill(a[i], ins[i][0], ins[i][1], T)
    K.kvarn_quantize_prefill_layers(b[0].g, [c.buf for c in b], [from_u16(k) for k, _ in ins],
                                    [from_u16(v) for _, v in ins], T)
    torch.cuda.synchronize()
    for i in range(n):
        ha, hb = a[i].host_cache(), b[i].host_cache()
        m = ha.defined_mask()
        assert np.array_equal(ha.buf[m], hb.buf[m]), i
        assert K.kvarn_cache_flags(a[i].buf) == K.kvarn_cache_flags(b[i].buf), i
    check_prefill(b[0], ins[0][0], ins[0][1], T)


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("G", [32, 64])
def test_dequantize_bits_parity(bits, G):
    say("dequantize bits", bits, G)
    B, H, T, maxT = 2, 2, 150, 160
    k, v = synth.kv_host(96, B, T, H)
    gc = GpuCache(B, H, 256, G, 3, bits=bits)
    gpu_prefill(gc, k, v, T)
    kr, vr = R.dequantize(gc.host_cache(), maxT)
    for dt in (K.KVARN_OUT_F32, K.KVARN_OUT_BF16):
        tdt = torch.float32 if dt == K.KVARN_OUT_F32 else torch.bfloat16
        ko = torch.full((B, maxT, H, 128), 7.0, dtype=tdt, device="cuda")
        vo = torch.full((B, maxT, H, 128), 7.0, dtype=tdt, device="cuda")
        K.kvarn_dequantize(gc.g, gc.buf, ko, vo, maxT, dt)
        torch.cuda.synchronize()
        for got, ref in ((ko, kr), (vo, vr)):
            g = got.float().cpu().numpy().astype(np.float64)
            rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
            if dt == K.KVARN_OUT_F32:
                assert np.all(np.abs(g - ref) <= 1e-5 * np.maximum(rms, 1e-30) + 1e-30)
            else:  # one bf16 rounding of a value that already carries the fp32 error
                assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) * 1.01 + 1e-5 * rms + 1e-30)
            assert np.all(g[:, T:] == 0)


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("T,Hq,H,G", [(250, 8, 2, 32), (1000, 4, 2, 64), (33, 2, 1, 32), (600, 6, 2, 32)])
def test_attention_bits_parity(bits, T, Hq, H, G):
    say("attn bits", bits, T, Hq, H, G)
    B = 2
    k, v = synth.kv_host(97, B, T, H)
    gc = GpuCache(B, H, 1024, G, 3, bits=bits)
    gpu_prefill(gc, k, v, T)
    qb = synth.q_host(98, B, Hq)
    ws, n = K.alloc_workspace(gc.g, Hq)
    out = torch.full((B, Hq, 128), float("nan"), device="cuda")
    K.kvarn_attn_decode(gc.g, gc.buf, from_u16(qb), Hq, 0.0, 0, ws, n, out)
    torch.cuda.synchronize()
    say("worst rel", check_attention(out.cpu().numpy().astype(np.float64), gc.host_cache(), qb, Hq))


@pytest.mark.parametrize("bits", [3, 4])
def test_fused_step_and_paged_bits(bits):
    """The fused step on a paged 3/4-bit cache equals the oracle's step, and the bytes
    equal a per-sequence cache fed the same calls."""
    say("fused paged bits", bits)
    B, H, Hq, G = 2, 2, 8, 32
    cap, tiles = 4 * G, 4
    T0, steps = 2 * G - 3, 6
    k, v = synth.kv_host(99, B, T0 + steps, H)
    kd, vd = from_u16(k), from_u16(v)
    g = K.geom(B, H, cap, G, 3, bits=bits, num_pages=B * tiles)
    og = R.Geom(B, H, 128, cap, G, 3, bits, 0, B * tiles)
    sig = synth.sign_vector(0)
    buf = K.alloc_cache(g, sig)
    pages = torch.from_numpy(np.arange(B * tiles, dtype=np.int32)[::-1].copy().reshape(B, tiles)).cuda()
    K.kvarn_cache_set_pages(g, buf, pages, 0, tiles)
    K.kvarn_quantize_prefill(g, buf, kd[:, :T0].contiguous(), vd[:, :T0].contiguous(), T0)
    flat = GpuCache(B, H, cap, G, 3, bits=bits)
    gpu_prefill(flat, k, v, T0)
    ws, n = K.alloc_workspace(g, Hq)
    for t in range(T0, T0 + steps):
        qb = synth.q_host(200 + t, B, Hq)
        torch.cuda.synchronize()
        hc = R.Cache(og, sig)
        hc.buf[:] = buf.cpu().numpy()
        ref = R.append_attn_decode(hc, k[:, t], v[:, t], qb, Hq)
        out = torch.full((B, Hq, 128), float("nan"), device="cuda")
        K.kvarn_append_attn_decode(g, buf, kd[:, t].contiguous(), vd[:, t].contiguous(), from_u16(qb), Hq, 0.0, 0,
                                   ws, n, out)
        K.kvarn_append_decode(flat.g, flat.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        for bb in range(B):
            for qq in range(Hq):
                m = np.abs(ref[bb, qq]).max()
                assert np.abs(got[bb, qq] - ref[bb, qq]).max() <= 2e-3 * m, (t, bb, qq)
    hp = R.Cache(og, sig)
    hp.buf[:] = buf.cpu().numpy()
    hf = flat.host_cache()
    for bb in range(B):
        for h in range(H):
            for s in range(2):
                nlen = int(hf.lens[bb, h, s])
                assert nlen == int(hp.lens[bb, h, s]) == T0 + steps
                for tile in range(nlen // G):
                    assert np.array_equal(hp.record(bb, h, tile, s), hf.record(bb, h, tile, s))


def test_error_falls_with_bits_on_gpu():
    say("error vs bits")
    k, v = synth.kv_host(5, 1, 512, 2)
    errs = {}
    for bits in (2, 3, 4):
        gc = GpuCache(1, 2, 512, 32, 3, bits=bits)
        gpu_prefill(gc, k, v, 512)
        ko = torch.empty(1, 512, 2, 128, device="cuda")
        vo = torch.empty(1, 512, 2, 128, device="cuda")
        K.kvarn_dequantize(gc.g, gc.buf, ko, vo, 512, K.KVARN_OUT_F32)
        torch.cuda.synchronize()
        x = R.canonicalize(k)[0]
        errs[bits] = float(np.mean(R.relative_token_error(x, ko.cpu().numpy())))
    say("errors", errs)
    assert errs[2] > 2.5 * errs[3] > 2.5 * 2.5 * errs[4]
