"""GPU parity of the ablation variants (ai-paper-analysis page, section 5: VarN without
the Hadamard rotation, VarN along one axis only; Hadamard only is varn_iters = 0, covered
by the prefill iteration tests) against the oracle, through the C ABI: prefill with the
fp32 intermediates, append equal to prefill, dequantization and decode attention.
"""
import numpy as np
import pytest
import torch

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth
from oracle import kvarn_ref as R

from parity import GpuCache, check_attention, check_prefill, from_u16, gpu_prefill

pytestmark = pytest.mark.gpu

VARIANTS = [K.KVARN_VARIANT_NO_ROTATION, K.KVARN_VARIANT_NO_CHANNEL_PASS, K.KVARN_VARIANT_NO_TOKEN_PASS,
            K.KVARN_VARIANT_NO_ROTATION | K.KVARN_VARIANT_NO_CHANNEL_PASS,
            K.KVARN_VARIANT_NO_ROTATION | K.KVARN_VARIANT_NO_TOKEN_PASS,
            K.KVARN_VARIANT_NO_CHANNEL_PASS | K.KVARN_VARIANT_NO_TOKEN_PASS,
            K.KVARN_VARIANT_CENTERED, K.KVARN_VARIANT_CENTERED | K.KVARN_VARIANT_NO_ROTATION,
            K.KVARN_VARIANT_CENTERED | K.KVARN_VARIANT_NO_CHANNEL_PASS]


def say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("G,n_it,T", [(32, 3, 250), (64, 2, 300)])
def test_prefill_variant_parity(variant, G, n_it, T):
    say("prefill variant", variant, G, n_it, T)
    B, H = 2, 2
    k, v = synth.kv_host(30 + variant, B, T, H)
    gc = GpuCache(B, H, 320, G, n_it, variant=variant)
    w, y = gpu_prefill(gc, k, v, T, debug=True)
    st = check_prefill(gc, k, v, T, w=w, y=y)
    say("stats", st)


@pytest.mark.parametrize("variant", [K.KVARN_VARIANT_NO_ROTATION, K.KVARN_VARIANT_NO_TOKEN_PASS,
                                     K.KVARN_VARIANT_CENTERED])
@pytest.mark.parametrize("G,n_it", [(32, 3), (64, 2)])
def test_append_equals_prefill_variant(variant, G, n_it):
    T = 2 * G + 5
    say("append==prefill variant", variant, G, n_it, T)
    B, H = 2, 2
    k, v = synth.kv_host(40, B, T, H)
    a = GpuCache(B, H, 4 * G, G, n_it, variant=variant)
    gpu_prefill(a, k, v, T)
    b = GpuCache(B, H, 4 * G, G, n_it, variant=variant)
    gpu_prefill(b, k, v, 0)
    kd, vd = from_u16(k), from_u16(v)
    for t in range(T):
        K.kvarn_append_decode(b.g, b.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
    ha, hb = a.host_cache(), b.host_cache()
    m = ha.defined_mask()
    assert np.array_equal(m, hb.defined_mask())
    assert np.array_equal(ha.buf[m], hb.buf[m])
    check_prefill(b, k, v, T)


@pytest.mark.parametrize("variant", [K.KVARN_VARIANT_NO_ROTATION,
                                     K.KVARN_VARIANT_NO_ROTATION | K.KVARN_VARIANT_NO_CHANNEL_PASS,
                                     K.KVARN_VARIANT_NO_TOKEN_PASS])
def test_dequantize_variant_parity(variant):
    say("dequantize variant", variant)
    B, H, T, maxT = 2, 2, 150, 160
    k, v = synth.kv_host(50, B, T, H)
    gc = GpuCache(B, H, 256, 32, 3, variant=variant)
    gpu_prefill(gc, k, v, T)
    kr, vr = R.dequantize(gc.host_cache(), maxT)
    ko = torch.full((B, maxT, H, 128), 7.0, device="cuda")
    vo = torch.full((B, maxT, H, 128), 7.0, device="cuda")
    K.kvarn_dequantize(gc.g, gc.buf, ko, vo, maxT, K.KVARN_OUT_F32)
    torch.cuda.synchronize()
    for got, ref in ((ko, kr), (vo, vr)):
        g = got.cpu().numpy().astype(np.float64)
        # without the rotation each value is r c (z + s q): three fp32 roundings
        rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
        assert np.all(np.abs(g - ref) <= 1e-5 * np.maximum(rms, 1e-30) + 1e-30)
        assert np.all(g[:, T:] == 0)


@pytest.mark.parametrize("variant", [K.KVARN_VARIANT_NO_ROTATION, K.KVARN_VARIANT_NO_CHANNEL_PASS])
@pytest.mark.parametrize("T,Hq,H,G", [(250, 8, 2, 32), (1000, 4, 2, 64), (20, 2, 1, 32)])
def test_attention_variant_parity(variant, T, Hq, H, G):
    say("attn variant", variant, T, Hq, H, G)
    B = 2
    k, v = synth.kv_host(60, B, T, H)
    gc = GpuCache(B, H, 1024, G, 3, variant=variant)
    gpu_prefill(gc, k, v, T)
    qb = synth.q_host(61, B, Hq)
    q = from_u16(qb)
    ws, n = K.alloc_workspace(gc.g, Hq)
    hc = gc.host_cache()
    for flags in (0, K.KVARN_Q_PREROTATED):  # the flag is a no-op without the rotation
        out = torch.full((B, Hq, 128), float("nan"), device="cuda")
        K.kvarn_attn_decode(gc.g, gc.buf, q, Hq, 0.0, flags, ws, n, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        if variant & K.KVARN_VARIANT_NO_ROTATION or flags == 0:
            worst = check_attention(got, hc, qb, Hq, flags=flags)
            say("worst rel", flags, worst)
