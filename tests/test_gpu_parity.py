"""GPU parity of libkvarn against the CPU oracle (run on an MI355X: pytest -m gpu).

Every case prints its name before touching the GPU so a failing run names it.
"""
import numpy as np
import pytest
import torch

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth
from oracle import kvarn_ref as R

from parity import GpuCache, check_attention, check_prefill, from_u16, gpu_prefill, to_u16

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def outlier_kv(seed, B, T, H, law="lognormal", **kw):
    return synth.kv_host(seed, B, T, H, law=law, **kw)


# ----------------------------------------------------------------------------- prefill
@pytest.mark.parametrize("T", [256, 250, 31, 0])
def test_prefill_single_head_parity(T):
    say("prefill c1", T)
    k, v = outlier_kv(0, 1, max(T, 1), 1)
    gc = GpuCache(1, 1, 288)
    w, y = gpu_prefill(gc, k, v, T, debug=True)
    st = check_prefill(gc, k, v, T, w, y)
    say("stats", st)


@pytest.mark.parametrize("n_it", [0, 1, 2, 8])
def test_prefill_iterations(n_it):
    say("prefill n_it", n_it)
    k, v = outlier_kv(1, 1, 256, 2)
    gc = GpuCache(1, 2, 256, 32, n_it)
    w, y = gpu_prefill(gc, k, v, 256, debug=True)
    check_prefill(gc, k, v, 256, w, y)


def test_prefill_batch_heads_ragged():
    say("prefill B=2 H=3 T=100")
    k, v = outlier_kv(2, 2, 100, 3)
    gc = GpuCache(2, 3, 128)
    w, y = gpu_prefill(gc, k, v, 100, debug=True)
    check_prefill(gc, k, v, 100, w, y)


@pytest.mark.parametrize("T", [512, 532])
def test_prefill_group64_spike_law(T):
    say("prefill G=64 spike", T)
    k, v = outlier_kv(3, 2, T, 2, law="spike", p=0.02, factor=50.0)
    gc = GpuCache(2, 2, 576, 64, 2)
    w, y = gpu_prefill(gc, k, v, T, debug=True)
    check_prefill(gc, k, v, T, w, y)


def test_prefill_student_t_heavy_tail():
    say("prefill student-t")
    k, v = synth.kv_host(4, 1, 320, 2, n_outlier_ch=8, ch_mult=30.0, law="student_t", nu=3.0)
    gc = GpuCache(1, 2, 320)
    w, y = gpu_prefill(gc, k, v, 320, debug=True)
    check_prefill(gc, k, v, 320, w, y)


def test_prefill_near_constant_tokens_clamp_path():
    """All tokens equal up to tiny noise: after rotation every channel is nearly constant,
    so the grid step is tiny next to |Y| and fp16 rounding of z can push u outside
    [0, 3]; the kernel must take its clamping path and still match the oracle."""
    say("near-constant tokens")
    rng = np.random.default_rng(21)
    base = rng.standard_normal(128) * 3.0
    x = base[None, None, None, :] + 1e-3 * rng.standard_normal((1, 64, 2, 128))
    k = synth.f32_to_bf16_bits(x.astype(np.float32))
    v = synth.f32_to_bf16_bits((x[:, ::-1] * 0.5).astype(np.float32))
    gc = GpuCache(1, 2, 64)
    w, y = gpu_prefill(gc, k, v, 64, debug=True)
    st = check_prefill(gc, k, v, 64, w, y)
    say("stats", st)


def test_prefill_deterministic_and_debug_free_path_identical():
    say("determinism")
    k, v = outlier_kv(5, 2, 200, 4)
    a = GpuCache(2, 4, 256)
    b = GpuCache(2, 4, 256)
    gpu_prefill(a, k, v, 200, debug=False)
    gpu_prefill(b, k, v, 200, debug=True)
    ma = a.host_cache()
    mb = b.host_cache()
    m = ma.defined_mask()
    assert np.array_equal(ma.buf[m], mb.buf[m])
    gpu_prefill(a, k, v, 200)
    assert np.array_equal(a.host_cache().buf[m], ma.buf[m])


def test_saturation_and_scale_flags():
    say("flags")
    k, v = outlier_kv(6, 1, 64, 1)
    k[0, 3, 0, 5] = 0x4781   # 65792, beyond 2^16
    v[0, 40, 0, 7] = 0xC781  # -65792
    gc = GpuCache(1, 1, 64)
    gpu_prefill(gc, k, v, 64, debug=True)
    assert K.kvarn_cache_flags(gc.buf) & K.KVARN_FLAG_SATURATED
    check_prefill(gc, k, v, 64)
    z = np.zeros((1, 32, 1, 128), dtype=np.uint16)
    # 1e-6 everywhere gives r < 2^-14: clamped
    z[0, :, 0, :] = synth.f32_to_bf16_bits(np.full((32, 128), 1e-6, dtype=np.float32))
    gc2 = GpuCache(1, 1, 32)
    gpu_prefill(gc2, z, z, 32)
    assert K.kvarn_cache_flags(gc2.buf) & K.KVARN_FLAG_SCALE_CLAMPED
    check_prefill(gc2, z, z, 32)


# ----------------------------------------------------------------------------- append
@pytest.mark.parametrize("G,n_it,T", [(32, 3, 70), (64, 2, 140)])
def test_append_equals_prefill(G, n_it, T):
    say("append==prefill", G, n_it, T)
    B, H = 2, 3
    k, v = outlier_kv(7, B, T, H)
    cap = ((T + G - 1) // G + 1) * G
    a = GpuCache(B, H, cap, G, n_it)
    gpu_prefill(a, k, v, T)
    b = GpuCache(B, H, cap, G, n_it)
    gpu_prefill(b, k, v, 0)
    kd = from_u16(k)
    vd = from_u16(v)
    for t in range(T):
        K.kvarn_append_decode(b.g, b.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
    ha, hb = a.host_cache(), b.host_cache()
    m = ha.defined_mask()
    assert np.array_equal(m, hb.defined_mask())
    assert np.array_equal(ha.buf[m], hb.buf[m])
    check_prefill(b, k, v, T)


def test_append_capacity_flag():
    say("capacity")
    k, v = outlier_kv(8, 1, 33, 1)
    gc = GpuCache(1, 1, 32)
    gpu_prefill(gc, k, v, 32)
    kd, vd = from_u16(k), from_u16(v)
    K.kvarn_append_decode(gc.g, gc.buf, kd[:, 32].contiguous(), vd[:, 32].contiguous())
    torch.cuda.synchronize()
    assert K.kvarn_cache_flags(gc.buf) & K.KVARN_FLAG_CAPACITY
    assert np.all(gc.host_cache().lens == 32)


def test_checkpoint_restore_mid_decode():
    say("checkpoint")
    B, H, T0, steps = 2, 2, 50, 30
    k, v = outlier_kv(9, B, T0 + steps, H)
    kd, vd = from_u16(k), from_u16(v)
    a = GpuCache(B, H, 128)
    gpu_prefill(a, k, v, T0)
    for t in range(T0, T0 + 10):
        K.kvarn_append_decode(a.g, a.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
    snap = a.buf.clone()
    b = GpuCache(B, H, 128)
    b.buf.copy_(snap)
    for gc in (a, b):
        for t in range(T0 + 10, T0 + steps):
            K.kvarn_append_decode(gc.g, gc.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a.buf, b.buf)


# ----------------------------------------------------------------------------- dequantize
@pytest.mark.parametrize("G,n_it,T,maxT", [(32, 3, 250, 256), (64, 2, 150, 200), (32, 3, 20, 40)])
def test_dequantize_parity(G, n_it, T, maxT):
    say("dequantize", G, n_it, T, maxT)
    B, H = 2, 2
    k, v = outlier_kv(10, B, T, H)
    gc = GpuCache(B, H, 256, G, n_it)
    gpu_prefill(gc, k, v, T)
    hc = gc.host_cache()
    kr, vr = R.dequantize(hc, maxT)
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
                # fp32 bound: 3 roundings to form W_hat plus a 7-stage butterfly sum,
                # gamma_7 * sqrt(D) ~ 4.7e-6 of the row RMS, plus the final scalings
                assert np.all(np.abs(g - ref) <= 1e-5 * np.maximum(rms, 1e-30) + 1e-30)
            else:
                # one bf16 rounding of a value that already carries the fp32 error above
                assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) * 1.01 + 1e-5 * rms + 1e-30)
            assert np.all(g[:, T:] == 0)


def test_dequantize_roundtrip_quality_guard():
    say("roundtrip quality")
    k, v = outlier_kv(0, 1, 256, 1)
    errs = {}
    for n_it in (0, 3):
        gc = GpuCache(1, 1, 256, 32, n_it)
        gpu_prefill(gc, k, v, 256)
        ko = torch.empty(1, 256, 1, 128, device="cuda")
        vo = torch.empty(1, 256, 1, 128, device="cuda")
        K.kvarn_dequantize(gc.g, gc.buf, ko, vo, 256, K.KVARN_OUT_F32)
        torch.cuda.synchronize()
        e = []
        for bits, o in ((k, ko), (v, vo)):
            x = R.canonicalize(bits[0, :, 0])[0]
            e.append(R.relative_token_error(x, o[0, :, 0].cpu().numpy()).mean())
        errs[n_it] = float(np.mean(e))
    say("errors", errs)
    assert errs[3] < 0.2 and errs[3] < 0.1 * errs[0]


# ----------------------------------------------------------------------------- attention
def run_attn(gc, q_bits, Hq, scale=0.0, flags=0):
    q = from_u16(q_bits)
    ws, n = K.alloc_workspace(gc.g, Hq)
    out = torch.full((gc.og.batch, Hq, 128), float("nan"), device="cuda")
    K.kvarn_attn_decode(gc.g, gc.buf, q, Hq, scale, flags, ws, n, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,Hq,H", [(256, 4, 1), (250, 8, 2), (1, 1, 1), (20, 4, 2), (1000, 4, 2), (33, 2, 2),
                                    (300, 16, 2), (100, 6, 2), (300, 24, 2), (70, 32, 1)])
def test_attention_parity(T, Hq, H):
    say("attn", T, Hq, H)
    B = 2
    k, v = outlier_kv(11, B, T, H)
    gc = GpuCache(B, H, 1024 + 32)
    gpu_prefill(gc, k, v, T)
    q = synth.q_host(12, B, Hq)
    out = run_attn(gc, q, Hq)
    worst = check_attention(out, gc.host_cache(), q, Hq)
    say("worst rel", worst)


def test_attention_prerotated_scale_zero_query_and_empty():
    say("attn flags")
    B, H, Hq, T = 1, 2, 8, 300
    k, v = outlier_kv(13, B, T, H)
    gc = GpuCache(B, H, 512)
    gpu_prefill(gc, k, v, T)
    hc = gc.host_cache()
    q = synth.q_host(14, B, Hq)
    check_attention(run_attn(gc, q, Hq, flags=K.KVARN_Q_PREROTATED), hc, q, Hq, flags=R.Q_PREROTATED)
    check_attention(run_attn(gc, q, Hq, scale=0.3), hc, q, Hq, scale=0.3)
    zq = np.zeros_like(q)
    check_attention(run_attn(gc, zq, Hq), hc, zq, Hq)
    empty = GpuCache(B, H, 512)
    gpu_prefill(empty, k, v, 0)
    assert np.all(run_attn(empty, q, Hq) == 0)


@pytest.mark.parametrize("G,n_it", [(32, 3), (64, 2)])
def test_attention_after_appends_many_splits(G, n_it):
    say("attn after appends", G)
    B, H, Hq, T0, steps = 2, 2, 4, 2000, 45
    k, v = outlier_kv(15, B, T0 + steps, H)
    gc = GpuCache(B, H, 4096, G, n_it)
    gpu_prefill(gc, k, v, T0)
    kd, vd = from_u16(k), from_u16(v)
    q = synth.q_host(16, B, Hq)
    for t in range(T0, T0 + steps):
        K.kvarn_append_decode(gc.g, gc.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
    check_attention(run_attn(gc, q, Hq), gc.host_cache(), q, Hq)


@pytest.mark.parametrize("G,T,min_spans", [(32, 9000, 33), (64, 9000, 17)])
def test_attention_more_spans_than_merge_groups(G, T, min_spans):
    """One sequence, one KV head: the split gives each span few tiles, so a row has more
    span partials than the merge has lane groups (16) and some groups fold two or three."""
    say("attn many spans", G, T)
    B, H, Hq = 1, 1, 2
    k, v = outlier_kv(17, B, T, H)
    cap = (T // G + 2) * G
    gc = GpuCache(B, H, cap, G, 3 if G == 32 else 2)
    gpu_prefill(gc, k, v, T)
    ws_bytes = K.kvarn_attn_workspace_bytes(gc.g, Hq)
    nspan = (ws_bytes - 4 * B * H) // (B * Hq * (4 + 128) * 4)
    nsp = min(nspan, T // G)  # spans holding the stored full tiles
    assert nsp >= min_spans, (nspan, nsp)
    q = synth.q_host(18, B, Hq)
    check_attention(run_attn(gc, q, Hq), gc.host_cache(), q, Hq)


# ----------------------------------------------------------------------------- full-size spot checks
def test_full_size_llama_layer_prefill_sampled():
    """Llama-3.1-8B-shaped layer (8 KV heads, 32768 tokens, G=32, 3 iterations) through the
    per-layer call, as the benchmark's per-layer line launches it; 64 sampled tiles through
    the full chain."""
    say("full-size prefill layer")
    torch.manual_seed(0)
    kd, vd = synth.kv_device(synth.sub_seed(2, 0, 0), 1, 32768, 8)
    gc = GpuCache(1, 8, 32768)
    K.kvarn_quantize_prefill(gc.g, gc.buf, kd, vd, 32768)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    picks = sorted({(0, int(rng.integers(8)), int(rng.integers(1024))) for _ in range(64)} | {(0, 7, 1023), (0, 0, 0)})
    # host copies of just the sampled rows
    k = np.zeros((1, 32768, 8, 128), dtype=np.uint16)
    v = np.zeros_like(k)
    for _, h, t in picks:
        k[0, t * 32:(t + 1) * 32, h] = to_u16(kd[0, t * 32:(t + 1) * 32, h])
        v[0, t * 32:(t + 1) * 32, h] = to_u16(vd[0, t * 32:(t + 1) * 32, h])
    st = check_prefill(gc, k, v, 32768, tiles=picks)
    say("stats", st)


def test_full_size_llama_32_layer_prefill_sampled():
    """The benchmark's headline launch: the 32 Llama-3.1-8B-shaped layers (8 KV heads, 32768
    tokens each, G=32, 3 iterations, the benchmark's inputs and sign vector) quantized by one
    kvarn_quantize_prefill_layers call. Sampled tiles of the first, a middle and the last
    layer (their corner tiles included) go through the full chain against the oracle, and
    the last layer's cache equals, byte for byte, a per-layer call on the same input."""
    say("full-size 32-layer prefill launch")
    layers, T, H = 32, 32768, 8
    ks, vs = [], []
    for l in range(layers):
        k, v = synth.kv_device(synth.sub_seed(2, l, 0), 1, T, H)
        ks.append(k)
        vs.append(v)
    caches = [GpuCache(1, H, T) for _ in range(layers)]
    K.kvarn_quantize_prefill_layers(caches[0].g, [c.buf for c in caches], ks, vs, T)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for l in (0, 13, layers - 1):
        picks = sorted({(0, int(rng.integers(H)), int(rng.integers(T // 32))) for _ in range(16)}
                       | {(0, 0, 0), (0, H - 1, T // 32 - 1)})
        k = np.zeros((1, T, H, 128), dtype=np.uint16)
        v = np.zeros_like(k)
        for _, h, t in picks:
            k[0, t * 32:(t + 1) * 32, h] = to_u16(ks[l][0, t * 32:(t + 1) * 32, h])
            v[0, t * 32:(t + 1) * 32, h] = to_u16(vs[l][0, t * 32:(t + 1) * 32, h])
        st = check_prefill(caches[l], k, v, T, tiles=picks)
        say("layer", l, "stats", st)
    one = GpuCache(1, H, T)
    K.kvarn_quantize_prefill(one.g, one.buf, ks[-1], vs[-1], T)
    torch.cuda.synchronize()
    ha, hb = caches[-1].host_cache(), one.host_cache()
    m = ha.defined_mask()
    assert np.array_equal(ha.buf[m], hb.buf[m])
    assert K.kvarn_cache_flags(caches[-1].buf) == K.kvarn_cache_flags(one.buf)


def test_full_size_phi4_decode_sampled():
    """Phi-4-14B-shaped decode layer: 32 sequences x 10 KV heads x 16384 prior tokens,
    40 query heads, then appends across a group boundary; attention checked on
    sampled (batch, kv head) pairs against the oracle on the GPU-written bytes."""
    say("full-size decode layer")
    B, H, Hq, T0, cap = 32, 10, 40, 16384, 17408
    kd, vd = synth.kv_device(synth.sub_seed(4, 0, 0), B, T0, H)
    gc = GpuCache(B, H, cap)
    K.kvarn_quantize_prefill(gc.g, gc.buf, kd, vd, T0)
    del kd, vd
    kn, vn = synth.kv_device(synth.sub_seed(4, 0, 1), B, 40, H)
    for t in range(40):
        K.kvarn_append_decode(gc.g, gc.buf, kn[:, t].contiguous(), vn[:, t].contiguous())
    q = synth.q_host(17, B, Hq)
    out = run_attn(gc, q, Hq)
    hc = gc.host_cache()
    assert np.all(hc.lens == T0 + 40)
    pairs = [(0, 0), (5, 3), (31, 9), (17, 6)]
    ref = R.attn_decode(hc, q, Hq, pairs=pairs)
    grp = Hq // H
    for b, h in pairs:
        for g in range(h * grp, (h + 1) * grp):
            m = np.abs(ref[b, g]).max()
            assert np.abs(out[b, g] - ref[b, g]).max() <= 2e-3 * m, (b, g)
    assert np.all(np.isfinite(out))


def test_full_size_qwen3_prefill_dequant_sampled():
    """Qwen3-4B-shaped layer: 8 sequences x 8 KV heads x 16384 tokens, 2% of tokens with norm
    x50, G=64, 2 VarN iterations. Sampled tiles go through the full parity chain, and the bf16
    dequantization of the whole layer is compared on those tiles with the oracle's
    dequantization of the same bytes."""
    say("full-size qwen3 prefill + dequantize")
    B, H, T, G = 8, 8, 16384, 64
    kd, vd = synth.kv_device(synth.sub_seed(3, 0, 0), B, T, H, law="spike", p=0.02, factor=50.0)
    gc = GpuCache(B, H, T, G, 2)
    K.kvarn_quantize_prefill(gc.g, gc.buf, kd, vd, T)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    picks = sorted({(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(T // G))) for _ in range(40)}
                   | {(0, 0, 0), (B - 1, H - 1, T // G - 1)})
    k = np.zeros((B, T, H, 128), dtype=np.uint16)
    v = np.zeros_like(k)
    for b, h, t in picks:
        k[b, t * G:(t + 1) * G, h] = to_u16(kd[b, t * G:(t + 1) * G, h])
        v[b, t * G:(t + 1) * G, h] = to_u16(vd[b, t * G:(t + 1) * G, h])
    say("stats", check_prefill(gc, k, v, T, tiles=picks))
    del kd, vd
    ko = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    K.kvarn_dequantize(gc.g, gc.buf, ko, vo, T, K.KVARN_OUT_BF16)
    hc = gc.host_cache()
    for b, h, t in picks:
        for s, out in ((0, ko), (1, vo)):
            u = R.unpack_record(hc.record(b, h, t, s), G, 128, s)
            ref = R.unrotate(R.dequantize_tile(u["q"], u["r16"], u["c16"], u["s16"], u["z16"]), hc.sigma)
            got = out[b, t * G:(t + 1) * G, h].float().cpu().numpy().astype(np.float64)
            rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) * 1.01 + 1e-5 * rms + 1e-30), (b, h, t, s)


def test_full_size_long_reasoning_quantize_and_decode():
    """Long-reasoning stress shape: 64 sequences x 8 KV heads x 32768 prior tokens, Student-t
    (nu = 3) token norms, 8 outlier channels x30, G=32, 3 iterations, 32 query heads, in the
    benchmark's launch configuration. Prefill, then appends that complete one more group per
    sequence. Every tile whose stored scales hit the fp16 clamp (r or c at 2^-14 or 65504, or
    s / z saturated; found from the GPU bytes) goes through the full parity chain, with 64
    random tiles and tiles completed by the appends. Attention on sampled (batch, kv head)
    pairs against the oracle on the GPU-written bytes."""
    say("full-size long-reasoning quantize + decode")
    B, H, Hq, T0, steps, G = 64, 8, 32, 32768, 40, 32
    cap = T0 + 64
    law = dict(n_outlier_ch=8, ch_mult=30.0, law="student_t", nu=3.0)
    kd, vd = synth.kv_device(synth.sub_seed(5, 0, 0), B, T0, H, **law)
    gc = GpuCache(B, H, cap)
    K.kvarn_quantize_prefill(gc.g, gc.buf, kd, vd, T0)
    kn, vn = synth.kv_device(synth.sub_seed(5, 0, 1), B, steps, H, **law)
    for t in range(steps):
        K.kvarn_append_decode(gc.g, gc.buf, kn[:, t].contiguous(), vn[:, t].contiguous())
    torch.cuda.synchronize()
    T = T0 + steps
    nfull = T // G
    og = gc.og
    # the clamped tiles, from the stored scales of every full tile (scanned on the device)
    tiles = cap // G
    rec = gc.buf[og.header:og.header + B * H * tiles * 2 * og.tr].view(B, H, tiles, 2, og.tr)[:, :, :nfull]
    f16 = lambda lo, n: rec[..., lo:lo + 2 * n].contiguous().view(torch.int16)  # noqa: E731
    r16, c16 = f16(1024, G), f16(1024 + 2 * G, 128)
    s16, z16 = f16(1024 + 2 * G + 256, 128), f16(1024 + 2 * G + 512, 128)
    lo, hi = 0x0400, 0x7BFF  # fp16 bits of 2^-14 and 65504
    kinds = {"r_low": (r16 == lo).any(-1), "r_high": (r16 == hi).any(-1), "c_low": (c16 == lo).any(-1),
             "c_high": (c16 == hi).any(-1), "s_sat": (s16 == hi).any(-1),
             "z_sat": ((z16 & 0x7FFF) == hi).any(-1)}
    counts = {k: int(v.sum()) for k, v in kinds.items()}
    clamped = torch.stack(list(kinds.values())).any(0).any(-1)            # [B][H][nfull], either stream
    idx = torch.nonzero(clamped).cpu().numpy()
    del rec, r16, c16, s16, z16, kinds, clamped
    say("clamped records", counts, "tiles", len(idx), "of", B * H * nfull)
    assert K.kvarn_cache_flags(gc.buf) & K.KVARN_FLAG_SCALE_CLAMPED or len(idx) == 0
    rng = np.random.default_rng(5)
    picks = {(int(b), int(h), int(t)) for b, h, t in idx}
    picks |= {(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(nfull))) for _ in range(64)}
    picks |= {(int(rng.integers(B)), int(rng.integers(H)), nfull - 1) for _ in range(8)}  # completed by appends
    picks = sorted(picks)
    k = np.zeros((B, T, H, 128), dtype=np.uint16)
    v = np.zeros_like(k)
    for b, h, t in picks:
        for arr, dev, newd in ((k, kd, kn), (v, vd, vn)):
            lo_t, hi_t = t * G, (t + 1) * G
            if hi_t <= T0:
                arr[b, lo_t:hi_t, h] = to_u16(dev[b, lo_t:hi_t, h])
            else:
                arr[b, lo_t:hi_t, h] = to_u16(newd[b, lo_t - T0:hi_t - T0, h])
    k[:, nfull * G:T] = to_u16(kn[:, nfull * G - T0:])  # the tail rows
    v[:, nfull * G:T] = to_u16(vn[:, nfull * G - T0:])
    del kd, vd
    st = check_prefill(gc, k, v, T, tiles=picks)
    say("stats", st, "tiles checked", len(picks))
    q = synth.q_host(19, B, Hq)
    out = run_attn(gc, q, Hq)
    assert np.all(np.isfinite(out))
    hc = gc.host_cache()
    pairs = [(0, 0), (63, 7), (29, 4)]
    ref = R.attn_decode(hc, q, Hq, pairs=pairs)
    grp = Hq // H
    for b, h in pairs:
        for g in range(h * grp, (h + 1) * grp):
            m = np.abs(ref[b, g]).max()
            assert np.abs(out[b, g] - ref[b, g]).max() <= 2e-3 * m, (b, g)


@pytest.mark.parametrize("B,H,T,G,n_it,law", [(1, 1, 256, 32, 3, "lognormal"), (2, 3, 1000, 32, 3, "lognormal"),
                                              (3, 8, 4133, 32, 3, "student_t"), (2, 2, 532, 64, 2, "spike"),
                                              (1, 8, 9000, 64, 2, "lognormal"), (1, 1, 31, 32, 3, "lognormal")])
def test_prefill_entry_points_agree(B, H, T, G, n_it, law):
    """kvarn_quantize_prefill and the test hook kvarn_debug_prefill (the same kernel built with
    the debug outputs that the parity chain above reads) write bit-identical caches, flags
    included, across group sizes, data laws and ragged tails."""
    say("prefill entry points", B, H, T, G, law)
    kw = dict(nu=3.0) if law == "student_t" else {}
    k, v = outlier_kv(23, B, T, H, law=law, **kw)
    cap = (T // G + 1) * G
    a, b = GpuCache(B, H, cap, G, n_it), GpuCache(B, H, cap, G, n_it)
    gpu_prefill(a, k, v, T)
    gpu_prefill(b, k, v, T, debug=True)
    ha, hb = a.host_cache(), b.host_cache()
    m = ha.defined_mask()
    assert np.array_equal(ha.buf[m], hb.buf[m])
    assert K.kvarn_cache_flags(a.buf) == K.kvarn_cache_flags(b.buf)


@pytest.mark.parametrize("n,B,H,T,G,n_it,variant,law", [
    (3, 1, 2, 250, 32, 3, 0, "lognormal"),
    (2, 2, 3, 532, 64, 2, 0, "spike"),
    (70, 1, 1, 100, 32, 3, 0, "lognormal"),      # two launches (at most 64 layers each)
    (2, 1, 2, 96, 32, 2, K.KVARN_VARIANT_NO_TOKEN_PASS, "lognormal"),  # the extended build
    (3, 2, 2, 150, 32, 3, 0, "student_t"),        # paged caches, each with its own page map
])
def test_prefill_layers_equals_per_layer_calls(n, B, H, T, G, n_it, variant, law):
    """kvarn_quantize_prefill_layers over n caches of one geometry (each with its own sigma and
    inputs) writes the same bytes and flags as n calls of kvarn_quantize_prefill; the first
    layer also goes through the parity chain against the oracle."""
    say("prefill layers", n, B, H, T, G, variant, law)
    cap = (T // G + 1) * G
    paged = law == "student_t"
    kw = dict(nu=3.0) if law == "student_t" else {}
    ins = [outlier_kv(40 + i, B, T, H, law=law, **kw) for i in range(n)]
    if paged:
        tiles = cap // G
        geo = K.geom(B, H, cap, G, n_it, num_pages=B * tiles + 3)
        rng = np.random.default_rng(7)

        def make(i):
            c = GpuCache(B, H, cap, G, n_it, seed_sigma=i)
            c.g = geo
            c.og = R.Geom(B, H, 128, cap, G, n_it, 2, 0, B * tiles + 3)
            c.buf = K.alloc_cache(geo, c.sigma)
            pages = rng.permutation(B * tiles + 3)[:B * tiles].reshape(B, tiles).astype(np.int32)
            p = torch.from_numpy(pages).cuda()
            K.kvarn_cache_set_pages(geo, c.buf, p, 0, tiles)
            return c, pages
        pairs = [make(i) for i in range(n)]
        a = [p[0] for p in pairs]
        bl = []
        for i in range(n):  # the same page maps in the second set
            c = GpuCache(B, H, cap, G, n_it, seed_sigma=i)
            c.g, c.og = geo, a[i].og
            c.buf = K.alloc_cache(geo, c.sigma)
            K.kvarn_cache_set_pages(geo, c.buf, torch.from_numpy(pairs[i][1]).cuda(), 0, tiles)
            bl.append(c)
        b = bl
    else:
        a = [GpuCache(B, H, cap, G, n_it, seed_sigma=i, variant=variant) for i in range(n)]
        b = [GpuCache(B, H, cap, G, n_it, seed_sigma=i, variant=variant) for i in range(n)]
    for i in range(n):
        gpu_prefill(a[i], ins[i][0], ins[i][1], T)
    kd = [from_u16(k[:, :T]) for k, _ in ins]
    vd = [from_u16(v[:, :T]) for _, v in ins]
    K.kvarn_quantize_prefill_layers(b[0].g, [c.buf for c in b], kd, vd, T)
    torch.cuda.synchronize()
    for i in range(n):
        ha, hb = a[i].host_cache(), b[i].host_cache()
        m = ha.defined_mask()
        assert np.array_equal(ha.buf[m], hb.buf[m]), i
        assert K.kvarn_cache_flags(a[i].buf) == K.kvarn_cache_flags(b[i].buf), i
    if variant == 0:
        check_prefill(b[0], ins[0][0], ins[0][1], T)
