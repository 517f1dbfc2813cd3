"""The fused decode step (kvarn_append_attn_decode: the append runs inside the attention's
merge launch) against the oracle's append_attn_decode, step by step across group
boundaries: the attention output to the attention tolerance, the cache bytes bit-equal to
those of plain appends, the capacity path, and replay as a HIP graph.
"""
import numpy as np
import pytest
import torch

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth
from oracle import kvarn_ref as R

from parity import GpuCache, from_u16, gpu_prefill

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def attn_close(got, ref, tol=2e-3):
    for b in range(ref.shape[0]):
        for g in range(ref.shape[1]):
            m = np.abs(ref[b, g]).max()
            d = np.abs(got[b, g] - ref[b, g]).max()
            assert d <= tol * m or (m == 0 and d == 0), (b, g, d, m)


@pytest.mark.parametrize("G,n_it,H,Hq,variant,flags", [
    (32, 3, 2, 8, 0, 0), (64, 2, 2, 4, 0, 0), (32, 3, 1, 8, 0, K.KVARN_Q_PREROTATED),
    (32, 3, 2, 6, K.KVARN_VARIANT_NO_ROTATION, 0)])
def test_fused_steps_match_oracle(G, n_it, H, Hq, variant, flags):
    say("fused steps", G, n_it, H, Hq, variant, flags)
    B, T0, steps = 2, 2 * G - 5, 12  # step 4 completes a group
    k, v = synth.kv_host(70, B, T0 + steps, H)
    kd, vd = from_u16(k), from_u16(v)
    fused = GpuCache(B, H, 4 * G, G, n_it, variant=variant)
    plain = GpuCache(B, H, 4 * G, G, n_it, variant=variant)
    for c in (fused, plain):
        gpu_prefill(c, k, v, T0)
    ws, n = K.alloc_workspace(fused.g, Hq)
    out = torch.full((B, Hq, 128), float("nan"), device="cuda")
    for t in range(T0, T0 + steps):
        qb = synth.q_host(100 + t, B, Hq)
        q = from_u16(qb)
        oc = fused.host_cache()                       # the oracle starts from the GPU's bytes
        ref = R.append_attn_decode(oc, k[:, t], v[:, t], qb, Hq, 0.0, flags)
        K.kvarn_append_attn_decode(fused.g, fused.buf, kd[:, t].contiguous(), vd[:, t].contiguous(), q, Hq, 0.0,
                                   flags, ws, n, out)
        K.kvarn_append_decode(plain.g, plain.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
        torch.cuda.synchronize()
        attn_close(out.cpu().numpy().astype(np.float64), ref)
        hf, hp = fused.host_cache(), plain.host_cache()
        m = hf.defined_mask()
        assert np.array_equal(m, hp.defined_mask()) and np.array_equal(hf.buf[m], hp.buf[m]), ("cache", t)
        assert np.all(hf.lens == t + 1)


def test_fused_step_on_full_sequence():
    say("fused full")
    B, H, Hq, G = 1, 2, 4, 32
    k, v = synth.kv_host(71, B, 65, H)
    gc = GpuCache(B, H, 64, G, 3)
    gpu_prefill(gc, k, v, 64)
    before = gc.host_cache()
    qb = synth.q_host(72, B, Hq)
    ws, n = K.alloc_workspace(gc.g, Hq)
    out = torch.full((B, Hq, 128), float("nan"), device="cuda")
    K.kvarn_append_attn_decode(gc.g, gc.buf, from_u16(k)[:, 64].contiguous(), from_u16(v)[:, 64].contiguous(),
                               from_u16(qb), Hq, 0.0, 0, ws, n, out)
    torch.cuda.synchronize()
    attn_close(out.cpu().numpy().astype(np.float64), R.attn_decode(before, qb, Hq))
    assert K.kvarn_cache_flags(gc.buf) & K.KVARN_FLAG_CAPACITY
    assert np.all(gc.host_cache().lens == 64)


@pytest.mark.parametrize("G", [32, 64])
def test_fused_step_graph_replay(G):
    say("fused graph", G)
    B, H, Hq, layers, T0, steps = 2, 2, 8, 3, 2 * G - 4, 10
    k, v = synth.kv_host(73, B, T0 + steps, H)
    kd, vd = from_u16(k), from_u16(v)
    q = from_u16(synth.q_host(74, B, Hq))
    gcs = [GpuCache(B, H, 4 * G, G, 2) for _ in range(layers)]
    ecs = [GpuCache(B, H, 4 * G, G, 2) for _ in range(layers)]
    for c in gcs + ecs:
        K.kvarn_quantize_prefill(c.g, c.buf, kd[:, :T0].contiguous(), vd[:, :T0].contiguous(), T0)
    g = gcs[0].g
    ws_g, n = K.alloc_workspace(g, Hq)
    ws_e, _ = K.alloc_workspace(g, Hq)
    k_in = torch.empty(B, H, 128, dtype=torch.bfloat16, device="cuda")
    v_in = torch.empty_like(k_in)
    out_g = torch.full((layers, B, Hq, 128), float("nan"), device="cuda")
    out_e = torch.full_like(out_g, float("nan"))
    torch.cuda.synchronize()

    def step(caches, ws, out, kk, vv):
        for l, c in enumerate(caches):
            K.kvarn_append_attn_decode(c.g, c.buf, kk, vv, q, Hq, 0.0, 0, ws, n, out[l])

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gcs, ws_g, out_g, k_in, v_in)
    torch.cuda.synchronize()
    for t in range(T0, T0 + steps):
        k_in.copy_(kd[:, t])
        v_in.copy_(vd[:, t])
        graph.replay()
        step(ecs, ws_e, out_e, kd[:, t].contiguous(), vd[:, t].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), ("output", t)
        for a, b in zip(gcs, ecs):
            ha, hb = a.host_cache(), b.host_cache()
            m = ha.defined_mask()
            assert np.array_equal(ha.buf[m], hb.buf[m]), ("cache", t)
