"""A decode step (append + attention over every layer cache) captured in a HIP graph and
replayed gives the same cache bytes (those the format defines) and attention outputs as the same calls issued
eagerly. The entry points only enqueue kernels on the given stream (no allocation, no
memset, no host synchronization), so the step can be captured. Every replay is checked
against the eager run, with eager work between the replays.
"""
import numpy as np
import pytest
import torch

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth

from parity import GpuCache, from_u16

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("G,n_it", [(32, 3), (64, 2)])
def test_decode_step_graph_replay_matches_eager(G, n_it):
    say("graph replay", G)
    B, H, Hq, layers, T0, steps = 2, 2, 8, 3, 2 * G - 6, 12  # the replays cross a group boundary
    k, v = synth.kv_host(21, B, T0 + steps, H)
    kd, vd = from_u16(k), from_u16(v)
    q = from_u16(synth.q_host(22, B, Hq))
    graph_caches = [GpuCache(B, H, 4 * G, G, n_it) for _ in range(layers)]
    eager_caches = [GpuCache(B, H, 4 * G, G, n_it) for _ in range(layers)]
    for c in graph_caches + eager_caches:
        K.kvarn_quantize_prefill(c.g, c.buf, kd[:, :T0].contiguous(), vd[:, :T0].contiguous(), T0)
    g = graph_caches[0].g
    ws_g, n = K.alloc_workspace(g, Hq)
    ws_e, _ = K.alloc_workspace(g, Hq)
    k_in = torch.empty(B, H, 128, dtype=torch.bfloat16, device="cuda")
    v_in = torch.empty_like(k_in)
    out_g = torch.full((layers, B, Hq, 128), float("nan"), device="cuda")
    out_e = torch.full_like(out_g, float("nan"))
    torch.cuda.synchronize()

    def step(caches, ws, out, kk, vv):
        for l, c in enumerate(caches):
            K.kvarn_append_decode(c.g, c.buf, kk, vv)
            K.kvarn_attn_decode(c.g, c.buf, q, Hq, 0.0, 0, ws, n, out[l])

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):  # recorded, not run
        step(graph_caches, ws_g, out_g, k_in, v_in)
    torch.cuda.synchronize()
    for t in range(T0, T0 + steps):
        k_in.copy_(kd[:, t])
        v_in.copy_(vd[:, t])
        graph.replay()
        step(eager_caches, ws_e, out_e, kd[:, t].contiguous(), vd[:, t].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), ("attention output", t)
        for a, b in zip(graph_caches, eager_caches):  # bytes the format defines at this length
            ha, hb = a.host_cache(), b.host_cache()
            m = ha.defined_mask()
            assert np.array_equal(ha.buf[m], hb.buf[m]) and np.array_equal(m, hb.defined_mask()), ("cache", t)
        assert not torch.isnan(out_g).any()
    lens = graph_caches[0].host_cache().lens
    assert np.all(lens == T0 + steps), lens


def test_prefill_graph_replay_matches_eager():
    """Prefill launches of several layers captured once and replayed (with eager work between
    the replays) write the same cache bytes as eager calls."""
    say("prefill graph")
    B, H, T, G, layers = 2, 2, 100, 32, 3
    k, v = synth.kv_host(23, B, T, H)
    kd, vd = from_u16(k), from_u16(v)
    gcs = [GpuCache(B, H, 128, G, 3) for _ in range(layers)]
    ecs = [GpuCache(B, H, 128, G, 3) for _ in range(layers)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in gcs:
            K.kvarn_quantize_prefill(c.g, c.buf, kd, vd, T)
    torch.cuda.synchronize()
    for rep in range(3):
        for c in gcs:  # disturb the lengths between replays: the replay must reset them
            K.kvarn_append_decode(c.g, c.buf, kd[:, 0].contiguous(), vd[:, 0].contiguous())
        graph.replay()
        for c in ecs:
            K.kvarn_quantize_prefill(c.g, c.buf, kd, vd, T)
        torch.cuda.synchronize()
        for a, b in zip(gcs, ecs):
            ha, hb = a.host_cache(), b.host_cache()
            m = hb.defined_mask()
            assert np.array_equal(ha.buf[m], hb.buf[m]) and np.all(ha.lens == T), rep
