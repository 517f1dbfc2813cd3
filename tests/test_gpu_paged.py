"""Paged layout, multi-token appends and per-sequence counts on the GPU, through the C ABI.

* kvarn_append_tokens: a chunk appended to a prefilled cache, and a fresh append of a
  whole sequence, give the bytes of one prefill (the same tile code runs, so bit-equal),
  and pass the oracle parity chain; ragged counts give, per sequence, the bytes of a
  prefill of that sequence's tokens; counts of 0/1 (a mask) touch only the selected
  sequences.
* Paged caches: under a shuffled page map every call (prefill, appends, fused step,
  dequantize, attention) gives bit-equal results to the per-sequence layout; a tile
  without a page is dropped with KVARN_FLAG_UNMAPPED and skipped by the readers, as the
  oracle defines.
"""
import numpy as np
import pytest
import torch

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth
from oracle import kvarn_ref as R

from parity import GpuCache, PagedCache, check_prefill, from_u16, gpu_prefill, same_stored

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("G,n_it,T1,T2", [(32, 3, 45, 50), (64, 2, 64, 130), (32, 3, 0, 77)])
def test_append_tokens_equals_prefill(G, n_it, T1, T2):
    say("append_tokens", G, n_it, T1, T2)
    B, H, T = 2, 3, T1 + T2
    k, v = synth.kv_host(80, B, T, H)
    kd, vd = from_u16(k), from_u16(v)
    whole = GpuCache(B, H, 4 * G, G, n_it)
    gpu_prefill(whole, k, v, T)
    chunked = GpuCache(B, H, 4 * G, G, n_it)
    gpu_prefill(chunked, k, v, T1)
    K.kvarn_append_tokens(chunked.g, chunked.buf, kd[:, T1:].contiguous(), vd[:, T1:].contiguous(), T2)
    torch.cuda.synchronize()
    same_stored(whole.host_cache(), chunked.host_cache())
    check_prefill(chunked, k, v, T)
    assert K.kvarn_cache_flags(chunked.buf) == 0


def test_ragged_counts_and_mask():
    say("ragged")
    B, H, G, T = 3, 2, 32, 70
    k, v = synth.kv_host(81, B, T, H)
    kd, vd = from_u16(k), from_u16(v)
    counts = np.array([70, 0, 33], dtype=np.int32)
    gc = GpuCache(B, H, 128, G, 3)
    K.kvarn_append_tokens(gc.g, gc.buf, kd, vd, T, torch.from_numpy(counts).cuda())
    torch.cuda.synchronize()
    hc = gc.host_cache()
    assert np.array_equal(hc.lens[:, 0, 0], counts)
    for bb in range(B):
        one = GpuCache(B, H, 128, G, 3)
        gpu_prefill(one, k, v, int(counts[bb]))
        same_stored(one.host_cache(), hc, seqs=[bb])
    # a mask: counts 0/1 touch only the selected sequences
    before = hc.buf.copy()
    mask = np.array([0, 1, 0], dtype=np.int32)
    K.kvarn_append_tokens(gc.g, gc.buf, kd[:, :1].contiguous(), vd[:, :1].contiguous(), 1,
                          torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    after = gc.host_cache()
    assert np.array_equal(after.lens[:, 0, 0], counts + mask)
    changed = np.nonzero(before != after.buf)[0]
    rows = [after.g.tail_slot_offset(1, h, s, 0) for h in range(H) for s in range(2)]
    for o in changed:
        assert any(r <= o < r + 256 for r in rows) or 512 + 8 * H <= o < 512 + 16 * H, o  # tail rows, len
    # capacity: the tokens past 128 are dropped and flagged
    k2, v2 = synth.kv_host(82, B, 128, H)
    K.kvarn_append_tokens(gc.g, gc.buf, from_u16(k2), from_u16(v2), 128)
    torch.cuda.synchronize()
    assert np.all(gc.host_cache().lens == 128)
    assert K.kvarn_cache_flags(gc.buf) & K.KVARN_FLAG_CAPACITY


@pytest.mark.parametrize("G,bits", [(32, 2), (64, 2), (32, 3), (64, 4)])
def test_paged_equals_per_sequence_layout(G, bits):
    say("paged == per-sequence", G, bits)
    B, H, Hq, n_it = 3, 2, 8, 2
    cap = 4 * G
    tiles = cap // G
    rng = np.random.default_rng(G)
    npages = B * tiles + 3
    pages = rng.permutation(npages)[:B * tiles].reshape(B, tiles).astype(np.int32)
    T0, T1 = 2 * G - 3, 5
    k, v = synth.kv_host(83, B, T0 + T1 + 8, H)
    kd, vd = from_u16(k), from_u16(v)
    flat = GpuCache(B, H, cap, G, n_it, bits=bits)
    paged = PagedCache(B, H, cap, G, n_it, npages, bits=bits)
    paged.set_pages(pages[:, :2])
    paged.set_pages(pages[:, 2:], tile_first=2)
    ws, n = K.alloc_workspace(flat.g, Hq)
    outs = []
    for c in (flat, paged):
        gpu_prefill(c, k, v, T0)
        K.kvarn_append_tokens(c.g, c.buf, kd[:, T0:T0 + T1].contiguous(), vd[:, T0:T0 + T1].contiguous(), T1)
        o = []
        for t in range(T0 + T1, T0 + T1 + 8):
            q = from_u16(synth.q_host(90 + t, B, Hq))
            out = torch.empty(B, Hq, 128, device="cuda")
            if t % 2:
                K.kvarn_append_attn_decode(c.g, c.buf, kd[:, t].contiguous(), vd[:, t].contiguous(), q, Hq, 0.0, 0,
                                           ws, n, out)
            else:
                K.kvarn_append_decode(c.g, c.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
                K.kvarn_attn_decode(c.g, c.buf, q, Hq, 0.0, 0, ws, n, out)
            o.append(out.clone())
        kq = torch.empty(B, cap, H, 128, device="cuda")
        vq = torch.empty(B, cap, H, 128, device="cuda")
        K.kvarn_dequantize(c.g, c.buf, kq, vq, cap, K.KVARN_OUT_F32)
        torch.cuda.synchronize()
        outs.append((torch.stack(o), kq, vq))
    for x, y in zip(outs[0], outs[1]):
        assert torch.equal(x, y)
    hf, hp = flat.host_cache(), paged.host_cache()
    same_stored(hf, hp)
    assert np.array_equal(hp.page_map, pages)
    assert K.kvarn_cache_flags(paged.buf) & K.KVARN_FLAG_UNMAPPED == 0


def test_unmapped_tiles_dropped_and_skipped():
    say("unmapped")
    B, H, Hq, G = 2, 2, 4, 32
    T = 2 * G + 5
    k, v = synth.kv_host(84, B, T, H)
    pc = PagedCache(B, H, 4 * G, G, 3, 6)
    pc.set_pages(np.array([[0, -1, 2, 3], [4, 99, -7, 5]], dtype=np.int32))  # tile 1 has no page
    gpu_prefill(pc, k, v, T)
    assert K.kvarn_cache_flags(pc.buf) & K.KVARN_FLAG_UNMAPPED
    hc = pc.host_cache()
    kq = torch.full((B, T, H, 128), 7.0, device="cuda")
    vq = torch.full((B, T, H, 128), 7.0, device="cuda")
    K.kvarn_dequantize(pc.g, pc.buf, kq, vq, T, K.KVARN_OUT_F32)
    qb = synth.q_host(85, B, Hq)
    ws, n = K.alloc_workspace(pc.g, Hq)
    out = torch.empty(B, Hq, 128, device="cuda")
    K.kvarn_attn_decode(pc.g, pc.buf, from_u16(qb), Hq, 0.0, 0, ws, n, out)
    torch.cuda.synchronize()
    kr, _ = R.dequantize(hc, T)
    assert np.all(kq[:, G:2 * G].cpu().numpy() == 0)
    g = kq.cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(kr * kr, axis=-1, keepdims=True))
    assert np.all(np.abs(g - kr) <= 1e-5 * np.maximum(rms, 1e-30) + 1e-30)
    ref = R.attn_decode(hc, qb, Hq)
    got = out.cpu().numpy().astype(np.float64)
    for b in range(B):
        for q in range(Hq):
            m = np.abs(ref[b, q]).max()
            assert np.abs(got[b, q] - ref[b, q]).max() <= 2e-3 * m, (b, q)
