"""GPU parity over seeded random geometries (run on an MI355X: pytest -m gpu).

Each case draws batch, KV heads, query heads per KV head, group size, VarN iterations,
code width, token law, prefill length and a number of decode appends from its own seed,
then runs the whole path on the GPU against the oracle:

  prefill(T)                    full parity chain (W/Y chain through the stored fields,
                                codes, record bytes, bf16 tail)
  T + n single-token appends    byte-identical to prefill(T + n) of the same tokens
  decode attention              within 2e-3 of max |ref| (oracle over the same bytes)
  dequantization (f32 out)      within 1e-5 of the row RMS, zeros past each length

The geometries mix ragged tails, empty prefills, appends that complete one or more
groups, GQA ratios 1..8 and every code width, so combinations the fixed-shape tests do
not name are still checked against the oracle.

A second sweep drives kvarn_append_tokens with ragged per-sequence counts over several
calls, into a per-sequence cache and into a paged cache under a shuffled page map:

  each sequence                 records and tail equal to a prefill of that sequence's
                                own token stream, which passes the oracle parity chain
  paged against per-sequence    stored bytes, attention and dequantization bit-equal
  attention, dequantization     against the oracle over the stored bytes

A third sweep runs fused decode steps (kvarn_append_attn_decode) across group
boundaries: every step's output against the oracle's append_attn_decode on the same
bytes, the cache byte-equal to plain appends, and kvarn_attn_decode_noalloc equal to
kvarn_attn_decode on the final cache.
"""
import numpy as np
import pytest
import torch

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth
from oracle import kvarn_ref as R

from parity import GpuCache, PagedCache, check_attention, check_prefill, from_u16, gpu_prefill, same_stored

pytestmark = pytest.mark.gpu

LAWS = ("lognormal", "spike", "student_t", "none")


def draw(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    G = int(rng.choice((32, 64)))
    cfg = dict(
        B=int(rng.integers(1, 4)),
        H=int(rng.integers(1, 5)),
        grp=int(rng.choice((1, 2, 3, 4, 5, 8))),
        G=G,
        n_it=int(rng.integers(0, 5)),
        bits=int(rng.choice((2, 3, 4))),
        law=str(rng.choice(LAWS)),
        T=int(rng.integers(0, 5 * G + 18)),
        n_app=int(rng.integers(1, G + 4)),
    )
    if rng.random() < 0.2:
        cfg["T"] = 0  # an empty prefill, every token appended
    law_kw = {"lognormal": {}, "spike": {"p": 0.05, "factor": 40.0}, "student_t": {"nu": 3.0}, "none": {}}
    cfg["law_kw"] = law_kw[cfg["law"]]
    return cfg


SEEDS = list(range(40))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_geometry_path(seed):
    c = draw(1000 + seed)
    print("[case] random geometry", seed, {k: v for k, v in c.items() if k != "law_kw"}, flush=True)
    B, H, G, T, n_app = c["B"], c["H"], c["G"], c["T"], c["n_app"]
    total = T + n_app
    cap = (total // G + 1) * G
    k, v = synth.kv_host(synth.sub_seed(77, seed), B, total, H, law=c["law"], **c["law_kw"])

    # prefill of the first T tokens
    gc = GpuCache(B, H, cap, G, c["n_it"], seed_sigma=seed, bits=c["bits"])
    gpu_prefill(gc, k, v, T)
    check_prefill(gc, k, v, T)

    # n single-token appends == one prefill of T + n tokens
    kd, vd = from_u16(k), from_u16(v)
    for t in range(T, total):
        K.kvarn_append_decode(gc.g, gc.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
    ref = GpuCache(B, H, cap, G, c["n_it"], seed_sigma=seed, bits=c["bits"])
    gpu_prefill(ref, k, v, total)
    ha, hb = gc.host_cache(), ref.host_cache()
    m = hb.defined_mask()
    assert np.array_equal(ha.defined_mask(), m)
    assert np.array_equal(ha.buf[m], hb.buf[m]), "appends differ from prefill"
    assert np.all(ha.lens == total)

    # decode attention over the appended cache
    Hq = H * c["grp"]
    q = synth.q_host(synth.sub_seed(78, seed), B, Hq)
    ws, n = K.alloc_workspace(gc.g, Hq)
    out = torch.full((B, Hq, 128), float("nan"), device="cuda")
    K.kvarn_attn_decode(gc.g, gc.buf, from_u16(q), Hq, 0.0, 0, ws, n, out)
    torch.cuda.synchronize()
    check_attention(out.cpu().numpy().astype(np.float64), ha, q, Hq)

    # dequantization, f32 out, rows past the length where the capacity leaves room
    maxT = min(total + 5, cap)
    kr, vr = R.dequantize(ha, maxT)
    ko = torch.full((B, maxT, H, 128), 7.0, dtype=torch.float32, device="cuda")
    vo = torch.full((B, maxT, H, 128), 7.0, dtype=torch.float32, device="cuda")
    K.kvarn_dequantize(gc.g, gc.buf, ko, vo, maxT, K.KVARN_OUT_F32)
    torch.cuda.synchronize()
    for got, want in ((ko, kr), (vo, vr)):
        g = got.cpu().numpy().astype(np.float64)
        rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
        assert np.all(np.abs(g - want) <= 1e-5 * np.maximum(rms, 1e-30) + 1e-30)
        assert np.all(g[:, total:] == 0)


def check_dequant(gc, hc, maxT, lens):
    """f32 dequantization of gc against the oracle over hc: 1e-5 of the row RMS, zeros past
    each sequence's length. Returns the device outputs."""
    B, H = gc.og.batch, gc.og.num_kv_heads
    kr, vr = R.dequantize(hc, maxT)
    ko = torch.full((B, maxT, H, 128), 7.0, dtype=torch.float32, device="cuda")
    vo = torch.full((B, maxT, H, 128), 7.0, dtype=torch.float32, device="cuda")
    K.kvarn_dequantize(gc.g, gc.buf, ko, vo, maxT, K.KVARN_OUT_F32)
    torch.cuda.synchronize()
    for got, want in ((ko, kr), (vo, vr)):
        g = got.cpu().numpy().astype(np.float64)
        rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
        assert np.all(np.abs(g - want) <= 1e-5 * np.maximum(rms, 1e-30) + 1e-30)
        for b in range(B):
            assert np.all(g[b, lens[b]:] == 0)
    return ko, vo


@pytest.mark.parametrize("seed", list(range(24)))
def test_random_chunked_paged(seed):
    c = draw(5000 + seed)
    rng = np.random.Generator(np.random.PCG64(6000 + seed))
    B, H, G, bits, n_it = c["B"], c["H"], c["G"], c["bits"], c["n_it"]
    calls = int(rng.integers(2, 6))
    counts = rng.integers(0, 2 * G + 8, size=(calls, B)).astype(np.int32)
    counts[rng.random((calls, B)) < 0.2] = 0  # sequences left out of a call
    lens = counts.sum(axis=0)
    cap = (int(lens.max()) // G + 2) * G
    print("[case] random chunked/paged", seed, {k: v for k, v in c.items() if k not in ("law_kw", "T", "n_app")},
          "counts", counts.tolist(), "cap", cap, flush=True)
    tiles = cap // G
    npages = B * tiles + int(rng.integers(0, 5))
    pages = rng.permutation(npages)[:B * tiles].reshape(B, tiles).astype(np.int32)

    flat = GpuCache(B, H, cap, G, n_it, seed_sigma=seed, bits=bits)
    paged = PagedCache(B, H, cap, G, n_it, npages, seed_sigma=seed, bits=bits)
    paged.set_pages(pages)
    streams = [[[], []] for _ in range(B)]  # per sequence: K rows, V rows (uint16 [H][D] each)
    for i in range(calls):
        n = int(counts[i].max())
        k, v = synth.kv_host(synth.sub_seed(79, seed, i), B, max(n, 1), H, law=c["law"], **c["law_kw"])
        for b in range(B):
            streams[b][0].extend(k[b, :counts[i, b]])
            streams[b][1].extend(v[b, :counts[i, b]])
        cnt = torch.from_numpy(counts[i].copy()).cuda()
        kd, vd = from_u16(k[:, :n]), from_u16(v[:, :n])
        for gc in (flat, paged):
            K.kvarn_append_tokens(gc.g, gc.buf, kd, vd, n, cnt)
    torch.cuda.synchronize()
    hf, hp = flat.host_cache(), paged.host_cache()
    assert np.array_equal(hf.lens[:, 0, 0], lens)
    same_stored(hf, hp)
    assert np.array_equal(hp.page_map, pages)
    assert K.kvarn_cache_flags(flat.buf) & (K.KVARN_FLAG_CAPACITY | K.KVARN_FLAG_UNMAPPED) == 0
    assert K.kvarn_cache_flags(paged.buf) & (K.KVARN_FLAG_CAPACITY | K.KVARN_FLAG_UNMAPPED) == 0

    # every sequence: the bytes of a prefill of its own stream, which passes the oracle chain
    for b in range(B):
        T = int(lens[b])
        one = GpuCache(B, H, cap, G, n_it, seed_sigma=seed, bits=bits)
        ks = np.zeros((B, max(T, 1), H, 128), np.uint16)
        vs = np.zeros((B, max(T, 1), H, 128), np.uint16)
        if T:
            ks[:] = np.stack(streams[b][0])[None]
            vs[:] = np.stack(streams[b][1])[None]
        gpu_prefill(one, ks, vs, T)
        same_stored(one.host_cache(), hf, seqs=[b])
        if b == 0:
            check_prefill(one, ks, vs, T)

    # attention and dequantization: paged bit-equal to per-sequence, both against the oracle
    Hq = H * c["grp"]
    q = synth.q_host(synth.sub_seed(80, seed), B, Hq)
    ws, n = K.alloc_workspace(flat.g, Hq)
    outs = []
    for gc in (flat, paged):
        out = torch.full((B, Hq, 128), float("nan"), device="cuda")
        K.kvarn_attn_decode(gc.g, gc.buf, from_u16(q), Hq, 0.0, 0, ws, n, out)
        torch.cuda.synchronize()
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])
    check_attention(outs[0].numpy().astype(np.float64), hf, q, Hq)
    maxT = min(int(lens.max()) + 3, cap)
    kf, vf = check_dequant(flat, hf, maxT, lens)
    kp, vp = check_dequant(paged, hp, maxT, lens)
    assert torch.equal(kf, kp) and torch.equal(vf, vp)


def attn_close(got, ref, tol=2e-3):
    for b in range(ref.shape[0]):
        for g in range(ref.shape[1]):
            m = np.abs(ref[b, g]).max()
            d = np.abs(got[b, g] - ref[b, g]).max()
            assert d <= tol * m or (m == 0 and d == 0), (b, g, d, m)


@pytest.mark.parametrize("seed", list(range(12)))
def test_random_fused_steps(seed):
    rng = np.random.Generator(np.random.PCG64(70000 + seed))
    G = int(rng.choice((32, 64)))
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    grp, n_it, bits = int(rng.choice((1, 2, 3, 4, 8))), int(rng.integers(0, 5)), int(rng.choice((2, 3, 4)))
    T0, steps = int(rng.integers(0, 4 * G)), int(rng.integers(G // 2, G + 6))
    cap, Hq = ((T0 + steps) // G + 1) * G, H * grp
    print("[case] random fused steps", seed, dict(B=B, H=H, grp=grp, G=G, n_it=n_it, bits=bits, T0=T0, steps=steps),
          flush=True)
    k, v = synth.kv_host(synth.sub_seed(71, seed), B, T0 + steps, H)
    kd, vd = from_u16(k), from_u16(v)
    fused = GpuCache(B, H, cap, G, n_it, seed_sigma=seed, bits=bits)
    plain = GpuCache(B, H, cap, G, n_it, seed_sigma=seed, bits=bits)
    for gc in (fused, plain):
        gpu_prefill(gc, k, v, T0)
    ws, n = K.alloc_workspace(fused.g, Hq)
    out = torch.full((B, Hq, 128), float("nan"), device="cuda")
    for t in range(T0, T0 + steps):
        qb = synth.q_host(synth.sub_seed(72, seed, t), B, Hq)
        ref = R.append_attn_decode(fused.host_cache(), k[:, t], v[:, t], qb, Hq, 0.0, 0)
        K.kvarn_append_attn_decode(fused.g, fused.buf, kd[:, t].contiguous(), vd[:, t].contiguous(), from_u16(qb), Hq,
                                   0.0, 0, ws, n, out)
        K.kvarn_append_decode(plain.g, plain.buf, kd[:, t].contiguous(), vd[:, t].contiguous())
        torch.cuda.synchronize()
        attn_close(out.cpu().numpy().astype(np.float64), ref)
    hf, hp = fused.host_cache(), plain.host_cache()
    m = hf.defined_mask()
    assert np.array_equal(m, hp.defined_mask()) and np.array_equal(hf.buf[m], hp.buf[m])
    assert np.all(hf.lens == T0 + steps)
    q = from_u16(synth.q_host(synth.sub_seed(73, seed), B, Hq))
    o1, o2 = torch.empty(B, Hq, 128, device="cuda"), torch.empty(B, Hq, 128, device="cuda")
    K.kvarn_attn_decode(fused.g, fused.buf, q, Hq, 0.0, 0, ws, n, o1)
    K.kvarn_attn_decode_noalloc(fused.g, fused.buf, q, Hq, 0.0, 0, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
