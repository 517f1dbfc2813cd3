#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X.

Headline (`value`): prefill quantization throughput in GB/s of bf16 input on the
Llama-3.1-8B-shaped KV workload -- 32 layers x 8 KV heads x head_dim 128, 32768
tokens, batch 1, group 32, 3 VarN iterations, 2 bits -- one step = the 32 layer
caches quantized from 32 distinct input buffers resident in HBM by one
kvarn_quantize_prefill_layers call (one launch), issued eagerly. The step as 32
kvarn_quantize_prefill calls is reported beside it (`per_layer_calls`, also replayed as one
HIP graph). Beside it:
  * roofline of the quantize kernel: algorithmic bytes per launch (bf16 in + tile
    records out) over the launch time, measured with HIP events on the launch stream
    around the whole timed step loop and divided by the number of launches, against the
    8 TB/s HBM peak, the 4 GiB copy ceiling and a streaming kernel with the prefill's
    read/write mix;
  * long_prefill: the same quantizer on the long-reasoning shape (64 x 32768 tokens per
    layer, Student-t token norms), 32 launches;
  * decode: the Phi-4-14B-shaped run as configured (40 layers x 10 KV heads, 40 query
    heads, batch 32, 16384 -> 17408 tokens: 1024 steps of append + attention, every step
    timed), eagerly, fused, and as a HIP graph;
  * long_decode: the long-reasoning run (32 layers x 8 KV heads, 32 query heads, batch 64,
    32768 -> 36864 tokens: 4096 steps), timed on 16 windows of 8 steps spread evenly over
    the run; the steps between windows only append;
  * roundtrip: Qwen3-4B-shaped prefill (36 layers x 8 KV heads, batch 8 x 16384
    tokens, group 64, 2 VarN iterations) followed by a bf16 dequantization of every
    layer, with both kernels' launch times and algorithmic GB/s;
  * paged_chunked: decode attention of one Phi-4-shaped layer over a paged cache (a
    shuffled page map) against the per-sequence layout, and a Llama-3.1-8B-shaped layer
    written as 4 chunks by kvarn_append_tokens against one prefill call;
  * cpu_baseline: the CPU oracle on a bounded sample of the same workloads, one
    single-threaded process per host core used (at most --cpu-workers).

Prints one JSON line. Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
METRIC = "KV quantize GB/s (bf16 in) & % of HBM peak; decode-append tokens/s at 1 GPU"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def record_bytes(g: int, bits: int = 2) -> int:
    return g * 128 * bits // 8 + 2 * g + 6 * 128


def settle(torch, step, seconds=0.25):
    """Untimed steps until the GPU has been busy for `seconds`, before the warm-up steps:
    clocks rise over the first tens of milliseconds under load (a one-layer launch measured
    45.7 us after 3 warm-up steps, 43.4 us after 30 and 43.0 us after 200 on one box)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        step()
        torch.cuda.synchronize()


def bench_prefill(K, synth, torch, steps, warmup, layers=32, T=32768, H=8, G=32, n_it=3, bits=2, B=1,
                  distinct=True, graph=True, law=None, tag="prefill", batched=False):
    """`steps` steps of the `layers`-layer prefill, issued eagerly with nothing between them:
    one kvarn_quantize_prefill_layers call per step (batched; one launch per 64 layers), or
    one kvarn_quantize_prefill call per layer. The timed region is bracketed by HIP events
    on the launch stream (so the per-launch average is the kernel time of the step, gaps
    included) and by the wall clock."""
    g = K.geom(B, H, T, G, n_it, bits=bits)
    sig = synth.sign_vector(0)
    law = law or {}
    log(f"{tag} workload: {layers} layers x B={B} x T={T} x Hkv={H}, G={G}, iters={n_it}, {law or 'lognormal'}")
    n_in = layers if distinct else 1
    ks, vs = [], []
    for l in range(n_in):
        k, v = synth.kv_device(synth.sub_seed(2 if B == 1 else 5, l, 0), B, T, H, **law)
        ks.append(k)
        vs.append(v)
    caches = [K.alloc_cache(g, sig) for _ in range(layers if distinct else 1)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    if batched:
        assert distinct, "the multi-layer call needs distinct caches"

    def step(st=stream):
        if batched:
            K.kvarn_quantize_prefill_layers(g, caches, ks, vs, T, st)
            return
        for l in range(layers):
            i = l if distinct else 0
            K.kvarn_quantize_prefill(g, caches[i], ks[i], vs[i], T, st)

    launches_per_step = (layers + 63) // 64 if batched else layers
    settle(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = e0.elapsed_time(e1)
    # diagnostic only: every call bracketed by its own event pair (adds a dispatch per call)
    if batched:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
        for a0, a1 in ev:
            a0.record(stream)
            step()
            a1.record(stream)
    else:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(layers)]
        for l in range(layers):
            i = l if distinct else 0
            ev[l][0].record(stream)
            K.kvarn_quantize_prefill(g, caches[i], ks[i], vs[i], T, stream)
            ev[l][1].record(stream)
    torch.cuda.synchronize()
    isolated_ms = sorted(a.elapsed_time(b) for a, b in ev)
    graph_wall = None
    if graph:  # the same step as one HIP graph of its launches, replayed
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step(None)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            gr.replay()
        torch.cuda.synchronize()
        graph_wall = time.perf_counter() - t0
        del gr
    bytes_in = B * 2 * 2 * T * H * 128                       # K and V, bf16
    bytes_out = B * 2 * H * (T // G) * record_bytes(G, bits)  # tile records
    flags = K.kvarn_cache_flags(caches[0])
    del ks, vs, caches
    torch.cuda.empty_cache()
    return dict(wall=wall, graph_wall=graph_wall, region_ms=region_ms, launches=steps * launches_per_step,
                layers_per_launch=layers // launches_per_step,
                isolated_ms=isolated_ms, bytes_in=bytes_in, bytes_out=bytes_out, layers=layers, T=T, H=H, G=G,
                n_it=n_it, B=B, flags=flags)


def bench_decode(K, synth, torch, run_steps, windows=0, win_steps=8, warmup=4, layers=40, B=32, H=10, Hq=40,
                 T0=16384, cap=17408, G=32, n_it=3, pool=128, bits=2, kv_kw=None, variants=True, tag="decode"):
    """The configured decode run: `run_steps` steps of append + attention on every layer,
    from T0 prior tokens. windows == 0 times every step of the run. windows > 0 times
    `windows` windows of `win_steps` steps spread evenly over the run; the steps between
    them only append, so each window sees the cache the full run would have at that point.
    Decode K, V and Q come from a pool of `pool` pre-generated steps, cycled (the bytes
    moved do not depend on the values)."""
    assert T0 + run_steps <= cap, "the decode run does not fit the cache capacity"
    g = K.geom(B, H, cap, G, n_it, bits=bits)
    sig = synth.sign_vector(0)
    kv_kw = kv_kw or {}
    log(f"{tag} workload: {layers} layers x B={B} x Hkv={H} x Hq={Hq}, {T0} -> {T0 + run_steps} tokens, "
        + (f"{windows} windows x {win_steps} steps" if windows else "every step timed"))
    k0, v0 = synth.kv_device(synth.sub_seed(4 if B == 32 else 5, 0, 0), B, T0, H, **kv_kw)
    caches = [K.alloc_cache(g, sig) for _ in range(layers)]

    def reset():  # every layer back to the T0 prior tokens
        for c in caches:
            K.kvarn_quantize_prefill(g, c, k0, v0, T0)
        torch.cuda.synchronize()

    kp, vp = synth.kv_device(synth.sub_seed(4, 0, 1), B, pool, H, **kv_kw)  # [B][pool][H][D]
    kp = kp.transpose(0, 1).contiguous()                              # [pool][B][H][D]
    vp = vp.transpose(0, 1).contiguous()
    qp = torch.stack([synth.q_device(synth.sub_seed(4, 0, 2, s), B, Hq) for s in range(pool)])
    ws, nws = K.alloc_workspace(g, Hq)
    out = torch.empty(B, Hq, 128, device="cuda")
    stream = torch.cuda.current_stream()

    def step(s, fused=False, ev=None):
        kk, vv, qq = kp[s % pool], vp[s % pool], qp[s % pool]
        for l in range(layers):
            if fused:
                K.kvarn_append_attn_decode(g, caches[l], kk, vv, qq, Hq, 0.0, 0, ws, nws, out, stream)
                continue
            K.kvarn_append_decode(g, caches[l], kk, vv, stream)
            if ev is not None and l == layers - 1:
                ev[0].record(stream)
            K.kvarn_attn_decode(g, caches[l], qq, Hq, 0.0, 0, ws, nws, out, stream)
            if ev is not None and l == layers - 1:
                ev[1].record(stream)

    def advance(s):  # append-only step: the cache moves on as in the full run
        for l in range(layers):
            K.kvarn_append_decode(g, caches[l], kp[s % pool], vp[s % pool], stream)

    def run(fused=False):
        """The configured run (or its windows); returns (timed steps, wall s, event ms, mean context)."""
        reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if not windows:
            t0 = time.perf_counter()
            e0.record(stream)
            for s in range(run_steps):
                step(s, fused)
            e1.record(stream)
            torch.cuda.synchronize()
            return run_steps, time.perf_counter() - t0, e0.elapsed_time(e1), T0 + (run_steps - 1) / 2
        starts = [i * run_steps // windows for i in range(windows)]
        done, wall, ev_ms, ctx = 0, 0.0, 0.0, []
        s = 0
        for st in starts:
            while s < st:
                advance(s)
                s += 1
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record(stream)
            for _ in range(win_steps):
                step(s, fused)
                ctx.append(T0 + s)
                s += 1
            e1.record(stream)
            torch.cuda.synchronize()
            wall += time.perf_counter() - t0
            ev_ms += e0.elapsed_time(e1)
            done += win_steps
        return done, wall, ev_ms, sum(ctx) / len(ctx)

    # warm-up on the prefilled caches, then every run starts from T0 again
    reset()
    for s in range(warmup):
        step(s)
        step(s, fused=True)
    torch.cuda.synchronize()
    res = {}
    n, wall, ev_ms, ctx = run()
    res["eager"] = dict(steps=n, wall=wall, event_ms=ev_ms, ctx=ctx)
    if variants:
        n, wall, ev_ms, ctx = run(fused=True)
        res["fused"] = dict(steps=n, wall=wall, event_ms=ev_ms, ctx=ctx)
        # the fused step as one HIP graph, replayed once per step with the step's inputs
        # copied into the captured buffers first (inside the timed region)
        reset()
        k_in, v_in, q_in = torch.empty_like(kp[0]), torch.empty_like(vp[0]), torch.empty_like(qp[0])
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for l in range(layers):
                K.kvarn_append_attn_decode(g, caches[l], k_in, v_in, q_in, Hq, 0.0, 0, ws, nws, out)
        reset()  # the capture itself launched nothing, but start clean
        steps_g = run_steps if not windows else 0
        if steps_g:
            t0 = time.perf_counter()
            for s in range(steps_g):
                k_in.copy_(kp[s % pool])
                v_in.copy_(vp[s % pool])
                q_in.copy_(qp[s % pool])
                gr.replay()
            torch.cuda.synchronize()
            res["fused_graph"] = dict(steps=steps_g, wall=time.perf_counter() - t0)
        del gr
    # kernel timing at the middle of the run: the last layer's attention of 8 steps and
    # the first layer's append of 4 steps, each bracketed by events
    reset()
    mid = run_steps // 2
    for s in range(mid):
        advance(s)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(8)]
    for i in range(8):
        step(mid + i, ev=evs[i])
    ctx_attn = T0 + mid + 4
    ea = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
    for i, (a0, a1) in enumerate(ea):
        s = mid + 8 + i
        a0.record(stream)
        K.kvarn_append_decode(g, caches[0], kp[s % pool], vp[s % pool], stream)
        a1.record(stream)
        for l in range(1, layers):
            K.kvarn_append_decode(g, caches[l], kp[s % pool], vp[s % pool], stream)
    torch.cuda.synchronize()
    attn_ms = sorted(a.elapsed_time(b) for a, b in evs)
    append_ms = sorted(a.elapsed_time(b) for a, b in ea)
    flags = K.kvarn_cache_flags(caches[0])
    # attention bytes per call at the event-timed context: K and V records of the full
    # tiles + tail rows + q + out
    nfull = ctx_attn // G
    attn_bytes = B * H * (2 * nfull * record_bytes(G, bits) + 2 * (ctx_attn % G) * 256) + B * Hq * (256 + 512)
    del caches, k0, v0
    torch.cuda.empty_cache()
    return dict(res=res, B=B, layers=layers, H=H, Hq=Hq, T0=T0, run_steps=run_steps, windows=windows,
                win_steps=win_steps, attn_ms=attn_ms, append_ms=append_ms, attn_bytes=attn_bytes, ctx_attn=ctx_attn,
                flags=flags)


def bench_roundtrip(K, synth, torch, steps, warmup=2, layers=36, B=8, T=16384, H=8, G=64, n_it=2, bits=2,
                    n_inputs=4):
    """Qwen3-4B-shaped prefill + dequantize round trip: per layer, quantize a batch of 8
    sequences x 16384 tokens (G = 64, 2 VarN iterations, 2% of tokens with norm x50), then
    dequantize the whole cache back to bf16. Inputs cycle over n_inputs distinct buffers."""
    g = K.geom(B, H, T, G, n_it, bits=bits)
    sig = synth.sign_vector(0)
    log(f"round-trip workload: {layers} layers x B={B} x T={T} x Hkv={H}, G={G}, iters={n_it}")
    ins = [synth.kv_device(synth.sub_seed(3, l, 0), B, T, H, law="spike", p=0.02, factor=50.0)
           for l in range(n_inputs)]
    caches = [K.alloc_cache(g, sig) for _ in range(layers)]
    ko = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        for l in range(layers):
            k, v = ins[l % n_inputs]
            if ev is not None:
                ev[l][0].record(stream)
            K.kvarn_quantize_prefill(g, caches[l], k, v, T, stream)
            if ev is not None:
                ev[l][1].record(stream)
            K.kvarn_dequantize(g, caches[l], ko, vo, T, K.KVARN_OUT_BF16, stream)
            if ev is not None:
                ev[l][2].record(stream)

    settle(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(layers)]
    step(ev)
    torch.cuda.synchronize()
    pf_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    dq_ms = sorted(e[1].elapsed_time(e[2]) for e in ev)
    flags = K.kvarn_cache_flags(caches[0])
    bytes_in = 2 * B * T * H * 128 * 2                          # K and V, bf16
    bytes_rec = 2 * B * H * (T // G) * record_bytes(G, bits)    # tile records
    del ins, caches, ko, vo
    torch.cuda.empty_cache()
    pf_avg, dq_avg = sum(pf_ms) / layers, sum(dq_ms) / layers
    pf_gbs = (bytes_in + bytes_rec) / (pf_avg * 1e-3) / 1e9
    dq_gbs = (bytes_rec + bytes_in) / (dq_avg * 1e-3) / 1e9
    return {
        "workload": "qwen3-4b-shaped prefill quantize + bf16 dequantize round trip", "layers": layers,
        "batch": B, "tokens": T, "kv_heads": H, "group": G, "varn_iters": n_it, "bits": bits,
        "input": "bf16, outlier channels x20, 2% of tokens x50",
        "ms_per_step": round(wall * 1e3 / steps, 3), "steps": steps,
        "prefill": {"kernel": f"prefill_kernel<2,false,{'false' if bits == 2 else 'true'},1>",
                    "avg_launch_us": round(pf_avg * 1e3, 2), "bytes_per_launch": bytes_in + bytes_rec,
                    "achieved": round(pf_gbs, 1), "frac": round(pf_gbs / HBM_PEAK_GBS, 4), "unit": "GB/s"},
        "dequantize": {"kernel": f"dequant_kernel<{bits}> (bf16 out)",
                       "avg_launch_us": round(dq_avg * 1e3, 2),
                       "bytes_per_launch": bytes_rec + bytes_in, "bytes_read": bytes_rec, "bytes_written": bytes_in,
                       "achieved": round(dq_gbs, 1), "frac": round(dq_gbs / HBM_PEAK_GBS, 4), "unit": "GB/s"},
        "flags": flags,
    }


def bench_paged_chunked(K, synth, torch, reps=5, calls=20, bits=2):
    """The paged and ragged row, each measured beside the per-sequence layout it replaces:
    decode attention of one Phi-4-shaped layer (B = 32, 10 KV heads, 40 query heads, 16,900
    stored tokens) over a paged cache whose page map is a seeded permutation of the pool,
    against the same tokens in a per-sequence cache (calls alternate between the two); and
    a Llama-3.1-8B-shaped layer (32,768 tokens, 8 KV heads) written as 4 chunks of 8,192
    tokens by kvarn_append_tokens into an emptied cache, against one kvarn_quantize_prefill
    of all of it. Event-timed, `calls` calls per sample, best of `reps` samples."""
    import numpy as np
    stream = torch.cuda.current_stream()
    sig = synth.sign_vector(0)
    B, H, Hq, cap, ctx, G, n_it = 32, 10, 40, 17408, 16900, 32, 3
    tiles = cap // G
    log(f"paged attention workload: B={B} x Hkv={H} x Hq={Hq}, {ctx} tokens, pool of {B * tiles} pages")
    gs = K.geom(B, H, cap, G, n_it, bits=bits)
    gp = K.geom(B, H, cap, G, n_it, bits=bits, num_pages=B * tiles)
    k, v = synth.kv_device(synth.sub_seed(4, 0, 0), B, ctx, H)
    cs, cp = K.alloc_cache(gs, sig), K.alloc_cache(gp, sig)
    perm = np.random.default_rng(11).permutation(B * tiles).reshape(B, tiles).astype(np.int32)
    K.kvarn_cache_set_pages(gp, cp, torch.from_numpy(perm).cuda(), 0, tiles)
    K.kvarn_quantize_prefill(gs, cs, k, v, ctx)
    K.kvarn_quantize_prefill(gp, cp, k, v, ctx)
    del k, v
    q = synth.q_device(synth.sub_seed(4, 0, 2, 0), B, Hq)
    runs = {}
    for name, g, c in (("per_sequence", gs, cs), ("paged", gp, cp)):
        ws, nws = K.alloc_workspace(g, Hq)
        runs[name] = (g, c, ws, nws, torch.empty(B, Hq, 128, device="cuda"))

    def attn(name):
        g, c, ws, nws, out = runs[name]
        K.kvarn_attn_decode(g, c, q, Hq, 0.0, 0, ws, nws, out, stream)

    def timed(fns, n):
        best = {}
        for f in fns:
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(reps):
            for f in fns:
                e0.record(stream)
                for _ in range(n):
                    f()
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / n
                best[f] = min(best.get(f, us), us)
        return [best[f] for f in fns]

    us_seq, us_pg = timed([lambda: attn("per_sequence"), lambda: attn("paged")], calls)
    nfull = ctx // G
    bytes_seq = B * H * (2 * nfull * record_bytes(G, bits) + 2 * (ctx % G) * 256) + B * Hq * (256 + 512)
    bytes_pg = bytes_seq + B * nfull * 4  # plus the page map entries
    same = torch.equal(runs["per_sequence"][4], runs["paged"][4])
    paged = {"workload": f"phi-4-14b-shaped decode attention, one layer, {ctx} stored tokens per sequence",
             "page_map": "a seeded permutation of a pool of B x capacity/G pages",
             "us_per_call_paged": round(us_pg, 2), "us_per_call_per_sequence": round(us_seq, 2),
             "paged_over_per_sequence": round(us_pg / us_seq, 4), "bytes_per_call": bytes_pg,
             "achieved_paged": round(bytes_pg / (us_pg * 1e-6) / 1e9, 1),
             "frac_paged": round(bytes_pg / (us_pg * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
             "outputs_bit_equal": bool(same)}
    log(f"paged attention: {paged}")
    del runs, cs, cp
    torch.cuda.empty_cache()

    Bc, Tc, Hc, nch = 1, 32768, 8, 4
    gc = K.geom(Bc, Hc, Tc, G, n_it, bits=bits)
    kc, vc = synth.kv_device(synth.sub_seed(2, 0, 0), Bc, Tc, Hc)
    step = Tc // nch
    chunks = [(kc[:, i * step:(i + 1) * step].contiguous(), vc[:, i * step:(i + 1) * step].contiguous())
              for i in range(nch)]
    ca, cb = K.alloc_cache(gc, sig), K.alloc_cache(gc, sig)

    def one():
        K.kvarn_quantize_prefill(gc, ca, kc, vc, Tc, stream)

    def chunked():
        K.kvarn_quantize_prefill(gc, cb, kc, vc, 0, stream)  # empties the cache (len = 0)
        for kk, vv in chunks:
            K.kvarn_append_tokens(gc, cb, kk, vv, step, None, stream)

    us_one, us_ch = timed([one, chunked], 10)
    bytes_in = 2 * 2 * Bc * Tc * Hc * 128
    bytes_all = bytes_in + 2 * Bc * Hc * (Tc // G) * record_bytes(G, bits)
    chunk = {"workload": f"llama3.1-8b-shaped layer, {Tc} tokens x {Hc} KV heads, {nch} chunks of {step} tokens "
                         "appended to an emptied cache",
             "us_one_prefill_call": round(us_one, 2), "us_chunked": round(us_ch, 2),
             "chunked_over_one_call": round(us_ch / us_one, 4),
             "value_chunked": round(bytes_in / (us_ch * 1e-6) / 1e9, 1), "unit": "GB/s bf16-in",
             "frac_chunked": round(bytes_all / (us_ch * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"chunked prefill: {chunk}")
    del ca, cb, kc, vc, chunks
    torch.cuda.empty_cache()
    return {"paged_attention": paged, "chunked_prefill": chunk}


def bench_bf16_decode(torch, steps=8, warmup=2, layers=40, B=32, H=10, Hq=40, T=16384):
    """Plain bf16 decode attention over a bf16 KV cache of the same shapes (no quantization):
    per layer scores = q K^T (K stored transposed, [B][H][D][T]), fp32 softmax, out = p V,
    as batched matrix products whose right operands are contiguous."""
    grp = Hq // H
    gen = torch.Generator(device="cuda").manual_seed(5)
    kt = [torch.randn(B, H, 128, T, generator=gen, device="cuda", dtype=torch.bfloat16) for _ in range(layers)]
    vv = [torch.randn(B, H, T, 128, generator=gen, device="cuda", dtype=torch.bfloat16) for _ in range(layers)]
    q = torch.randn(B, H, grp, 128, generator=gen, device="cuda", dtype=torch.bfloat16)
    scale = 1.0 / 128 ** 0.5

    def step():
        for l in range(layers):
            sc = torch.matmul(q, kt[l]).float() * scale
            p = torch.softmax(sc, dim=-1).to(torch.bfloat16)
            torch.matmul(p, vv[l])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cache_bytes = layers * 2 * B * H * T * 128 * 2
    del kt, vv
    torch.cuda.empty_cache()
    return dict(ms_per_step=round(wall * 1e3 / steps, 3), tokens_per_s=round(B * steps / wall, 1),
                cache_GB=round(cache_bytes / 1e9, 2), context=T)


def copy_ceiling(torch, gib=4):
    """Device-to-device copy of `gib` GiB: the practical HBM ceiling (read + write bytes / time)."""
    n = gib * (1 << 30)
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return dict(bytes=2 * n, ms=round(ms, 3), GBps=round(2 * n / (ms * 1e-3) / 1e9, 1))


def mix_ceiling(torch, bytes_in, bytes_out, layers=32, steps=10, grids=(1024, 2048, 4096, 8192)):
    """The practical ceiling of a kernel with a given mix of reads and writes (the prefill's
    or the dequantizer's): a plain streaming kernel (libkvarn_bench.so) that reads `bytes_in`
    and writes `bytes_out` per launch, over `layers` distinct buffer pairs per step like the
    benchmarked step; the best of a small sweep over grids and over plain or non-temporal
    stores, timed with events over `steps` steps."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)), "kv_cache_bit_amd",
                                   "libkvarn_bench.so"))
    kernels = {"plain": lib.kvarn_bench_stream_mix, "nt_stores": lib.kvarn_bench_stream_mix_nt}
    for f in kernels.values():
        f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                      ctypes.c_void_p]
        f.restype = ctypes.c_int
    ins = [torch.ones(bytes_in, dtype=torch.uint8, device="cuda") for _ in range(layers)]
    outs = [torch.empty(bytes_out, dtype=torch.uint8, device="cuda") for _ in range(layers)]
    st = torch.cuda.current_stream()
    best = None
    for (kind, f), grid in [(kf, g) for kf in kernels.items() for g in grids]:
        def step():
            for l in range(layers):
                assert f(ins[l].data_ptr(), bytes_in, outs[l].data_ptr(), bytes_out, grid, st.cuda_stream) == 0
        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(steps):
            step()
        e1.record(st)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (steps * layers)
        gbs = (bytes_in + bytes_out) / (us * 1e-6) / 1e9
        if best is None or gbs > best["GBps"]:
            best = dict(GBps=round(gbs, 1), launch_us=round(us, 2), grid=grid, stores=kind)
    del ins, outs
    torch.cuda.empty_cache()
    return dict(best, bytes_read=bytes_in, bytes_written=bytes_out,
                read_share=round(bytes_in / (bytes_in + bytes_out), 4))


def _oracle_prefill_layer(job):
    """One layer of the prefill workload through the oracle, in a worker process with one
    BLAS thread; returns the oracle's seconds."""
    tokens, layer = job
    from threadpoolctl import threadpool_limits

    from kv_cache_bit_amd import synth
    from oracle import kvarn_ref as R
    with threadpool_limits(1):
        H, G = 8, 32
        k, v = synth.kv_host(synth.sub_seed(2, layer, 0), 1, tokens, H)
        c = R.Cache(R.Geom(1, H, 128, tokens, G, 3, 2), synth.sign_vector(0))
        t0 = time.perf_counter()
        R.quantize_prefill(c, k, v, tokens)
        return time.perf_counter() - t0


def _oracle_decode_row(job):
    """One batch row of the Phi-4-shaped decode through the oracle (one BLAS thread): set-up
    (untimed), then one append + attention step; returns the step's seconds."""
    T, H, Hq, row = job
    from threadpoolctl import threadpool_limits

    from kv_cache_bit_amd import synth
    from oracle import kvarn_ref as R
    with threadpool_limits(1):
        G = 32
        c = R.Cache(R.Geom(1, H, 128, T + 2 * G, G, 3, 2), synth.sign_vector(0))
        k, v = synth.kv_host(synth.sub_seed(4, row, 0), 1, T, H)
        R.quantize_prefill(c, k, v, T)
        kn, vn = synth.kv_host(synth.sub_seed(4, row, 1), 1, 1, H)
        q = synth.q_host(synth.sub_seed(4, row, 2), 1, Hq)
        t0 = time.perf_counter()
        R.append_decode(c, kn[:, 0], vn[:, 0])
        R.attn_decode(c, q, Hq)
        return time.perf_counter() - t0


def _pool_map(fn, jobs, workers):
    """Run fn(job) for every job in a child interpreter of its own, at most `workers` at a
    time. The children are plain subprocesses: they never touch the GPU, every one of them
    has exited when this returns, and no helper process (such as the multiprocessing
    module's resource tracker) is left running. Returns (results, wall seconds from the
    first job's start to the last job's end)."""
    import subprocess
    from concurrent.futures import ThreadPoolExecutor
    root = os.path.dirname(os.path.abspath(__file__))
    prog = ("import json, sys, time; import bench; t0 = time.time(); "
            "r = getattr(bench, sys.argv[1])(json.loads(sys.argv[2])); print(json.dumps([r, t0, time.time()]))")

    def run(job):
        p = subprocess.run([sys.executable, "-c", prog, fn.__name__, json.dumps(list(job))], cwd=root,
                           capture_output=True, text=True, timeout=900)
        if p.returncode != 0:
            raise RuntimeError(f"oracle worker failed ({p.returncode}): {p.stderr[-2000:]}")
        return json.loads(p.stdout.strip().splitlines()[-1])

    with ThreadPoolExecutor(workers) as ex:  # threads only wait on the children
        res = list(ex.map(run, jobs))
    return [r[0] for r in res], max(r[2] for r in res) - min(r[1] for r in res)


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(tokens, layers, workers):
    """The oracle's prefill on layers 0..layers-1 of the prefill workload, one layer per
    worker process (one thread each), all workers at once: GB/s of bf16 input."""
    dts, wall = _pool_map(_oracle_prefill_layer, [(tokens, l) for l in range(layers)], workers)
    gb = layers * 2 * 2 * tokens * 8 * 128 / 1e9
    return dict(value=round(gb / wall, 5), unit="GB/s", cores=workers, kind="oracle",
                single_thread_value=round(gb / sum(dts), 5), host_cores=host_cores(),
                sample=f"layers 0..{layers - 1} of the prefill workload ({tokens} tokens x 8 KV heads x K and V "
                       f"each, {layers * 2 * 8 * tokens // 32} tiles), one layer per process on {workers} "
                       f"processes with one thread each: {sum(dts):.1f} s of oracle time in {wall:.1f} s; "
                       "NumPy fp64")


def cpu_baseline_decode(workers, T=16384, H=10, Hq=40, layers=40):
    """The oracle's decode step (append + attention by definition over the dequantized cache)
    on `workers` batch rows of the Phi-4-shaped decode at once, one row per process, scaled
    to the 40-layer step: tokens/s."""
    dts, _ = _pool_map(_oracle_decode_row, [(T, H, Hq, r) for r in range(workers)], workers)
    step = max(dts) * layers  # the rows run side by side; one step of every row and layer
    return dict(value=round(workers / step, 6), unit="tokens/s", cores=workers, kind="oracle",
                host_cores=host_cores(),
                sample=f"{workers} batch rows of the decode workload ({H} KV heads x {Hq} query heads, {T}-token "
                       f"context), one per process with one thread each: one append + attention step, "
                       f"{max(dts):.1f} s per row-layer, scaled to {layers} layers; NumPy fp64")


# HBM traffic of a kernel from committed rocprofv3 counter summaries: FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch) scaled by what the same counters read for a 4 GiB device
# copy. The figures stand only while the kernel sources hash to the digest recorded
# with them; otherwise traffic is reported as null.
KERNEL_SOURCES = ["kv_cache_bit_amd/csrc/kvarn_common.h", "kv_cache_bit_amd/csrc/kvarn_launch.h"]
PREFILL_SOURCES = ["kv_cache_bit_amd/csrc/quantize.hip", "kv_cache_bit_amd/csrc/quantize_dev.h"]
ATTN_SOURCES = ["kv_cache_bit_amd/csrc/attn.hip", "kv_cache_bit_amd/csrc/quantize_dev.h"]
DEQUANT_SOURCES = ["kv_cache_bit_amd/csrc/dequant.hip"]


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for f in files:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counted_traffic(profile, sources):
    """Bytes per launch from a profiles/ counter summary, or None if stale or absent."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", profile)
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_digest") != source_digest(sources + KERNEL_SOURCES):
            return None
        fetch = float(kv["FETCH_SIZE_KiB"]) * float(kv["fetch_scale"])
        write = float(kv["WRITE_SIZE_KiB"]) * float(kv["write_scale"])
        return int(round((fetch + write) * 1024))
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1024,
                    help="decode steps of the Phi-4-shaped run (16384 -> 17408 tokens), every step timed")
    ap.add_argument("--long-steps", type=int, default=4096,
                    help="decode steps of the long-reasoning run (32768 -> 36864 tokens)")
    ap.add_argument("--long-windows", type=int, default=16, help="timed windows of 8 steps over the long run")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-reasoning prefill and decode (64 x 32768-token contexts, Llama-3.1-8B KV geometry)")
    ap.add_argument("--no-roundtrip", action="store_true",
                    help="skip the Qwen3-4B-shaped prefill + dequantize round trip")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-attention and chunked-prefill measurements")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--cpu-workers", type=int, default=8,
                    help="oracle processes (one thread each) of the CPU baseline, at most the host's cores")
    ap.add_argument("--no-copy", action="store_true", help="skip the 4 GiB device copy ceiling")
    ap.add_argument("--no-bf16", action="store_true", help="skip the plain bf16 decode-attention baseline")
    ap.add_argument("--bits", type=int, default=2, choices=(2, 3, 4),
                    help="code width of both workloads (the pages' method, and the headline, use 2)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the quantizer shards by KV head and sequence with no exchange, see the design notes.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from kv_cache_bit_amd import kvarn as K
    from kv_cache_bit_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    log("device", torch.cuda.get_device_name(0))
    # the headline: the 32-layer prefill as one kvarn_quantize_prefill_layers call per step
    # (one launch); beside it the same step as 32 kvarn_quantize_prefill calls
    # (no graph replay of the one-launch step: a graph of one launch adds nothing, and its
    # replays would mix into the kernel's trace average)
    pf = bench_prefill(K, synth, torch, args.steps, args.warmup, bits=args.bits, batched=True, graph=False)
    pl = bench_prefill(K, synth, torch, args.steps, args.warmup, bits=args.bits, graph=True, tag="prefill per layer")

    def prefill_figures(r):
        ms = r["wall"] * 1e3 / args.steps
        bpl = r["layers_per_launch"] * (r["bytes_in"] + r["bytes_out"])
        us = r["region_ms"] * 1e3 / r["launches"]  # events over the timed region, per launch
        iso = r["isolated_ms"]
        return dict(ms_step=ms, value=r["layers"] * r["bytes_in"] / (ms * 1e-3) / 1e9,
                    total_gbs=r["layers"] * (r["bytes_in"] + r["bytes_out"]) / (ms * 1e-3) / 1e9,
                    bpl=bpl, launch_us=us, achieved=bpl / (us * 1e-6) / 1e9,
                    graph_ms=(r["graph_wall"] * 1e3 / args.steps if r["graph_wall"] else None),
                    iso_us=iso[len(iso) // 2] * 1e3)

    f, fl = prefill_figures(pf), prefill_figures(pl)
    ms_step, value, achieved, launch_us = f["ms_step"], f["value"], f["achieved"], f["launch_us"]
    log(f"prefill (one call): {ms_step:.3f} ms/step, {value:.1f} GB/s bf16-in; "
        f"{launch_us:.2f} us per launch of {pf['layers_per_launch']} layers -> {achieved:.1f} GB/s")
    log(f"prefill (a call per layer): {fl['ms_step']:.3f} ms/step, {fl['value']:.1f} GB/s bf16-in; "
        f"{fl['launch_us']:.2f} us per launch -> {fl['achieved']:.1f} GB/s")
    abl = "true" if args.bits != 2 else "false"
    kname = f"prefill_layers_kernel<1, {abl}, 1>"
    per_layer_bytes = pf["bytes_in"] + pf["bytes_out"]
    traffic_layer = counted_traffic("prefill_kernel_llama8b_32k_pmc.txt", PREFILL_SOURCES) if args.bits == 2 else None
    # the multi-layer launch's own counters hold for a launch of 32 layers
    traffic_launch = (counted_traffic("prefill_layers_kernel_llama8b_32k_pmc.txt", PREFILL_SOURCES)
                      if args.bits == 2 and pf["layers_per_launch"] == 32 else None)
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "llama3.1-8b-shaped KV prefill quantize", "layers": pf["layers"], "batch": 1,
                   "tokens": pf["T"], "kv_heads": pf["H"], "head_dim": 128, "group": pf["G"],
                   "varn_iters": pf["n_it"], "bits": args.bits,
                   "input": "bf16, outlier channels x20, 5% lognormal tokens",
                   "call": "kvarn_quantize_prefill_layers: the 32 layers' caches in one call (one launch)"},
        "hbm_frac_step": round(f["total_gbs"] / HBM_PEAK_GBS, 4),

        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_launch, "traffic_unit": "bytes/launch",
                     "traffic_over_bytes": (round(traffic_launch / f["bpl"], 4) if traffic_launch else None),
                     "kernel": kname, "layers_per_launch": pf["layers_per_launch"], "bytes_per_launch": f["bpl"],
                     "avg_launch_us": round(launch_us, 2), "launches_timed": pf["launches"],
                     "timing": "HIP events on the launch stream around the timed step loop, / launches",
                     "isolated_launch_us_median": round(f["iso_us"], 2),
                     "source_digest": source_digest(PREFILL_SOURCES + KERNEL_SOURCES)},
        "per_layer_calls": {
            "call": "kvarn_quantize_prefill once per layer (32 launches per step)",
            "value": round(fl["value"], 2), "unit": "GB/s bf16-in", "ms_per_step": round(fl["ms_step"], 4),
            "step_as_graph": {"ms_per_step": round(fl["graph_ms"], 4),
                              "value": round(pl["layers"] * pl["bytes_in"] / (fl["graph_ms"] * 1e-3) / 1e9, 2)},
            "roofline": {"kernel": "prefill_kernel<1, %s, %s, 1>" % ("false", abl), "bytes_per_launch": per_layer_bytes,
                         "avg_launch_us": round(fl["launch_us"], 2), "achieved": round(fl["achieved"], 1),
                         "frac": round(fl["achieved"] / HBM_PEAK_GBS, 4), "traffic": traffic_layer,
                         "isolated_launch_us_median": round(fl["iso_us"], 2)}},
        "flags": pf["flags"],
    }
    if not args.no_copy:
        res["copy_ceiling"] = copy_ceiling(torch)
        log(f"copy ceiling: {res['copy_ceiling']}")
        mc = mix_ceiling(torch, pf["bytes_in"], pf["bytes_out"])
        res["mix_ceiling"] = mc
        res["roofline"]["frac_of_mix_ceiling"] = round(achieved / mc["GBps"], 4)
        res["per_layer_calls"]["roofline"]["frac_of_mix_ceiling"] = round(fl["achieved"] / mc["GBps"], 4)
        log(f"streaming ceiling at the prefill's read/write mix: {mc}")
    if not args.no_long:
        lp = bench_prefill(K, synth, torch, 1, 1, layers=32, B=64, distinct=False, graph=False, bits=args.bits,
                           law=dict(law="student_t", nu=3.0, n_outlier_ch=8, ch_mult=30.0), tag="long prefill")
        lus = lp["region_ms"] * 1e3 / lp["launches"]
        lb = lp["bytes_in"] + lp["bytes_out"]
        res["long_prefill"] = {
            "workload": "long-reasoning prefill quantize: llama3.1-8b KV geometry, 64 x 32768 tokens per layer",
            "layers": lp["layers"], "batch": lp["B"], "tokens": lp["T"], "kv_heads": lp["H"],
            "input": "bf16, Student-t (nu 3) token norms, 8 outlier channels x30",
            "ms_per_step": round(lp["wall"] * 1e3, 3),
            "value": round(lp["layers"] * lp["bytes_in"] / lp["wall"] / 1e9, 1), "unit": "GB/s bf16-in",
            "avg_launch_us": round(lus, 2), "bytes_per_launch": lb,
            "achieved": round(lb / (lus * 1e-6) / 1e9, 1), "frac": round(lb / (lus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "flags": lp["flags"], "note": "one input buffer and cache reused by the 32 launches (8.6 GB each)"}
        log(f"long prefill: {res['long_prefill']}")
    if not args.no_decode:
        dc = bench_decode(K, synth, torch, args.decode_steps, bits=args.bits)
        res["decode"] = decode_report(dc, args.bits, "phi-4-14b-shaped decode: append + attn_decode")
        ah = res["decode"]
        ah["roofline"]["traffic"] = (counted_traffic("attn_kernel_phi4_decode_pmc.txt", ATTN_SOURCES)
                                     if args.bits == 2 else None)
        ah["roofline"]["traffic_unit"] = "bytes/launch (tile pass)"
        log(f"decode: {ah}")
        if not args.no_bf16:
            bf = bench_bf16_decode(torch)
            ah["bf16_baseline"] = dict(bf, kind="plain bf16 KV cache, torch batched products, same shapes")
            best = max(v for k, v in ah.items() if k.endswith("tokens_per_s"))
            ah["speedup_vs_bf16"] = round(best / bf["tokens_per_s"], 2)
            log(f"bf16 baseline: {bf}")
    if not args.no_long:
        torch.cuda.empty_cache()
        lg = bench_decode(K, synth, torch, args.long_steps, windows=args.long_windows, win_steps=8, warmup=2,
                          layers=32, B=64, H=8, Hq=32, T0=32768, cap=36864, bits=args.bits,
                          kv_kw=dict(law="student_t", nu=3.0, n_outlier_ch=8, ch_mult=30.0), tag="long decode")
        res["long_decode"] = decode_report(lg, args.bits,
                                           "long-reasoning stress decode: llama3.1-8b KV geometry, 64 sequences")
        res["long_decode"]["input"] = "bf16, Student-t (nu 3) token norms, 8 outlier channels x30"
        log(f"long decode: {res['long_decode']}")
    if not args.no_roundtrip:
        rt = bench_roundtrip(K, synth, torch, max(1, args.steps // 3), bits=args.bits)
        dq = rt["dequantize"]
        if args.bits == 2:
            dq["traffic"] = counted_traffic("dequant_kernel_qwen3_pmc.txt", DEQUANT_SOURCES)
            dq["source_digest"] = source_digest(DEQUANT_SOURCES + KERNEL_SOURCES)
        if not args.no_copy:  # the streaming ceiling at the dequantizer's mix (15% read, 85% written)
            # (grids other than the prefill mix's, so a counter summary keyed by kernel and
            # grid keeps the two mixes apart)
            mc = mix_ceiling(torch, dq["bytes_read"], dq["bytes_written"], layers=8,
                             grids=(1536, 3072, 6144, 12288))
            dq["mix_ceiling"] = mc
            dq["frac_of_mix_ceiling"] = round(dq["achieved"] / mc["GBps"], 4)
        res["roundtrip"] = rt
        log(f"round trip: {rt['ms_per_step']} ms/step; prefill {rt['prefill']['avg_launch_us']} us "
            f"({rt['prefill']['achieved']} GB/s), dequantize {rt['dequantize']['avg_launch_us']} us "
            f"({rt['dequantize']['achieved']} GB/s) per layer")
    if not args.no_paged:
        res["paged_chunked"] = bench_paged_chunked(K, synth, torch, bits=args.bits)
    if not args.no_cpu:
        workers = max(1, min(args.cpu_workers, host_cores()))
        log(f"cpu baseline (oracle) on {workers} processes ...")
        res["cpu_baseline"] = cpu_baseline(args.cpu_tokens, workers, workers)
        if "decode" in res:
            log("cpu baseline, decode step (oracle) ...")
            res["decode"]["cpu_baseline"] = cpu_baseline_decode(workers)
    print(json.dumps(res), flush=True)


def decode_report(dc, bits, workload):
    r = dc["res"]
    B = dc["B"]
    e = r["eager"]
    rep = {"workload": workload, "layers": dc["layers"], "batch": B, "kv_heads": dc["H"], "q_heads": dc["Hq"],
           "context_start": dc["T0"], "context_end": dc["T0"] + dc["run_steps"], "run_steps": dc["run_steps"],
           "timed": ("every step of the run" if not dc["windows"] else
                     f"{dc['windows']} windows x {dc['win_steps']} steps spread evenly over the run (the steps "
                     "between windows append only)"),
           "steps_timed": e["steps"], "mean_context_timed": round(e["ctx"], 1),
           "tokens_per_s": round(B * e["steps"] / e["wall"], 1), "ms_per_step": round(e["wall"] * 1e3 / e["steps"], 3),
           "tokens_per_s_events": round(B * e["steps"] / (e["event_ms"] * 1e-3), 1), "flags": dc["flags"]}
    if "fused" in r:
        rep["fused_tokens_per_s"] = round(B * r["fused"]["steps"] / r["fused"]["wall"], 1)
    if "fused_graph" in r:
        rep["fused_graph_tokens_per_s"] = round(B * r["fused_graph"]["steps"] / r["fused_graph"]["wall"], 1)
    am, apm = dc["attn_ms"], dc["append_ms"]
    a_avg = sum(am) / len(am)
    gbs = dc["attn_bytes"] / (a_avg * 1e-3) / 1e9
    rep["attn_avg_us"] = round(a_avg * 1e3, 2)
    rep["append_us"] = round(apm[len(apm) // 2] * 1e3, 2)
    rep["append_share"] = round(apm[len(apm) // 2] / (apm[len(apm) // 2] + a_avg), 4)
    rep["roofline"] = {"bound": "hbm", "kernel": f"attn_kernel<32, {bits}> + merge_kernel", "achieved": round(gbs, 1),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                       "bytes_per_launch": dc["attn_bytes"], "context": dc["ctx_attn"],
                       "timing": "events around the last layer's attention call of 8 steps at mid-run"}
    # at 100% of HBM the step would move every layer's attention bytes once
    rep["tokens_per_s_at_hbm_peak"] = round(B / (dc["layers"] * dc["attn_bytes"] / (HBM_PEAK_GBS * 1e9)), 1)
    return rep


if __name__ == "__main__":
    main()
