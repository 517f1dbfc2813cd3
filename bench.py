#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X.

Headline (`value`): prefill quantization throughput in GB/s of bf16 input on the
Llama-3.1-8B-shaped KV workload -- 32 layers x 8 KV heads x head_dim 128, 32768
tokens, batch 1, group 32, 3 VarN iterations, 2 bits -- one step = the 32 layer
caches quantized from 32 distinct input buffers resident in HBM, issued eagerly (the
same step replayed as one HIP graph is reported beside it). Beside it:
  * roofline of the quantize kernel: algorithmic bytes per launch (bf16 in + tile
    records out) over its average launch time measured with HIP events on the
    launch stream, against the 8 TB/s HBM peak;
  * decode: Phi-4-14B-shaped decode (40 layers x 10 KV heads, 40 query heads,
    batch 32, 16384 prior tokens), tokens/s of the append + fused attention loop;
  * long_decode: the long-reasoning stress shape (32 layers x 8 KV heads, 32 query heads,
    batch 64 x 32768-token contexts, Student-t token norms), decode tokens/s;
  * roundtrip: Qwen3-4B-shaped prefill (36 layers x 8 KV heads, batch 8 x 16384
    tokens, group 64, 2 VarN iterations) followed by a bf16 dequantization of every
    layer, with both kernels' launch times and algorithmic GB/s;
  * cpu_baseline: the CPU oracle on a bounded sample of the same prefill workload.

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


def bench_prefill(K, synth, torch, steps, warmup, layers=32, T=32768, H=8, G=32, n_it=3, bits=2):
    g = K.geom(1, H, T, G, n_it, bits=bits)
    sig = synth.sign_vector(0)
    log(f"prefill workload: {layers} layers x B=1 x T={T} x Hkv={H}, G={G}, iters={n_it}")
    ks, vs, caches = [], [], []
    for l in range(layers):
        k, v = synth.kv_device(synth.sub_seed(2, l, 0), 1, T, H)
        ks.append(k)
        vs.append(v)
        caches.append(K.alloc_cache(g, sig))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for l in range(layers):
            K.kvarn_quantize_prefill(g, caches[l], ks[l], vs[l], T, stream)
    torch.cuda.synchronize()
    # per-launch kernel time: every launch bracketed by HIP events on its stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps * layers)]
    i = 0
    for _ in range(steps):
        for l in range(layers):
            ev[i][0].record(stream)
            K.kvarn_quantize_prefill(g, caches[l], ks[l], vs[l], T, stream)
            ev[i][1].record(stream)
            i += 1
    torch.cuda.synchronize()
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    # the timed step: issued eagerly, one C-ABI call per layer, nothing between the launches
    t0 = time.perf_counter()
    for _ in range(steps):
        for l in range(layers):
            K.kvarn_quantize_prefill(g, caches[l], ks[l], vs[l], T, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same step as one HIP graph of its layer launches, replayed
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(layers):
            K.kvarn_quantize_prefill(g, caches[l], ks[l], vs[l], T)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_wall = time.perf_counter() - t0
    del graph
    bytes_in = 2 * 2 * T * H * 128                       # K and V, bf16
    bytes_out = 2 * H * (T // G) * record_bytes(G, bits)  # tile records
    flags = K.kvarn_cache_flags(caches[0])
    del ks, vs, caches
    torch.cuda.empty_cache()
    return dict(wall=wall, graph_wall=graph_wall, launch_ms=launch_ms, bytes_in=bytes_in, bytes_out=bytes_out,
                layers=layers, T=T, H=H, G=G, n_it=n_it, flags=flags)


def bench_decode(K, synth, torch, steps, warmup=4, layers=40, B=32, H=10, Hq=40, T0=16384, cap=17408, G=32,
                 n_it=3, pool=128, bits=2, kv_kw=None):
    g = K.geom(B, H, cap, G, n_it, bits=bits)
    sig = synth.sign_vector(0)
    kv_kw = kv_kw or {}
    log(f"decode workload: {layers} layers x B={B} x Hkv={H} x Hq={Hq}, {T0} prior tokens, {steps} timed steps")
    k0, v0 = synth.kv_device(synth.sub_seed(4, 0, 0), B, T0, H, **kv_kw)
    caches = []
    for l in range(layers):
        c = K.alloc_cache(g, sig)
        K.kvarn_quantize_prefill(g, c, k0, v0, T0)
        caches.append(c)
    del k0, v0
    kp, vp = synth.kv_device(synth.sub_seed(4, 0, 1), B, pool, H, **kv_kw)  # [B][pool][H][D]
    kp = kp.transpose(0, 1).contiguous()                              # [pool][B][H][D]
    vp = vp.transpose(0, 1).contiguous()
    qp = torch.stack([synth.q_device(synth.sub_seed(4, 0, 2, s), B, Hq) for s in range(pool)])
    ws, nws = K.alloc_workspace(g, Hq)
    out = torch.empty(B, Hq, 128, device="cuda")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(s, ev=None):
        for l in range(layers):
            K.kvarn_append_decode(g, caches[l], kp[s % pool], vp[s % pool], stream)
            if ev is not None:
                ev[0].record(stream)
            K.kvarn_attn_decode(g, caches[l], qp[s % pool], Hq, 0.0, 0, ws, nws, out, stream)
            if ev is not None:
                ev[1].record(stream)

    sc = 0  # decode steps issued so far (every step appends one token to every sequence)
    for _ in range(warmup):
        step(sc)
        sc += 1
    torch.cuda.synchronize()
    ctx_start = T0 + sc
    t0 = time.perf_counter()
    for _ in range(steps):  # the timed steps: nothing but the library calls
        step(sc)
        sc += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the attention call of the last layer of each of 8 further steps, bracketed by events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(8)]
    ctx_attn = T0 + sc + 4  # context of the middle one
    for i in range(8):
        step(sc, evs[i])
        sc += 1
    torch.cuda.synchronize()
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    # one append launch per layer-step, timed the same way
    ea = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
    for e0, e1 in ea:
        e0.record(stream)
        K.kvarn_append_decode(g, caches[0], kp[sc % pool], vp[sc % pool], stream)
        e1.record(stream)
        for l in range(1, layers):
            K.kvarn_append_decode(g, caches[l], kp[sc % pool], vp[sc % pool], stream)
        for l in range(layers):
            K.kvarn_attn_decode(g, caches[l], qp[sc % pool], Hq, 0.0, 0, ws, nws, out, stream)
        sc += 1
    torch.cuda.synchronize()
    append_ms = [a.elapsed_time(b) for a, b in ea]
    # the same step as one HIP graph: 40 x (append + attention) replayed, the step's inputs
    # copied into the captured buffers first (inside the timed region)
    k_in, v_in, q_in = torch.empty_like(kp[0]), torch.empty_like(vp[0]), torch.empty_like(qp[0])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(layers):
            K.kvarn_append_decode(g, caches[l], k_in, v_in)
            K.kvarn_attn_decode(g, caches[l], q_in, Hq, 0.0, 0, ws, nws, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        k_in.copy_(kp[sc % pool])
        v_in.copy_(vp[sc % pool])
        q_in.copy_(qp[sc % pool])
        graph.replay()
        sc += 1
    torch.cuda.synchronize()
    graph_wall = time.perf_counter() - t0
    del graph
    # the fused step (kvarn_append_attn_decode: the append runs in the merge launch), eager
    # and as a graph, over the same shapes
    def fstep(s, kk, vv, qq):
        for l in range(layers):
            K.kvarn_append_attn_decode(g, caches[l], kk, vv, qq, Hq, 0.0, 0, ws, nws, out, stream)

    for _ in range(2):
        fstep(sc, kp[sc % pool], vp[sc % pool], qp[sc % pool])
        sc += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fstep(sc, kp[sc % pool], vp[sc % pool], qp[sc % pool])
        sc += 1
    torch.cuda.synchronize()
    fused_wall = time.perf_counter() - t0
    fgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(fgraph):
        for l in range(layers):
            K.kvarn_append_attn_decode(g, caches[l], k_in, v_in, q_in, Hq, 0.0, 0, ws, nws, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        k_in.copy_(kp[sc % pool])
        v_in.copy_(vp[sc % pool])
        q_in.copy_(qp[sc % pool])
        fgraph.replay()
        sc += 1
    torch.cuda.synchronize()
    fused_graph_wall = time.perf_counter() - t0
    del fgraph
    assert T0 + sc <= cap, "the decode workload outgrew its capacity"
    flags = K.kvarn_cache_flags(caches[0])
    # attention bytes per call at the event-timed context: K and V records of the full
    # tiles + tail rows + q + out
    nfull = ctx_attn // G
    attn_bytes = B * H * (2 * nfull * record_bytes(G, bits) + 2 * (ctx_attn % G) * 256) + B * Hq * (256 + 512)
    del caches
    torch.cuda.empty_cache()
    return dict(wall=wall, steps=steps, B=B, layers=layers, attn_ms=attn_ms, attn_bytes=attn_bytes, flags=flags,
                ctx_start=ctx_start, H=H, Hq=Hq, graph_wall=graph_wall, append_ms=append_ms, fused_wall=fused_wall,
                fused_graph_wall=fused_graph_wall)


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
        "dequantize": {"kernel": "dequant_kernel (bf16 out)", "avg_launch_us": round(dq_avg * 1e3, 2),
                       "bytes_per_launch": bytes_rec + bytes_in, "achieved": round(dq_gbs, 1),
                       "frac": round(dq_gbs / HBM_PEAK_GBS, 4), "unit": "GB/s"},
        "flags": flags,
    }


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


def cpu_baseline(synth, tokens, layers):
    """The oracle's prefill on the first `layers` layers of the prefill workload (host cores)."""
    from oracle import kvarn_ref as R
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    H, G = 8, 32
    dt = 0.0
    for l in range(layers):
        k, v = synth.kv_host(synth.sub_seed(2, l, 0), 1, tokens, H)
        c = R.Cache(R.Geom(1, H, 128, tokens, G, 3, 2), synth.sign_vector(0))
        t0 = time.perf_counter()
        R.quantize_prefill(c, k, v, tokens)
        dt += time.perf_counter() - t0
    gbs = layers * 2 * 2 * tokens * H * 128 / dt / 1e9
    return dict(value=round(gbs, 5), unit="GB/s", cores=int(blas), kind="oracle",
                sample=f"layers 0..{layers - 1} of the prefill workload, {tokens} tokens x 8 KV heads x K and V "
                       f"each ({layers * 2 * H * tokens // G} tiles), {dt:.1f} s of oracle time; NumPy fp64, "
                       "BLAS threads = cores")


def cpu_baseline_decode(synth, T=16384, H=10, Hq=40, layers=40):
    """The oracle's decode step (append + attention, by definition over the dequantized
    cache) on one batch row of the Phi-4-shaped decode, extrapolated to the full step."""
    from oracle import kvarn_ref as R
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    G = 32
    c = R.Cache(R.Geom(1, H, 128, T + 2 * G, G, 3, 2), synth.sign_vector(0))
    k, v = synth.kv_host(synth.sub_seed(4, 0, 0), 1, T, H)
    R.quantize_prefill(c, k, v, T)                      # set-up, not timed
    kn, vn = synth.kv_host(synth.sub_seed(4, 0, 1), 1, 1, H)
    q = synth.q_host(synth.sub_seed(4, 0, 2), 1, Hq)
    t0 = time.perf_counter()
    R.append_decode(c, kn[:, 0], vn[:, 0])
    R.attn_decode(c, q, Hq)
    dt = time.perf_counter() - t0
    # a step of B rows costs B times one row per layer and yields B tokens
    return dict(value=round(1.0 / (dt * layers), 6), unit="tokens/s", cores=int(blas), kind="oracle",
                sample=f"one batch row of the decode workload ({H} KV heads x {Hq} query heads, {T}-token "
                       f"context): one append + attention step, {dt:.1f} s of oracle time, extrapolated "
                       f"to {layers} layers; NumPy fp64, BLAS threads = cores")


# HBM traffic of a kernel from committed rocprofv3 counter summaries: FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch) scaled by what the same counters read for a 4 GiB device
# copy. The figures stand only while the kernel sources hash to the digest recorded
# with them; otherwise traffic is reported as null.
KERNEL_SOURCES = ["kv_cache_bit_amd/csrc/kvarn_common.h", "kv_cache_bit_amd/csrc/kvarn_launch.h"]
PREFILL_SOURCES = ["kv_cache_bit_amd/csrc/quantize.hip", "kv_cache_bit_amd/csrc/quantize_dev.h"]
ATTN_SOURCES = ["kv_cache_bit_amd/csrc/attn.hip", "kv_cache_bit_amd/csrc/quantize_dev.h"]


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
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=32)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-reasoning decode (64 x 32768-token contexts, Llama-3.1-8B KV geometry)")
    ap.add_argument("--no-roundtrip", action="store_true",
                    help="skip the Qwen3-4B-shaped prefill + dequantize round trip")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--cpu-layers", type=int, default=5, help="layers of the prefill workload the oracle runs")
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
    pf = bench_prefill(K, synth, torch, args.steps, args.warmup, bits=args.bits)
    ms_step = pf["wall"] * 1e3 / args.steps
    value = pf["layers"] * pf["bytes_in"] / (ms_step * 1e-3) / 1e9
    total_gbs = pf["layers"] * (pf["bytes_in"] + pf["bytes_out"]) / (ms_step * 1e-3) / 1e9
    lm = sorted(pf["launch_ms"])
    avg_launch = sum(lm) / len(lm)
    achieved = (pf["bytes_in"] + pf["bytes_out"]) / (avg_launch * 1e-3) / 1e9
    graph_ms = pf["graph_wall"] * 1e3 / args.steps
    log(f"prefill: {ms_step:.3f} ms/step ({graph_ms:.3f} as a graph), {value:.1f} GB/s bf16-in, "
        f"{total_gbs:.1f} GB/s total; kernel avg {avg_launch * 1e3:.1f} us -> {achieved:.1f} GB/s")
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "llama3.1-8b-shaped KV prefill quantize", "layers": pf["layers"], "batch": 1,
                   "tokens": pf["T"], "kv_heads": pf["H"], "head_dim": 128, "group": pf["G"],
                   "varn_iters": pf["n_it"], "bits": args.bits,
                   "input": "bf16, outlier channels x20, 5% lognormal tokens"},
        "hbm_frac_step": round(total_gbs / HBM_PEAK_GBS, 4),
        "step_as_graph": {"ms_per_step": round(graph_ms, 4),
                          "value": round(pf["layers"] * pf["bytes_in"] / (graph_ms * 1e-3) / 1e9, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (counted_traffic("prefill_kernel_llama8b_32k_pmc.txt", PREFILL_SOURCES)
                                 if args.bits == 2 else None),
                     "traffic_unit": "bytes/launch",
                     "kernel": "prefill_kernel<1,false,false,1>" if args.bits == 2 else "prefill_kernel<1,false,true,1>", "bytes_per_launch": pf["bytes_in"] + pf["bytes_out"],
                     "avg_launch_us": round(avg_launch * 1e3, 2), "median_launch_us": round(lm[len(lm) // 2] * 1e3, 2)},
        "flags": pf["flags"],
    }
    if not args.no_copy:
        res["copy_ceiling"] = copy_ceiling(torch)
        log(f"copy ceiling: {res['copy_ceiling']}")
    if not args.no_decode:
        dc = bench_decode(K, synth, torch, args.decode_steps, bits=args.bits)
        tok_s = dc["B"] * dc["steps"] / dc["wall"]
        am = sorted(dc["attn_ms"])
        a_avg = sum(am) / len(am)
        res["decode"] = {
            "workload": "phi-4-14b-shaped decode: append + attn_decode", "tokens_per_s": round(tok_s, 1),
            "ms_per_step": round(dc["wall"] * 1e3 / dc["steps"], 3), "steps_timed": dc["steps"],
            "layers": dc["layers"], "batch": dc["B"], "kv_heads": dc["H"], "q_heads": dc["Hq"],
            "context_at_start": dc["ctx_start"], "attn_avg_us": round(a_avg * 1e3, 2),
            "attn_GBps": round(dc["attn_bytes"] / (a_avg * 1e-3) / 1e9, 1),
            "attn_frac": round(dc["attn_bytes"] / (a_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "flags": dc["flags"],
            "roofline": {"bound": "hbm", "kernel": f"attn_kernel<32, {args.bits}> + merge_kernel",
                         "achieved": round(dc["attn_bytes"] / (a_avg * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(dc["attn_bytes"] / (a_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": dc["attn_bytes"],
                         "traffic": (counted_traffic("attn_kernel_phi4_decode_pmc.txt", ATTN_SOURCES)
                                     if args.bits == 2 else None),
                         "traffic_unit": "bytes/launch (tile pass)"}}
        ap = sorted(dc["append_ms"])
        res["decode"]["graph_tokens_per_s"] = round(dc["B"] * dc["steps"] / dc["graph_wall"], 1)
        res["decode"]["graph_ms_per_step"] = round(dc["graph_wall"] * 1e3 / dc["steps"], 3)
        res["decode"]["append_us"] = round(ap[len(ap) // 2] * 1e3, 2)
        res["decode"]["fused_tokens_per_s"] = round(dc["B"] * dc["steps"] / dc["fused_wall"], 1)
        res["decode"]["fused_graph_tokens_per_s"] = round(dc["B"] * dc["steps"] / dc["fused_graph_wall"], 1)
        res["decode"]["append_share"] = round(ap[len(ap) // 2] / (ap[len(ap) // 2] + a_avg), 4)
        log(f"decode: {tok_s:.1f} tok/s eager, {res['decode']['graph_tokens_per_s']} tok/s as a graph; "
            f"attn {a_avg * 1e3:.1f} us, append {res['decode']['append_us']} us per layer-step")
        log(f"fused step: {res['decode']['fused_tokens_per_s']} tok/s eager, "
            f"{res['decode']['fused_graph_tokens_per_s']} tok/s as a graph")
        if not args.no_bf16:
            bf = bench_bf16_decode(torch)
            res["decode"]["bf16_baseline"] = dict(bf, kind="plain bf16 KV cache, torch batched products, same shapes")
            best = max(res["decode"]["graph_tokens_per_s"], res["decode"]["fused_graph_tokens_per_s"])
            res["decode"]["speedup_vs_bf16"] = round(best / bf["tokens_per_s"], 2)
            log(f"bf16 baseline: {bf}")
    if not args.no_long:
        torch.cuda.empty_cache()
        lg = bench_decode(K, synth, torch, 8, warmup=2, layers=32, B=64, H=8, Hq=32, T0=32768, cap=36864,
                          bits=args.bits, kv_kw=dict(law="student_t", nu=3.0, n_outlier_ch=8, ch_mult=30.0))
        lam = sorted(lg["attn_ms"])
        la_avg = sum(lam) / len(lam)
        res["long_decode"] = {
            "workload": "long-reasoning stress decode: llama3.1-8b KV geometry, 64 x 32768-token contexts",
            "layers": lg["layers"], "batch": lg["B"], "kv_heads": lg["H"], "q_heads": lg["Hq"],
            "context_at_start": lg["ctx_start"], "input": "bf16, Student-t (nu 3) token norms, 8 outlier channels x30",
            "tokens_per_s": round(lg["B"] * lg["steps"] / lg["wall"], 1),
            "ms_per_step": round(lg["wall"] * 1e3 / lg["steps"], 3), "steps_timed": lg["steps"],
            "fused_tokens_per_s": round(lg["B"] * lg["steps"] / lg["fused_wall"], 1),
            "attn_avg_us": round(la_avg * 1e3, 2),
            "attn_GBps": round(lg["attn_bytes"] / (la_avg * 1e-3) / 1e9, 1),
            "attn_frac": round(lg["attn_bytes"] / (la_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "flags": lg["flags"]}
        log(f"long decode: {res['long_decode']['tokens_per_s']} tok/s eager, "
            f"{res['long_decode']['fused_tokens_per_s']} fused; attn {res['long_decode']['attn_avg_us']} us "
            f"({res['long_decode']['attn_GBps']} GB/s) per layer-step")
    if not args.no_roundtrip:
        rt = bench_roundtrip(K, synth, torch, max(1, args.steps // 3), bits=args.bits)
        res["roundtrip"] = rt
        log(f"round trip: {rt['ms_per_step']} ms/step; prefill {rt['prefill']['avg_launch_us']} us "
            f"({rt['prefill']['achieved']} GB/s), dequantize {rt['dequantize']['avg_launch_us']} us "
            f"({rt['dequantize']['achieved']} GB/s) per layer")
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(synth, args.cpu_tokens, args.cpu_layers)
        if "decode" in res:
            log("cpu baseline, decode step (oracle) ...")
            res["decode"]["cpu_baseline"] = cpu_baseline_decode(synth)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
