"""Synthetic pseudo-decode: how the 2-bit cache's error builds up over a long decode.

The ai-paper-analysis page (section 4, pseudo-decode evaluation) replays a written answer
token by token on a model whose KV cache is quantized, so every step reads keys and values
that earlier steps wrote through the quantizer, and compares each step's output
distribution with the full-precision run; evaluating with one parallel prefill instead
hides the build-up (section 4, figure 4). The researchpapers and friday-blog pages make
the same point about long reasoning traces.

Without trained weights this module builds the same experiment on a random decoder:

  * L layers, each h <- h + attn(q, K, V) W_o with q = rms(h) W_q s_q, k = rms(h) W_k,
    v = rms(h) W_v (pre-norm; with kv_prenorm=False k and v come from h itself, so the
    inputs' token norms reach the cache and the largest tokens take all the attention),
    W ~ N(0, 1/fan_in), a few K and V channels per head scaled by `ch_mult` (the channel
    outliers of the ai-paper-analysis page, section 3.1);
  * teacher-forced inputs h0_t = m_t z_t, z_t ~ N(0, I), m_t the lognormal outlier-token
    law of the synthetic K/V generator (a fraction p of tokens with norm exp(sigma N));
  * a readout logits = rms(h_L) W_u (vocabulary V, W_u ~ N(0, tau^2 / d)).

Three runs share the inputs: the reference keeps K and V exactly (the bf16 values, read
in fp32); "pseudo-decode" appends its own k, v to libkvarn caches (kvarn_append_decode)
and attends over them (kvarn_attn_decode), so quantization error in one layer's output
reaches the keys and values later steps read; "parallel" appends the reference's k, v to
libkvarn caches and attends with its own query, which is the error a one-shot evaluation
sees. Per step it records the KL divergence of the readout distribution from the
reference, top-1 agreement, and the relative error of the last layer's attention output.
Each ablation variant (section 5) runs beside the full method in the same loop.

A second experiment (--pairwise) measures how quantization moves the attention-score gap
between an outlier-norm token and a normal token of the same tile, split into the error's
magnitude and direction parts (section 2, figure 1).

Usage: python -m kv_cache_bit_amd.pseudo_decode [--steps 4096] [--json out.json]
       python -m kv_cache_bit_amd.pseudo_decode --pairwise
"""
from __future__ import annotations

import argparse
import json
import math
import time

import torch

from . import kvarn as K
from . import synth

# name -> (varn_iters, variant bits)
VARIANTS = {
    "kvarn": (3, 0),
    "hadamard_only": (0, 0),
    "varn_only": (3, K.KVARN_VARIANT_NO_ROTATION),
    "token_axis_only": (3, K.KVARN_VARIANT_NO_CHANNEL_PASS),
    "channel_axis_only": (3, K.KVARN_VARIANT_NO_TOKEN_PASS),
}


def rms_norm(x: torch.Tensor) -> torch.Tensor:
    return x * torch.rsqrt(torch.mean(x * x, dim=-1, keepdim=True) + 1e-6)


class RandomDecoder:
    """Weights of the random decoder, fp32 on the device."""

    def __init__(self, seed, layers, hq, hkv, d_head=128, vocab=4096, ch_outliers=4, ch_mult=20.0,
                 q_scale=0.25, tau=3.0, kv_prenorm=True, device="cuda"):
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        self.L, self.hq, self.hkv, self.D = layers, hq, hkv, d_head
        self.kv_prenorm = kv_prenorm
        self.d = hq * d_head
        f32 = dict(device=device, dtype=torch.float32)
        d, nq, nk = self.d, hq * d_head, hkv * d_head
        self.w_qkv, self.w_o = [], []
        for _ in range(layers):
            wq = torch.randn(d, nq, generator=g, **f32) * (q_scale / math.sqrt(d))
            wk = torch.randn(d, nk, generator=g, **f32) / math.sqrt(d)
            wv = torch.randn(d, nk, generator=g, **f32) / math.sqrt(d)
            for w in (wk, wv):
                for h in range(hkv):
                    idx = torch.randperm(d_head, generator=g, device=device)[:ch_outliers]
                    w[:, h * d_head + idx] *= ch_mult
            self.w_qkv.append(torch.cat([wq, wk, wv], dim=1).contiguous())
            self.w_o.append((torch.randn(nq, d, generator=g, **f32) / math.sqrt(nq)).contiguous())
        self.w_u = (torch.randn(d, vocab, generator=g, **f32) * (tau / math.sqrt(d))).contiguous()

    def qkv(self, l, h):
        """bf16 q [B][Hq][D], k and v [B][Hkv][D] (contiguous) for hidden states h [B][d]."""
        B = h.shape[0]
        nq, nk = self.hq * self.D, self.hkv * self.D
        q = rms_norm(h) @ self.w_qkv[l][:, :nq]
        kv = (rms_norm(h) if self.kv_prenorm else h) @ self.w_qkv[l][:, nq:]
        return (q.to(torch.bfloat16).view(B, self.hq, self.D).contiguous(),
                kv[:, :nk].to(torch.bfloat16).view(B, self.hkv, self.D).contiguous(),
                kv[:, nk:].to(torch.bfloat16).view(B, self.hkv, self.D).contiguous())

    def logp(self, h):
        return torch.log_softmax(rms_norm(h) @ self.w_u, dim=-1)


def inputs(seed, B, T, d, p=0.05, sigma=1.5, device="cuda"):
    """Teacher-forced inputs h0 [B][T][d]: N(0, I) rows times the outlier-token multiplier."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = dict(device=device, dtype=torch.float32)
    sel = torch.rand(B, T, generator=g, **f32) < p
    m = torch.where(sel, torch.exp(sigma * torch.randn(B, T, generator=g, **f32)), torch.ones(B, T, **f32))
    return torch.randn(B, T, d, generator=g, **f32) * m[..., None]


class ExactCache:
    """The reference's K and V in fp32 (from the same bf16 values), K stored as [D][T]."""

    def __init__(self, B, hkv, D, T, device="cuda"):
        self.kt = torch.zeros(B, hkv, D, T, device=device)
        self.v = torch.zeros(B, hkv, T, D, device=device)

    def append_attend(self, t, q, k, v, grp):
        self.kt[:, :, :, t] = k.float()
        self.v[:, :, t] = v.float()
        B, hq, D = q.shape
        qf = q.float().view(B, hq // grp, grp, D)
        s = torch.matmul(qf, self.kt[:, :, :, :t + 1]) * (1.0 / math.sqrt(D))
        p = torch.softmax(s, dim=-1)
        self.pmax = p.amax(dim=-1).mean()  # how concentrated the attention is
        return torch.matmul(p, self.v[:, :, :t + 1]).view(B, hq, D)


def run(steps=4096, B=4, layers=4, hq=32, hkv=8, group=32, seed=0, variants=None, log_every=512,
        q_scale=0.25, kv_prenorm=True, device="cuda"):
    variants = variants or list(VARIANTS)
    torch.manual_seed(seed)
    model = RandomDecoder(seed, layers, hq, hkv, q_scale=q_scale, kv_prenorm=kv_prenorm, device=device)
    h0 = inputs(seed + 1, B, steps, model.d, device=device)
    cap = (steps + group - 1) // group * group
    grp = hq // hkv
    sigma = synth.sign_vector(seed + 2, 128)

    ref = [ExactCache(B, hkv, 128, cap, device) for _ in range(layers)]
    runs = {}
    for name in variants:
        n_it, var = VARIANTS[name]
        g = K.geom(B, hkv, cap, group, n_it, variant=var)
        ws, nws = K.alloc_workspace(g, hq, device)
        runs[name] = dict(
            g=g, ws=ws, nws=nws,
            pd=[K.alloc_cache(g, sigma, device) for _ in range(layers)],
            par=[K.alloc_cache(g, sigma, device) for _ in range(layers)],
            out=torch.empty(B, hq, 128, device=device),
            stats={m: torch.zeros(steps, device=device) for m in
                   ("pd_kl", "pd_top1", "pd_attn", "par_kl", "par_top1", "par_attn")})

    def rel(a, b):  # per (b, head) relative L2 error, averaged
        return (torch.linalg.vector_norm(a - b, dim=-1) /
                torch.linalg.vector_norm(b, dim=-1).clamp_min(1e-30)).mean()

    ref_pmax = torch.zeros(steps, device=device)
    t0 = time.perf_counter()
    for t in range(steps):
        # reference
        h = h0[:, t].clone()
        kv_ref = []
        for l in range(layers):
            q, k, v = model.qkv(l, h)
            kv_ref.append((k, v))
            o_ref = ref[l].append_attend(t, q, k, v, grp)
            h = h + o_ref.reshape(B, -1) @ model.w_o[l]
        lp_ref = model.logp(h)
        top_ref = lp_ref.argmax(-1)
        ref_pmax[t] = ref[-1].pmax
        for name in variants:
            r = runs[name]
            for mode in ("pd", "par"):
                hx = h0[:, t].clone()
                for l in range(layers):
                    q, k, v = model.qkv(l, hx)
                    if mode == "par":
                        k, v = kv_ref[l]
                    c = r[mode][l]
                    K.kvarn_append_decode(r["g"], c, k, v)
                    K.kvarn_attn_decode(r["g"], c, q, hq, 0.0, 0, r["ws"], r["nws"], r["out"])
                    hx = hx + r["out"].reshape(B, -1) @ model.w_o[l]
                lp = model.logp(hx)
                st = r["stats"]
                st[mode + "_kl"][t] = torch.sum(lp_ref.exp() * (lp_ref - lp), dim=-1).mean()
                st[mode + "_top1"][t] = (lp.argmax(-1) == top_ref).float().mean()
                st[mode + "_attn"][t] = rel(r["out"], o_ref)
        if log_every and (t + 1) % log_every == 0:
            torch.cuda.synchronize()
            print(f"[pseudo-decode] step {t + 1}/{steps} ({time.perf_counter() - t0:.1f} s)", flush=True)
    torch.cuda.synchronize()
    stats = {name: {k: v.cpu().numpy() for k, v in runs[name]["stats"].items()} for name in variants}
    return stats, dict(steps=steps, B=B, layers=layers, hq=hq, hkv=hkv, group=group, seed=seed, q_scale=q_scale,
                       kv_prenorm=kv_prenorm, ref_pmax=ref_pmax.cpu().numpy())


def windows(steps, group):
    edges = [0, group, 256, 1024, 2048, 4096, 8192, 16384]
    edges = [e for e in edges if e < steps] + [steps]
    return list(zip(edges[:-1], edges[1:]))


def summarize(stats, cfg):
    wins = windows(cfg["steps"], cfg["group"])
    out = {}
    for name, st in stats.items():
        out[name] = {m: [float(st[m][a:b].mean()) for a, b in wins] for m in st}
    out["reference"] = {"ref_pmax": [float(cfg["ref_pmax"][a:b].mean()) for a, b in wins]}
    return wins, out


def table(wins, summ, metric):
    head = "| variant | " + " | ".join(f"steps {a}-{b - 1}" for a, b in wins) + " |"
    lines = [head, "|" + "---|" * (len(wins) + 1)]
    for name, m in summ.items():
        if metric not in m:
            continue
        lines.append(f"| {name} | " + " | ".join(f"{x:.3g}" for x in m[metric]) + " |")
    return "\n".join(lines)


# ----------------------------------------------------------------------------- pairwise token error
def error_split(x, xh):
    """Magnitude and direction parts of eps = xh - x per row (ai-paper-analysis page,
    section 2, error equation): E_M = (|xh| - |x|) x/|x|, E_D = |xh| (xh/|xh| - x/|x|)."""
    nx = torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)
    nxh = torch.linalg.vector_norm(xh, dim=-1, keepdim=True)
    ux = x / nx
    uxh = xh / nxh.clamp_min(1e-30)
    return (nxh - nx) * ux, nxh * (uxh - ux)


def pairwise(ratios=(1, 2, 4, 8, 16, 32, 64), tiles=512, group=32, seed=0, n_queries=64,
             variants=("kvarn", "hadamard_only", "varn_only"), device="cuda"):
    """Attention-score error of token pairs (ai-paper-analysis page, section 2, figure 1):
    in every tile of G tokens the first token's norm is `ratio` times the others'. The
    pair (outlier a, normal b) competes through the logit gap l_a - l_b = q.(k_a - k_b)/sqrt(D);
    quantization moves it by q.(eps_a - eps_b)/sqrt(D), split into the magnitude part
    (E_M) and the direction part (E_D). Returns, per variant and ratio, the mean absolute
    gap change of each part over pairs and random queries, and the mean relative error
    of the normal tokens."""
    g_rng = torch.Generator(device=device)
    g_rng.manual_seed(seed)
    f32 = dict(device=device, dtype=torch.float32)
    T = tiles * group
    a = torch.ones(128, **f32)
    a[torch.randperm(128, generator=g_rng, device=device)[:4]] = 20.0   # channel outliers
    z = torch.randn(T, 128, generator=g_rng, **f32)
    q = torch.randn(n_queries, 128, generator=g_rng, **f32)
    sigma = synth.sign_vector(seed + 2, 128)
    out = {}
    for name in variants:
        n_it, var = VARIANTS[name]
        g = K.geom(1, 1, T, group, n_it, variant=var)
        cache = K.alloc_cache(g, sigma, device)
        kh = torch.empty(1, T, 1, 128, **f32)
        vh = torch.empty(1, T, 1, 128, **f32)
        rows = {}
        for ratio in ratios:
            m = torch.ones(T, 1, **f32)
            m[::group] = float(ratio)
            k = (z * a * m).to(torch.bfloat16).view(1, T, 1, 128).contiguous()
            K.kvarn_quantize_prefill(g, cache, k, k, T)
            K.kvarn_dequantize(g, cache, kh, vh, T, K.KVARN_OUT_F32)
            x = k.float().view(tiles, group, 128)
            xh = kh.view(tiles, group, 128)
            e_m, e_d = error_split(x, xh)
            # pair (token 0, token j) of each tile: gap change per query
            dm = (e_m[:, :1] - e_m[:, 1:]) @ q.T / math.sqrt(128)      # [tiles][G-1][nq]
            dd = (e_d[:, :1] - e_d[:, 1:]) @ q.T / math.sqrt(128)
            nrm = torch.linalg.vector_norm(x, dim=-1)
            rel = torch.linalg.vector_norm(xh - x, dim=-1) / nrm
            rel_m = torch.linalg.vector_norm(e_m, dim=-1) / nrm
            rel_d = torch.linalg.vector_norm(e_d, dim=-1) / nrm
            rows[ratio] = dict(gap_change_EM=float(dm.abs().mean()), gap_change_ED=float(dd.abs().mean()),
                               rel_err_normal=float(rel[:, 1:].mean()), rel_err_outlier=float(rel[:, 0].mean()),
                               rel_EM_normal=float(rel_m[:, 1:].mean()), rel_ED_normal=float(rel_d[:, 1:].mean()))
        out[name] = rows
    return out


def pairwise_table(res):
    lines = ["| variant | norm ratio | rel. error, normal tokens (E_M, E_D parts) | rel. error, outlier token | "
             "score-gap change from E_M | from E_D |", "|---|---|---|---|---|---|"]
    for name, rows in res.items():
        for ratio, r in rows.items():
            lines.append(f"| {name} | {ratio} | {r['rel_err_normal']:.3g} ({r['rel_EM_normal']:.3g}, "
                         f"{r['rel_ED_normal']:.3g}) | {r['rel_err_outlier']:.3g} | {r['gap_change_EM']:.3g} | "
                         f"{r['gap_change_ED']:.3g} |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--steps", type=int, default=4096)
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--hq", type=int, default=32)
    ap.add_argument("--hkv", type=int, default=8)
    ap.add_argument("--group", type=int, default=32)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--variants", default=",".join(VARIANTS))
    ap.add_argument("--q-scale", type=float, default=0.25, help="query scale: sets how peaked attention is")
    ap.add_argument("--kv-residual", action="store_true",
                    help="k, v from the raw residual stream h instead of rms(h): token norms reach the cache")
    ap.add_argument("--pairwise", action="store_true", help="run the pairwise token-error experiment instead")
    ap.add_argument("--json", default=None)
    a = ap.parse_args(argv)
    if a.pairwise:
        res = pairwise(group=a.group, seed=a.seed)
        print(pairwise_table(res))
        if a.json:
            with open(a.json, "w") as f:
                json.dump(res, f, indent=1)
        return
    stats, cfg = run(a.steps, a.batch, a.layers, a.hq, a.hkv, a.group, a.seed, a.variants.split(","),
                     q_scale=a.q_scale, kv_prenorm=not a.kv_residual)
    wins, summ = summarize(stats, cfg)
    print(f"config: {dict((k, v) for k, v in cfg.items() if k != 'ref_pmax')}")
    for metric in ("ref_pmax", "pd_kl", "par_kl", "pd_top1", "par_top1", "pd_attn", "par_attn"):
        print(f"\n{metric} (mean over the step window)\n" + table(wins, summ, metric))
    if a.json:
        with open(a.json, "w") as f:
            cfg = {k: v for k, v in cfg.items() if k != "ref_pmax"}
            json.dump(dict(config=cfg, windows=wins, summary=summ), f, indent=1)


if __name__ == "__main__":
    main()
