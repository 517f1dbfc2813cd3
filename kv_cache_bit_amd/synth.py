"""Seeded synthetic inputs for the KVarN quantizer: K/V tensors, queries, sign vectors.

This module only draws random numbers and casts them to bf16 bit patterns. It
holds none of the quantizer's arithmetic, so both the HIP path (through the
binding) and the CPU oracle can take their inputs from it.

Where the values come from (KVarN pages, as extracted text):
  * channel outliers that a Hadamard rotation spreads out -- ai-paper-analysis
    page, section 3.1; friday-blog page, section 2;
  * a few tokens with outlying norms that stretch a shared scale -- researchpapers
    page, "where the drift comes from"; ai-paper-analysis page, sections 1-2;
  * long reasoning contexts (32K tokens) -- ai-paper-analysis page, section 1.

The model of one K or V stream is x[t, j] = Z[t, j] * a[j] * m[t] with Z ~ N(0, 1)
i.i.d.; a[j] = A on n_c channels chosen without replacement (fixed across tokens),
1 elsewhere; m[t] the token multiplier, drawn once per (batch, token) and shared
by every head and by K and V. Values are rounded to bf16 with round-half-to-even.

Sign vectors are drawn with SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014): sigma[j] = 1 - 2 * (z_j >> 63),
z_j the j-th output of the generator seeded with `seed`.
"""
from __future__ import annotations

import numpy as np

_MASK64 = (1 << 64) - 1


def splitmix64(seed: int, n: int) -> list[int]:
    """First n outputs of SplitMix64 started from `seed` (published constants)."""
    state = seed & _MASK64
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def sign_vector(seed: int, d: int = 128) -> np.ndarray:
    """Random +-1 signs (int8[d]) for the randomized Hadamard matrix."""
    return np.array([1 - 2 * (z >> 63) for z in splitmix64(seed, d)], dtype=np.int8)


def sub_seed(*parts: int) -> int:
    """Derive an independent 63-bit seed from integer parts (config, layer, purpose ...)."""
    s = 0x1234_5678_9ABC_DEF0
    for p in parts:
        s = splitmix64((s ^ (p & _MASK64)) & _MASK64, 1)[0]
    return s & ((1 << 63) - 1)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-half-to-even) and return the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = ((b >> 16) & 1) + 0x7FFF
    return ((b + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- host draws
def token_multipliers(rng: np.random.Generator, n: int, law: str, **kw) -> np.ndarray:
    """Per-token norm multipliers m[t] for one of the outlier-token laws."""
    if law == "lognormal":  # fraction p of tokens get exp(sigma * N(0,1))
        p, sigma = kw.get("p", 0.05), kw.get("sigma", 1.5)
        m = np.ones(n)
        sel = rng.random(n) < p
        m[sel] = np.exp(sigma * rng.standard_normal(int(sel.sum())))
        return m
    if law == "spike":  # fraction p of tokens multiplied by a fixed factor
        p, factor = kw.get("p", 0.02), kw.get("factor", 50.0)
        m = np.ones(n)
        m[rng.random(n) < p] = factor
        return m
    if law == "student_t":  # |Student-t(nu)| norm scale, heavy tailed
        return np.abs(rng.standard_t(kw.get("nu", 3.0), size=n))
    if law == "none":
        return np.ones(n)
    raise ValueError(law)


def kv_host(seed: int, batch: int, tokens: int, kv_heads: int, head_dim: int = 128,
            n_outlier_ch: int = 4, ch_mult: float = 20.0, law: str = "lognormal",
            **law_kw) -> tuple[np.ndarray, np.ndarray]:
    """K and V as bf16 bit patterns, uint16[batch][tokens][kv_heads][head_dim].

    Small sizes only (host NumPy, PCG64); large workloads use `kv_device`.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    m = np.stack([token_multipliers(rng, tokens, law, **law_kw) for _ in range(batch)])  # [B][T]
    out = []
    for _stream in range(2):
        a = np.ones((kv_heads, head_dim))
        for h in range(kv_heads):
            a[h, rng.choice(head_dim, size=n_outlier_ch, replace=False)] = ch_mult
        z = rng.standard_normal((batch, tokens, kv_heads, head_dim))
        x = z * a[None, None] * m[:, :, None, None]
        out.append(f32_to_bf16_bits(x.astype(np.float32)))
    return out[0], out[1]


def q_host(seed: int, batch: int, q_heads: int, head_dim: int = 128) -> np.ndarray:
    """Queries ~ N(0, 1) as bf16 bit patterns, uint16[batch][q_heads][head_dim]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits(rng.standard_normal((batch, q_heads, head_dim)).astype(np.float32))


# --------------------------------------------------------------------------- device draws
def kv_device(seed: int, batch: int, tokens: int, kv_heads: int, head_dim: int = 128,
              n_outlier_ch: int = 4, ch_mult: float = 20.0, law: str = "lognormal",
              device="cuda", **law_kw):
    """Same law as `kv_host`, drawn with a torch.Generator on `device`; returns bf16 tensors.

    Used for the full-size workloads, where host generation would dominate the run.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = dict(device=device, dtype=torch.float32)
    if law == "lognormal":
        p, sigma = law_kw.get("p", 0.05), law_kw.get("sigma", 1.5)
        sel = torch.rand(batch, tokens, generator=g, **f32) < p
        m = torch.where(sel, torch.exp(sigma * torch.randn(batch, tokens, generator=g, **f32)),
                        torch.ones(batch, tokens, **f32))
    elif law == "spike":
        p, factor = law_kw.get("p", 0.02), law_kw.get("factor", 50.0)
        sel = torch.rand(batch, tokens, generator=g, **f32) < p
        m = torch.where(sel, torch.full((batch, tokens), factor, **f32), torch.ones(batch, tokens, **f32))
    elif law == "student_t":
        nu = law_kw.get("nu", 3.0)
        zt = torch.randn(batch, tokens, generator=g, **f32)
        # chi-square(nu) as a sum of nu squared normals (nu is a small integer here)
        chi = sum(torch.randn(batch, tokens, generator=g, **f32) ** 2 for _ in range(int(nu)))
        m = (zt / torch.sqrt(chi / nu)).abs()
    elif law == "none":
        m = torch.ones(batch, tokens, **f32)
    else:
        raise ValueError(law)
    out = []
    for _stream in range(2):
        a = torch.ones(kv_heads, head_dim, **f32)
        for h in range(kv_heads):
            idx = torch.randperm(head_dim, generator=g, device=device)[:n_outlier_ch]
            a[h, idx] = ch_mult
        x = torch.empty(batch, tokens, kv_heads, head_dim, dtype=torch.bfloat16, device=device)
        for b in range(batch):  # one batch row at a time keeps the fp32 temporary small
            z = torch.randn(tokens, kv_heads, head_dim, generator=g, **f32)
            x[b] = (z * a[None] * m[b][:, None, None]).to(torch.bfloat16)
        out.append(x)
    return out[0], out[1]


def q_device(seed: int, batch: int, q_heads: int, head_dim: int = 128, device="cuda"):
    """Queries ~ N(0, 1) as a bf16 tensor [batch][q_heads][head_dim] on `device`."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(batch, q_heads, head_dim, generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)
