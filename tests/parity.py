"""Helpers shared by the GPU parity tests: run libkvarn on the GPU, run the oracle on
the same inputs, and compare with the conditional chain:

  W (rotated)            vs oracle rotation, |d| <= 1e-5 (|ref| + rms_row(ref))
  r16, c16               vs oracle VarN: <= 1 fp16 ulp, mismatch fraction <= 1e-2
  Y (normalized)         vs W_ref / (r16_gpu c16_gpu), same form as W
  s16, z16               vs the oracle grid of that Y_ref': <= 1 ulp, fraction <= 1e-2
  codes                  vs oracle codes of Y_ref' with the GPU's s16, z16: identical
                         except where |u - (k + 1/2)| < 1e-4 (either code is correct)
  record bytes, tail     vs the oracle's packing of the GPU's own fields: bit-exact

Stored fp16 values decided by fp32 (GPU) vs fp64 (oracle) arithmetic may land one
ulp apart; the chain re-derives each later quantity from the GPU's stored values
so that one such difference does not cascade.
"""
from __future__ import annotations

import numpy as np
import torch

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth
from oracle import kvarn_ref as R

EDGE_BAND = 1e-4


def to_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def from_u16(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def fp16_ulp_dist(a, b) -> np.ndarray:
    def ordered(x):
        bits = np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16).astype(np.int64)
        mag = bits & 0x7FFF
        return np.where(bits & 0x8000, -mag, mag)
    return np.abs(ordered(a) - ordered(b))


def close_rowwise(got, ref, rel, axis=-1):
    """|got - ref| <= rel (|ref| + rms of ref along the row)."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=axis, keepdims=True))
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    bound = rel * (np.abs(ref) + rms)
    return bool(np.all(err <= bound)), float((err / np.maximum(bound, 1e-300)).max())


class GpuCache:
    """One layer cache in device memory plus host copies for the oracle."""

    def __init__(self, B, H, cap, G=32, n_it=3, seed_sigma=0, variant=0, bits=2):
        self.g = K.geom(B, H, cap, G, n_it, variant=variant, bits=bits)
        self.og = R.Geom(B, H, 128, cap, G, n_it, bits, variant)
        self.sigma = synth.sign_vector(seed_sigma, 128)
        self.buf = K.alloc_cache(self.g, self.sigma)

    def host_cache(self) -> R.Cache:
        c = R.Cache(self.og, self.sigma)
        torch.cuda.synchronize()
        c.buf[:] = self.buf.cpu().numpy()
        return c


def check_prefill(gc: GpuCache, k_bits: np.ndarray, v_bits: np.ndarray, T: int, w=None, y=None,
                  tiles=None) -> dict:
    """Full parity chain for a prefill of T tokens. w, y: GPU debug tensors
    [2][B][T_full][H][D] (or None). tiles: optional list of (b, h, tile) to check
    (default: all). Returns statistics for the report."""
    og = gc.og
    G = og.group
    hc = gc.host_cache()
    stats = dict(edge_exempt=0, codes=0, r_mis=0, c_mis=0, s_mis=0, z_mis=0, n_r=0, n_c=0)
    # header
    assert hc.buf[0:4].view(np.uint32)[0] == R.MAGIC
    assert hc.buf[4:8].view(np.uint32)[0] == R.VERSION
    assert hc.buf[R.NUM_PAGES_OFFSET:R.NUM_PAGES_OFFSET + 4].view(np.int32)[0] == og.num_pages
    assert hc.buf[8:36].view(np.int32).tolist() == list(og.as_tuple())
    assert hc.buf[R.VARIANT_OFFSET:R.VARIANT_OFFSET + 4].view(np.uint32)[0] == og.variant
    assert np.array_equal(hc.sigma, gc.sigma.astype(np.float64))
    sw = hc.buf[R.SIGN_WORDS_OFFSET:R.SIGN_WORDS_OFFSET + 2 * og.head_dim].view(np.uint32)
    assert np.array_equal(sw, R.sign_words(gc.sigma))
    assert np.all(hc.lens == T), hc.lens
    nfull = T // G
    if tiles is None:
        tiles = [(b, h, t) for b in range(og.batch) for h in range(og.num_kv_heads) for t in range(nfull)]
    for s, bits in enumerate((k_bits, v_bits)):
        for (b, h, tile) in tiles:
            x = R.canonicalize(bits[b, tile * G:(tile + 1) * G, h])[0]       # [G][D]
            w_ref = R.apply_rotation(x, gc.sigma, og.variant)
            if w is not None:
                ok, worst = close_rowwise(w[s][b, tile * G:(tile + 1) * G, h], w_ref, 1e-5)
                assert ok, ("W", s, b, h, tile, worst)
            rec = hc.record(b, h, tile, s)
            u = R.unpack_record(rec, G, 128, s, og.bits)
            # layout: the oracle's packing of the GPU's own fields is the GPU record
            assert np.array_equal(R.pack_record(u["q"], u["r16"], u["c16"], u["s16"], u["z16"], s, og.bits), rec)
            t_ref = R.quantize_tile(w_ref, og.varn_iters, og.variant, og.bits)
            dr = fp16_ulp_dist(u["r16"], t_ref["r16"])
            dc = fp16_ulp_dist(u["c16"], t_ref["c16"])
            assert dr.max() <= 1 and dc.max() <= 1, ("r/c ulp", s, b, h, tile, dr.max(), dc.max())
            stats["r_mis"] += int((dr > 0).sum())
            stats["c_mis"] += int((dc > 0).sum())
            stats["n_r"] += G
            stats["n_c"] += 128
            y_ref = R.normalize(w_ref, u["r16"], u["c16"])
            if y is not None:
                ok, worst = close_rowwise(y[s][b, tile * G:(tile + 1) * G, h], y_ref, 1e-5)
                assert ok, ("Y", s, b, h, tile, worst)
            s_ref, z_ref, _ = R.grid(y_ref, og.bits)
            ds = fp16_ulp_dist(u["s16"], s_ref)
            dz = fp16_ulp_dist(u["z16"], z_ref)
            assert ds.max() <= 1 and dz.max() <= 1, ("s/z ulp", s, b, h, tile)
            stats["s_mis"] += int((ds > 0).sum())
            stats["z_mis"] += int((dz > 0).sum())
            q_ref = R.codes(y_ref, u["s16"], u["z16"], og.bits)
            uu = R.pre_rounding(y_ref, u["s16"], u["z16"])
            frac = uu - np.floor(uu)
            near_edge = (np.abs(frac - 0.5) < EDGE_BAND) & (uu > -0.5) & (uu < 2 ** og.bits - 0.5)
            bad = (q_ref != u["q"]) & ~near_edge
            assert not bad.any(), ("codes", s, b, h, tile, int(bad.sum()))
            stats["edge_exempt"] += int(((q_ref != u["q"]) & near_edge).sum())
            stats["codes"] += q_ref.size
    # tail bytes and lengths
    for s, bits in enumerate((k_bits, v_bits)):
        for b in range(og.batch):
            for h in range(og.num_kv_heads):
                tail = hc.tail(b, h, s)
                for t in range(nfull * G, T):
                    want = R.bf16_bits(R.canonicalize(bits[b, t, h])[0])
                    assert np.array_equal(tail[t % G], want), ("tail", s, b, h, t)
    if stats["n_r"]:
        assert stats["r_mis"] / (2 * stats["n_r"]) <= 1e-2
        assert stats["c_mis"] / (2 * stats["n_c"]) <= 1e-2
        assert (stats["s_mis"] + stats["z_mis"]) / (4 * stats["n_c"]) <= 1e-2
        assert stats["edge_exempt"] / stats["codes"] <= 1e-3
    return stats


def gpu_prefill(gc: GpuCache, k_bits, v_bits, T, debug=False):
    """Prefill with the first T tokens of k_bits, v_bits (uint16 [B][>= T][H][D]): the
    library reads a contiguous [B][T][H][D] input, so longer arrays are cut first."""
    k = from_u16(k_bits[:, :T])
    v = from_u16(v_bits[:, :T])
    B, H = gc.og.batch, gc.og.num_kv_heads
    tf = (T // gc.og.group) * gc.og.group
    if debug:
        w = torch.full((2, B, max(tf, 1), H, 128), float("nan"), device="cuda")
        y = torch.full((2, B, max(tf, 1), H, 128), float("nan"), device="cuda")
        K.kvarn_debug_prefill(gc.g, gc.buf, k, v, T, w[0], w[1], y[0], y[1])
        torch.cuda.synchronize()
        return w.cpu().numpy().astype(np.float64), y.cpu().numpy().astype(np.float64)
    K.kvarn_quantize_prefill(gc.g, gc.buf, k, v, T)
    torch.cuda.synchronize()
    return None, None


def check_attention(out_gpu: np.ndarray, hc: R.Cache, q_bits, Hq, scale=0.0, flags=0, bh=None):
    """attn output vs the oracle's attention over the same (GPU-written) cache bytes."""
    ref = R.attn_decode(hc, q_bits, Hq, scale, flags)
    worst = 0.0
    for b in range(ref.shape[0]):
        for g in range(Hq):
            m = np.abs(ref[b, g]).max()
            d = np.abs(out_gpu[b, g] - ref[b, g]).max()
            assert d <= 2e-3 * m + 1e-30 or (m == 0 and d == 0), ("attn", b, g, d, m)
            worst = max(worst, d / m if m > 0 else 0.0)
    return worst


class PagedCache(GpuCache):
    """A layer cache whose tiles live in a page pool behind a per-sequence page map."""

    def __init__(self, B, H, cap, G, n_it, num_pages, seed_sigma=0, bits=2):
        self.g = K.geom(B, H, cap, G, n_it, bits=bits, num_pages=num_pages)
        self.og = R.Geom(B, H, 128, cap, G, n_it, bits, 0, num_pages)
        self.sigma = synth.sign_vector(seed_sigma, 128)
        self.buf = K.alloc_cache(self.g, self.sigma)

    def set_pages(self, pages, tile_first=0):
        p = torch.from_numpy(np.ascontiguousarray(pages, dtype=np.int32)).cuda()
        K.kvarn_cache_set_pages(self.g, self.buf, p, tile_first, p.shape[1])


def same_stored(a: R.Cache, b: R.Cache, seqs=None):
    """Equal lengths, and equal tail bytes and records of every stored tile."""
    g = a.g
    seqs = range(g.batch) if seqs is None else seqs
    for bb in seqs:
        assert np.array_equal(a.lens[bb], b.lens[bb]), bb
        for h in range(g.num_kv_heads):
            for s in range(2):
                n = int(a.lens[bb, h, s])
                for tile in range(n // g.group):
                    ra, rb = a.record(bb, h, tile, s), b.record(bb, h, tile, s)
                    assert ra is not None and rb is not None and np.array_equal(ra, rb), (bb, h, tile, s)
                assert np.array_equal(a.tail(bb, h, s)[:n % g.group], b.tail(bb, h, s)[:n % g.group])
