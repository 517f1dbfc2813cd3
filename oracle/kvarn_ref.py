"""CPU oracle for the KVarN 2-bit KV-cache quantizer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. The library path never calls it; it shares no code, header,
table or constant generator with the HIP kernels.

It is a plain, slow, fp64 NumPy implementation of what the KVarN pages define,
written step by step in the pages' order. Citations name the page and its
section:

  [RP]  researchpapers.dev, "KVarN: calibration-free 2-bit KV cache quantization"
  [FB]  friday-blog, "Memory breakout: KVarN ..." (sections 1-5)
  [AP]  ai-paper-analysis, "KVarN: variance normalization lets 2-bit KV cache ..."
        (sections 1-8, subsections 3.1 and 3.2, the error equation in section 2)
  [CP]  chatpaper.ai abstract (Spanish and English)

Method ([AP] section 3; [RP] "how KVarN does it"; [CP] abstract):
  1. rotate each K/V token along head_dim by a randomized Hadamard matrix H with
     H H^T = I ([AP] 3.1);
  2. VarN: alternately bring every token's variance and every channel's variance
     to 1, repeated 2-3 times, Sinkhorn-Knopp style ([AP] 3.2 steps 1-3);
  3. keep the scales (grouped, restorable at dequantization) and quantize
     uniformly to 2 bits, 4 levels ([AP] 3.2 and the closing remark of 3.2);
  4. decode attention reads the cache with Q rotated by the same H, so that
     Q K^T is unchanged ([AP] 3.1).

Where the pages leave a step open, the reading taken is stated at the function
that implements it (bf16 inputs kept as given, second-moment "variance", Sylvester
ordering of H, fp16 stored scales, per-channel min/max grid over a group of G
tokens, round-half-to-even, bf16 tail of unrotated tokens, tile record layout).

Pinned by tests/test_oracle_*.py against closed forms, invariants, brute force
and library routines (see each test's docstring).
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------- format constants
# Written out here on purpose: the oracle includes nothing from the library.
MAGIC = 0x4E52564B          # bytes 'K','V','R','N' little-endian
VERSION = 3                 # 3: the tail holds bf16 (2: fp16)
FLAG_CAPACITY = 1           # an append found the cache full (token dropped)
FLAG_SATURATED = 2          # an input value was beyond +-2^16 (or infinite) and was saturated
FLAG_SCALE_CLAMPED = 4      # a stored scale hit the fp16 clamp range
FLAG_UNMAPPED = 8           # a paged cache had no page for a tile that was written
FLAG_NAN = 16               # an input value was NaN (stored as 0)
Q_PREROTATED = 1            # attention flag: the query is already rotated (q H)
FP16_MAX = 65504.0
IN_MAX = 65536.0            # inputs saturate at +-2^16 (a bf16 value)
SCALE_MIN = 2.0 ** -14      # smallest normal fp16; lower clamp of r and c
HEADER_FIXED = 512          # len[] starts here
SIGMA_OFFSET = 64
SIGN_WORDS_OFFSET = 192     # uint32[head_dim / 2]: word d has bit 15 set where sigma[2d] = -1
                            # and bit 31 where sigma[2d + 1] = -1 (sigma restated as the sign
                            # bits of a packed pair of 16-bit floats)
FLAGS_OFFSET = 36
VARIANT_OFFSET = 40
NUM_PAGES_OFFSET = 44
# Ablation variants ([AP] section 5, ablations: Hadamard only, VarN only, VarN along one
# axis only). A bit set removes one component; 0 is the method as defined.
VARIANT_NO_ROTATION = 1       # H_D replaced by the identity ("VarN only")
VARIANT_NO_CHANNEL_PASS = 2   # VarN keeps the token-axis passes only
VARIANT_NO_TOKEN_PASS = 4     # VarN keeps the channel-axis passes only
VARIANT_CENTERED = 8          # "variance" about the mean instead of the mean square


def align256(n: int) -> int:
    return (n + 255) // 256 * 256


# ----------------------------------------------------------------------------- number formats
def fp16_round(x) -> np.ndarray:
    """Round to IEEE binary16, round-half-to-even, subnormals kept, overflow to inf."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def fp16_saturate(x) -> tuple[np.ndarray, np.ndarray]:
    """Clamp to [-65504, 65504], then round to fp16. Returns (values, was_clamped)."""
    x = np.asarray(x, dtype=np.float64)
    clamped = np.abs(x) > FP16_MAX
    return fp16_round(np.clip(x, -FP16_MAX, FP16_MAX)), clamped


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def canonicalize(bits) -> tuple[np.ndarray, bool, bool]:
    """Reading: the K/V inputs are taken as given, bf16 values, and the decode-time
    tail stores them unchanged (bf16), so a token quantizes identically whether it
    arrives in a prefill or through the tail. The pages fix neither the dtype of the
    tokens not yet quantized nor any conversion of the inputs (their "FP16" names the
    16-bit cache the method is compared with); keeping the model's bf16 values stores
    those tokens exactly. Values beyond +-2^16, infinities included, saturate at +-2^16
    (a bf16 value), which bounds every sum the method takes; the pages assume finite
    inputs, so a NaN is stored as 0 and reported. Returns (values, saturated, had_nan)."""
    x = bf16_to_f64(bits)
    nan = np.isnan(x)
    x = np.where(nan, 0.0, x)
    sat = np.abs(x) > IN_MAX
    return np.clip(x, -IN_MAX, IN_MAX), bool(sat.any()), bool(nan.any())


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of values that bf16 holds exactly (canonical inputs)."""
    x = np.asarray(x, dtype=np.float64)
    u = x.astype(np.float32).view(np.uint32)
    assert not np.any(u & 0xFFFF) and np.array_equal(x.astype(np.float32).astype(np.float64), x)
    return (u >> 16).astype(np.uint16)


def fp16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def fp16_from_bits(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------------------- rotation ([AP] 3.1)
def hadamard_sylvester(d: int) -> np.ndarray:
    """Reading of "Hadamard matrix": Sylvester ordering, H[i, j] = (-1)^popcount(i & j)."""
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pc = np.zeros_like(bits)
    while bits.any():
        pc += bits & 1
        bits >>= 1
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def rotation_matrix(sigma) -> np.ndarray:
    """H_D = diag(sigma) H_syl / sqrt(D): the randomized Hadamard matrix, H_D H_D^T = I."""
    s = np.asarray(sigma, dtype=np.float64)
    d = s.shape[0]
    return s[:, None] * hadamard_sylvester(d) / np.sqrt(d)


def rotate(x, sigma) -> np.ndarray:
    """Row vectors x (last axis = head_dim) times H_D."""
    return np.asarray(x, dtype=np.float64) @ rotation_matrix(sigma)


def unrotate(w, sigma) -> np.ndarray:
    """Inverse rotation: w H_D^T."""
    return np.asarray(w, dtype=np.float64) @ rotation_matrix(sigma).T


def apply_rotation(x, sigma, variant: int = 0) -> np.ndarray:
    """x H_D, or x itself for the "VarN only" ablation (VARIANT_NO_ROTATION)."""
    return np.asarray(x, dtype=np.float64) if variant & VARIANT_NO_ROTATION else rotate(x, sigma)


def undo_rotation(w, sigma, variant: int = 0) -> np.ndarray:
    """w H_D^T, or w itself for the "VarN only" ablation."""
    return np.asarray(w, dtype=np.float64) if variant & VARIANT_NO_ROTATION else unrotate(w, sigma)


# ----------------------------------------------------------------------------- VarN ([AP] 3.2)
def _spread(y, axis: int, centered: bool) -> np.ndarray:
    """Mean square of y along `axis`; with `centered`, the variance about the mean."""
    if centered:
        y = y - np.mean(y, axis=axis, keepdims=True)
    return np.mean(y * y, axis=axis)


def varn(w, n_it: int, variant: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Dual-axis variance normalization of tile(s) w[..., G, D]; returns (r[..., G], c[..., D]).

    [AP] 3.2: (1) normalize along the token axis so each token's variance is 1,
    (2) normalize along the channel axis so each channel's variance is 1,
    (3) repeat 2-3 times so both axes approach 1 together (Sinkhorn-Knopp like).
    Readings: "variance" is the mean square (second moment about zero, divide by N);
    the scales are cumulative and multiplicative, Y = W / (r_t c_j), starting at 1;
    one iteration is a token pass followed by a channel pass; a pass leaves the
    scale unchanged where the mean square is 0 (all-zero row or column).
    Ablations ([AP] section 5): VARIANT_NO_CHANNEL_PASS / VARIANT_NO_TOKEN_PASS drop
    one of the two passes (the other then reaches its fixed point after one pass),
    VARIANT_CENTERED measures the variance about the mean.
    """
    w = np.asarray(w, dtype=np.float64)
    r = np.ones(w.shape[:-1])
    c = np.ones(w.shape[:-2] + w.shape[-1:])
    centered = bool(variant & VARIANT_CENTERED)
    for _ in range(n_it):
        if not variant & VARIANT_NO_TOKEN_PASS:
            y = w / (r[..., :, None] * c[..., None, :])
            ms_t = _spread(y, -1, centered)                  # token axis: one value per token
            r = np.where(ms_t > 0, r * np.sqrt(ms_t), r)
        if not variant & VARIANT_NO_CHANNEL_PASS:
            y = w / (r[..., :, None] * c[..., None, :])
            ms_j = _spread(y, -2, centered)                  # channel axis: one value per channel
            c = np.where(ms_j > 0, c * np.sqrt(ms_j), c)
    return r, c


def stored_scales(r, c) -> tuple[np.ndarray, np.ndarray, bool]:
    """The scales are kept so dequantization can undo them ([AP] 3.2, grouped scales).
    Reading: stored as fp16 (RNE), clamped to [2^-14, 65504]."""
    r = np.asarray(r, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    rc = np.clip(r, SCALE_MIN, FP16_MAX)
    cc = np.clip(c, SCALE_MIN, FP16_MAX)
    clamped = bool((rc != r).any() or (cc != c).any())
    return fp16_round(rc), fp16_round(cc), clamped


def normalize(w, r16, c16) -> np.ndarray:
    """Y = W / (r16 (x) c16), with the stored scales so r16 c16 Y recovers W exactly."""
    return np.asarray(w, dtype=np.float64) / (np.asarray(r16)[..., :, None] * np.asarray(c16)[..., None, :])


# ----------------------------------------------------------------------------- 2-bit grid
def grid(y, bits: int = 2) -> tuple[np.ndarray, np.ndarray, bool]:
    """Uniform 2-bit grid, one per channel over the tile's G tokens ([AP] 3.2: one scale
    per group of 32 or 64 entries; [RP]: a scale shared across tokens is what outlier
    tokens stretch). Reading: asymmetric min/max, levels z + s*{0,1,2,3},
    s = (max - min)/3, both stored as fp16 (RNE, saturating). With bits = 3 or 4 (the
    widths beyond the pages' 2) the same grid has 2^bits levels, s = (max - min)/(2^bits - 1)."""
    y = np.asarray(y, dtype=np.float64)
    mn = y.min(axis=-2)
    mx = y.max(axis=-2)
    s16, sat_s = fp16_saturate((mx - mn) / (2 ** bits - 1))
    z16, sat_z = fp16_saturate(mn)
    return s16, z16, bool(sat_s.any() or sat_z.any())


def codes(y, s16, z16, bits: int = 2) -> np.ndarray:
    """q = clamp(round_half_even((Y - z) / s), 0, 2^bits - 1); q = 0 in a channel whose s is 0."""
    y = np.asarray(y, dtype=np.float64)
    s = np.asarray(s16)[..., None, :]
    z = np.asarray(z16)[..., None, :]
    safe = np.where(s == 0, 1.0, s)
    u = (y - z) / safe
    q = np.clip(np.rint(u), 0, 2 ** bits - 1)   # np.rint rounds half to even
    return np.where(s == 0, 0, q).astype(np.uint8)


def pre_rounding(y, s16, z16) -> np.ndarray:
    """u = (Y - z)/s, the value whose rounding gives the code (for edge-band checks)."""
    s = np.asarray(s16)[..., None, :]
    z = np.asarray(z16)[..., None, :]
    return (np.asarray(y) - z) / np.where(s == 0, 1.0, s)


def quantize_tile(w, n_it: int, variant: int = 0, bits: int = 2) -> dict:
    """Rotated tile(s) w[..., G, D] -> stored scales, grid, codes (steps of [AP] 3.2)."""
    r, c = varn(w, n_it, variant)
    r16, c16, clamped = stored_scales(r, c)
    y = normalize(w, r16, c16)
    s16, z16, sat = grid(y, bits)
    q = codes(y, s16, z16, bits)
    return dict(r=r, c=c, r16=r16, c16=c16, y=y, s16=s16, z16=z16, q=q,
                flags=(FLAG_SCALE_CLAMPED if (clamped or sat) else 0))


def dequantize_tile(q, r16, c16, s16, z16) -> np.ndarray:
    """W_hat = r16_t c16_j (z16_j + s16_j q_tj): undo the grid and both scales."""
    q = np.asarray(q, dtype=np.float64)
    return (np.asarray(r16)[..., :, None] * np.asarray(c16)[..., None, :]
            * (np.asarray(z16)[..., None, :] + np.asarray(s16)[..., None, :] * q))


# ----------------------------------------------------------------------------- tile record (unchanged since format v2)
def record_bytes(g: int, d: int, bits: int = 2) -> int:
    """codes G*D*bits/8 | r fp16[G] | c fp16[D] | s fp16[D] | z fp16[D]."""
    return g * d * bits // 8 + 2 * g + 6 * d


def k_code_position(j: int) -> tuple[int, int]:
    """K stream: (32-bit word w, 2-bit slot p) holding channel j of a token.
    Word w holds the 16 channels {16 m + 2 w + d : m < 8, d < 2} at slot
    p = 4 (m // 2) + m % 2 + 2 d, so byte k of the word holds m in {2k, 2k+1}, both d."""
    m, w, d = j // 16, (j % 16) // 2, j % 2
    return w, 4 * (m // 2) + m % 2 + 2 * d


def pack_codes(q, stream: int, bits: int = 2) -> np.ndarray:
    """Codes of `bits` bits as bit planes: plane A (bits 0-1 of every code) in the 2-bit
    layout below, then for bits = 4 plane B (bits 2-3) in the same 2-bit layout, or for
    bits = 3 plane B (bit 2) in the 1-bit layout of pack_bit_plane."""
    q = np.asarray(q, dtype=np.uint8)
    if bits == 2:
        return pack_2bit(q, stream)
    plane_b = pack_2bit(q >> 2, stream) if bits == 4 else pack_bit_plane(q >> 2, stream)
    return np.concatenate([pack_2bit(q & 3, stream), plane_b])


def unpack_codes(b, g: int, d: int, stream: int, bits: int = 2) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    if bits == 2:
        return unpack_2bit(b, g, d, stream)
    n = g * d // 4
    hi = unpack_2bit(b[n:], g, d, stream) if bits == 4 else unpack_bit_plane(b[n:], g, d, stream)
    return (unpack_2bit(b[:n], g, d, stream) | (hi << 2)).astype(np.uint8)


def k_bit_position(j: int) -> tuple[int, int]:
    """1-bit plane, K stream: (32-bit word u, bit p) of channel j of a token. Word u pairs the
    2-bit layout's words 2u and 2u + 1: the channel in word w, slot k sits at bit
    4 (k // 2) + k % 2 + 2 (w % 2) of word w // 2."""
    w, k = k_code_position(j)
    return w // 2, 4 * (k // 2) + k % 2 + 2 * (w % 2)


def v_bit_position(t: int, j: int, g: int) -> tuple[int, int]:
    """1-bit plane, V stream: (32-bit word index, bit) of code (t, j). With j = 16 blk + c,
    blk = i + 4 hh (i < 4), i = 2 ip + ii and t = 8 o + 2 n + par: word
    (16 ip + c) * G/8 + o, bit 4 (n + 4 hh) + par + 2 ii. A word holds the 8 tokens of an
    octet for the four channels c + 16 {2ip, 2ip + 1, 2ip + 4, 2ip + 5}."""
    blk, c = j // 16, j % 16
    i, hh = blk % 4, blk // 4
    ip, ii = i // 2, i % 2
    o, u = t // 8, t % 8
    n, par = u // 2, u % 2
    return (16 * ip + c) * (g // 8) + o, 4 * (n + 4 * hh) + par + 2 * ii


def pack_bit_plane(qb, stream: int) -> np.ndarray:
    """One bit per code, 32 per little-endian word: K token t owns words 4t .. 4t + 3
    (k_bit_position); V words as v_bit_position. G*D/8 bytes either way."""
    qb = np.asarray(qb, dtype=np.uint32) & 1
    g, d = qb.shape
    words = np.zeros(g * d // 32, dtype=np.uint32)
    for t in range(g):
        for j in range(d):
            if stream == 0:
                u, p = k_bit_position(j)
                words[(d // 32) * t + u] |= np.uint32(qb[t, j] << p)
            else:
                wi, p = v_bit_position(t, j, g)
                words[wi] |= np.uint32(qb[t, j] << p)
    return words.view(np.uint8)


def unpack_bit_plane(b, g: int, d: int, stream: int) -> np.ndarray:
    words = np.asarray(b, dtype=np.uint8).view(np.uint32)
    q = np.zeros((g, d), dtype=np.uint8)
    for t in range(g):
        for j in range(d):
            if stream == 0:
                u, p = k_bit_position(j)
                q[t, j] = (words[(d // 32) * t + u] >> p) & 1
            else:
                wi, p = v_bit_position(t, j, g)
                q[t, j] = (words[wi] >> p) & 1
    return q


def pack_2bit(q, stream: int) -> np.ndarray:
    """Four 2-bit codes per byte, slot k of a byte at bits 2k..2k+1 (little-endian words).
    K (stream 0): token t owns bytes t*D/4 .. t*D/4 + D/4 - 1, read as D/16 words;
                  channel j sits in word w, slot p (k_code_position): byte t*D/4 + 4w + p//4,
                  bits 2*(p%4);
    V (stream 1): code (t, j) in byte j*G/4 + t//4 at bits 2*(t%4) (tokens fastest)."""
    q = np.asarray(q, dtype=np.uint8)
    g, d = q.shape
    if stream == 0:
        out = np.zeros((g, d // 4), dtype=np.uint8)
        for j in range(d):
            w, p = k_code_position(j)
            out[:, 4 * w + p // 4] |= (q[:, j] << (2 * (p % 4))).astype(np.uint8)
        return out.reshape(-1)
    qq = q.T.reshape(d, g // 4, 4)                         # [j][t//4][t%4]
    b = (qq[..., 0] | (qq[..., 1] << 2) | (qq[..., 2] << 4) | (qq[..., 3] << 6)).astype(np.uint8)
    return b.reshape(-1)


def unpack_2bit(b, g: int, d: int, stream: int) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    if stream == 0:
        rows = b.reshape(g, d // 4)
        q = np.zeros((g, d), dtype=np.uint8)
        for j in range(d):
            w, p = k_code_position(j)
            q[:, j] = (rows[:, 4 * w + p // 4] >> (2 * (p % 4))) & 3
        return q
    parts = np.stack([(b >> (2 * m)) & 3 for m in range(4)], axis=-1)
    return parts.reshape(d, g).T.astype(np.uint8)


def pack_record(q, r16, c16, s16, z16, stream: int, bits: int = 2) -> np.ndarray:
    return np.concatenate([pack_codes(q, stream, bits),
                           fp16_bits(r16).view(np.uint8), fp16_bits(c16).view(np.uint8),
                           fp16_bits(s16).view(np.uint8), fp16_bits(z16).view(np.uint8)])


def unpack_record(rec, g: int, d: int, stream: int, bits: int = 2) -> dict:
    rec = np.asarray(rec, dtype=np.uint8)
    n = g * d * bits // 8
    f = lambda off, k: fp16_from_bits(rec[off:off + 2 * k].view(np.uint16))  # noqa: E731
    return dict(q=unpack_codes(rec[:n], g, d, stream, bits), r16=f(n, g), c16=f(n + 2 * g, d),
                s16=f(n + 2 * g + 2 * d, d), z16=f(n + 2 * g + 4 * d, d))


# ----------------------------------------------------------------------------- cache buffer (format v3)
class Geom:
    """batch, num_kv_heads, head_dim, capacity, group, varn_iters, bits, variant (VARIANT_* bits),
    num_pages (0: tiles stored per sequence; > 0: a pool of pages found through a page map)."""

    def __init__(self, batch, num_kv_heads, head_dim=128, capacity=0, group=32, varn_iters=3, bits=2,
                 variant=0, num_pages=0):
        self.batch, self.num_kv_heads, self.head_dim = batch, num_kv_heads, head_dim
        self.capacity, self.group, self.varn_iters, self.bits = capacity, group, varn_iters, bits
        self.variant = variant
        self.num_pages = num_pages

    def as_tuple(self):
        return (self.batch, self.num_kv_heads, self.head_dim, self.capacity, self.group,
                self.varn_iters, self.bits)

    # layout
    @property
    def tr(self):
        return record_bytes(self.group, self.head_dim, self.bits)

    @property
    def paged(self):
        return self.num_pages > 0

    @property
    def map_offset(self):
        """Page map int32 [B][capacity/G] (paged caches): right after len[]."""
        return HEADER_FIXED + 8 * self.batch * self.num_kv_heads

    @property
    def header(self):
        extra = 4 * self.batch * self.tiles_per_seq if self.paged else 0
        return align256(HEADER_FIXED + 8 * self.batch * self.num_kv_heads + extra)

    @property
    def tiles_per_seq(self):
        return self.capacity // self.group

    @property
    def pool_bytes(self):
        """Records: one page = the K and V records of every kv head for one group of G tokens
        of one sequence ([Hkv][2][TR]); per-sequence storage is [B][Hkv][capacity/G][2][TR]."""
        if self.paged:
            return self.num_pages * self.num_kv_heads * 2 * self.tr
        return self.batch * self.num_kv_heads * self.tiles_per_seq * 2 * self.tr

    @property
    def tail_offset(self):
        return self.header + align256(self.pool_bytes)

    @property
    def total(self):
        return self.tail_offset + align256(self.batch * self.num_kv_heads * 2 * self.group * self.head_dim * 2)

    def record_offset(self, b, h, tile, s):
        assert not self.paged
        return self.header + ((((b * self.num_kv_heads + h) * self.tiles_per_seq + tile) * 2 + s) * self.tr)

    def page_offset(self, page, h, s):
        return self.header + ((page * self.num_kv_heads + h) * 2 + s) * self.tr

    def tail_slot_offset(self, b, h, s, slot):
        return self.tail_offset + ((((b * self.num_kv_heads + h) * 2 + s) * self.group + slot)
                                   * self.head_dim * 2)


def sign_words(sigma) -> np.ndarray:
    """The header's restatement of sigma: for each channel pair (2d, 2d + 1) one uint32 with
    bit 15 set where sigma[2d] = -1 and bit 31 set where sigma[2d + 1] = -1."""
    neg = np.asarray(sigma, np.float64) < 0
    lo = np.where(neg[0::2], 0x8000, 0).astype(np.uint64)
    hi = np.where(neg[1::2], 0x80000000, 0).astype(np.uint64)
    return (lo | hi).astype(np.uint32)


class Cache:
    """A layer's cache as the byte buffer the library keeps in device memory."""

    def __init__(self, geom: Geom, sigma):
        self.g = geom
        self.buf = np.zeros(geom.total, dtype=np.uint8)
        hdr = self.buf[:geom.header]
        hdr[0:4].view(np.uint32)[0] = MAGIC
        hdr[4:8].view(np.uint32)[0] = VERSION
        hdr[8:36].view(np.int32)[:] = geom.as_tuple()
        hdr[VARIANT_OFFSET:VARIANT_OFFSET + 4].view(np.uint32)[0] = geom.variant
        hdr[NUM_PAGES_OFFSET:NUM_PAGES_OFFSET + 4].view(np.int32)[0] = geom.num_pages
        hdr[SIGMA_OFFSET:SIGMA_OFFSET + geom.head_dim].view(np.int8)[:] = np.asarray(sigma, np.int8)
        hdr[SIGN_WORDS_OFFSET:SIGN_WORDS_OFFSET + 2 * geom.head_dim].view(np.uint32)[:] = sign_words(sigma)
        if geom.paged:
            self.page_map[:] = -1                               # no page yet

    # header fields
    @property
    def sigma(self):
        d = self.g.head_dim
        return self.buf[SIGMA_OFFSET:SIGMA_OFFSET + d].view(np.int8).astype(np.float64)

    @property
    def flags(self) -> int:
        return int(self.buf[FLAGS_OFFSET:FLAGS_OFFSET + 4].view(np.uint32)[0])

    def or_flags(self, f: int):
        self.buf[FLAGS_OFFSET:FLAGS_OFFSET + 4].view(np.uint32)[0] |= np.uint32(f)

    @property
    def lens(self) -> np.ndarray:
        n = self.g.batch * self.g.num_kv_heads * 2
        return self.buf[HEADER_FIXED:HEADER_FIXED + 4 * n].view(np.int32).reshape(
            self.g.batch, self.g.num_kv_heads, 2)

    @property
    def page_map(self) -> np.ndarray:
        """int32 [B][capacity/G]: the page holding each tile of each sequence (-1: none)."""
        g = self.g
        n = g.batch * g.tiles_per_seq
        return self.buf[g.map_offset:g.map_offset + 4 * n].view(np.int32).reshape(g.batch, g.tiles_per_seq)

    def set_pages(self, pages, tile_first: int = 0):
        """Map tiles [tile_first, tile_first + n) of every sequence: pages int32 [B][n]."""
        pages = np.asarray(pages, dtype=np.int32)
        self.page_map[:, tile_first:tile_first + pages.shape[1]] = pages

    # records and tail
    def record(self, b, h, tile, s):
        """The tile's record bytes, or None for a paged cache without a valid page there."""
        g = self.g
        if g.paged:
            page = int(self.page_map[b, tile])
            if not 0 <= page < g.num_pages:
                return None
            o = g.page_offset(page, h, s)
        else:
            o = g.record_offset(b, h, tile, s)
        return self.buf[o:o + g.tr]

    def record_offset(self, b, h, tile, s):
        r = self.record(b, h, tile, s)
        return None if r is None else int(r.ctypes.data - self.buf.ctypes.data)

    def tail(self, b, h, s) -> np.ndarray:
        """bf16 bit patterns, a uint16 view [G][D] of one tail."""
        o = self.g.tail_slot_offset(b, h, s, 0)
        n = self.g.group * self.g.head_dim * 2
        return self.buf[o:o + n].view(np.uint16).reshape(self.g.group, self.g.head_dim)

    def tail_values(self, b, h, s) -> np.ndarray:
        """The values of one tail, fp64 [G][D]."""
        return bf16_to_f64(self.tail(b, h, s))

    def defined_mask(self) -> np.ndarray:
        """Bytes whose content the format defines given the current lengths."""
        g = self.g
        m = np.zeros(g.total, dtype=bool)
        m[:g.header] = True
        for b in range(g.batch):
            for h in range(g.num_kv_heads):
                for s in range(2):
                    n = int(self.lens[b, h, s])
                    for tile in range(n // g.group):
                        o = self.record_offset(b, h, tile, s)
                        if o is not None:
                            m[o:o + g.tr] = True
                    o = g.tail_slot_offset(b, h, s, 0)
                    m[o:o + (n % g.group) * g.head_dim * 2] = True
        return m


def _quantize_stream(x, sigma, g: Geom, stream: int):
    """x[..., n_tiles*G, D] canonical fp64 tokens -> (records [..., n_tiles, TR], flags)."""
    lead = x.shape[:-2]
    nt = x.shape[-2] // g.group
    w = apply_rotation(x, sigma, g.variant).reshape(lead + (nt, g.group, g.head_dim))
    t = quantize_tile(w, g.varn_iters, g.variant, g.bits)
    recs = np.zeros(lead + (nt, g.tr), dtype=np.uint8)
    for idx in np.ndindex(*(lead + (nt,))):
        recs[idx] = pack_record(t["q"][idx], t["r16"][idx], t["c16"][idx], t["s16"][idx],
                                t["z16"][idx], stream, g.bits)
    return recs, t["flags"]


def quantize_prefill(cache: Cache, k_bits, v_bits, num_tokens: int) -> None:
    """Reset the cache to hold tokens [0, T) of k, v (bf16 bits [B][T][Hkv][D]).
    Full groups of G tokens become tile records; the last T mod G tokens stay in
    the bf16 tail, unrotated ([AP] 3.2: the current group is still being filled)."""
    g = cache.g
    T = int(num_tokens)
    assert 0 <= T <= g.capacity
    nfull = T // g.group
    for s, bits in enumerate((k_bits, v_bits)):
        x, sat, nan = canonicalize(np.asarray(bits)[:, :T])     # [B][T][Hkv][D]
        if sat:
            cache.or_flags(FLAG_SATURATED)
        if nan:
            cache.or_flags(FLAG_NAN)
        xt = np.transpose(x, (0, 2, 1, 3))                       # [B][Hkv][T][D]
        if nfull:
            recs, f = _quantize_stream(xt[:, :, :nfull * g.group], cache.sigma, g, s)
            cache.or_flags(f)
            for b in range(g.batch):
                for h in range(g.num_kv_heads):
                    for tile in range(nfull):
                        rec = cache.record(b, h, tile, s)
                        if rec is None:
                            cache.or_flags(FLAG_UNMAPPED)
                        else:
                            rec[:] = recs[b, h, tile]
        for b in range(g.batch):
            for h in range(g.num_kv_heads):
                tail = cache.tail(b, h, s)
                for t in range(nfull * g.group, T):
                    tail[t % g.group] = bf16_bits(xt[b, h, t])
    cache.lens[:] = T


def append_decode(cache: Cache, k_bits, v_bits, mask=None) -> None:
    """Append one token per (batch, kv head) (bf16 bits [B][Hkv][D]) through the bf16 tail.
    When a group of G fills, it is rotated, normalized and quantized into the next
    tile record ([AP] 3.2: statistics of the current group are updated as tokens arrive).
    `mask` (bool [B]) restricts the append to the sequences it selects. Flags: a token
    dropped at capacity is not read (no saturation flag from it); a group quantized for a
    tile without a page still raises its scale flags."""
    g = cache.g
    bits_s = (np.asarray(k_bits), np.asarray(v_bits))
    for s in range(2):
        for b in range(g.batch):
            if mask is not None and not mask[b]:
                continue
            for h in range(g.num_kv_heads):
                pos = int(cache.lens[b, h, s])
                if pos >= g.capacity:
                    cache.or_flags(FLAG_CAPACITY)
                    continue
                x, sat, nan = canonicalize(bits_s[s][b, h])
                if sat:
                    cache.or_flags(FLAG_SATURATED)
                if nan:
                    cache.or_flags(FLAG_NAN)
                tail = cache.tail(b, h, s)
                tail[pos % g.group] = bf16_bits(x)
                if (pos + 1) % g.group == 0:
                    tile_x = cache.tail_values(b, h, s)[None]      # [1][G][D]
                    recs, f = _quantize_stream(tile_x, cache.sigma, g, s)
                    cache.or_flags(f)
                    rec = cache.record(b, h, (pos + 1) // g.group - 1, s)
                    if rec is None:
                        cache.or_flags(FLAG_UNMAPPED)
                    else:
                        rec[:] = recs[0]
                cache.lens[b, h, s] = pos + 1


def append_tokens(cache: Cache, k_bits, v_bits, counts=None) -> None:
    """Append counts[b] tokens (bf16 bits [B][T][Hkv][D], the first counts[b] rows of
    sequence b; all T when counts is None) to every sequence after its stored tokens:
    the same as that many single-token appends in order. Covers a chunk of a prefill into
    a non-empty cache, ragged batches and per-sequence append masks (counts 0 or 1)."""
    k_bits, v_bits = np.asarray(k_bits), np.asarray(v_bits)
    T = k_bits.shape[1]
    counts = np.full(cache.g.batch, T) if counts is None else np.asarray(counts)
    for t in range(int(counts.max(initial=0))):
        append_decode(cache, k_bits[:, t], v_bits[:, t], mask=counts > t)


def stream_values(cache: Cache, b: int, h: int, s: int, rotated: bool = False, with_mask: bool = False):
    """All stored tokens of one stream, dequantized, in original space (fp64 [len][D]).
    With rotated=True the tile tokens are returned in rotated space and tail tokens
    are rotated too (used for checks that work in the rotated basis). Tokens of a tile
    without a page (paged cache) are absent: 0 here, and False in the mask returned
    with with_mask=True."""
    g = cache.g
    n = int(cache.lens[b, h, s])
    out = np.zeros((n, g.head_dim))
    present = np.ones(n, dtype=bool)
    nfull = n // g.group
    for tile in range(nfull):
        rec = cache.record(b, h, tile, s)
        if rec is None:
            present[tile * g.group:(tile + 1) * g.group] = False
            continue
        u = unpack_record(rec, g.group, g.head_dim, s, g.bits)
        w = dequantize_tile(u["q"], u["r16"], u["c16"], u["s16"], u["z16"])
        out[tile * g.group:(tile + 1) * g.group] = w if rotated else undo_rotation(w, cache.sigma, g.variant)
    tail = bf16_to_f64(cache.tail(b, h, s)[:n - nfull * g.group])  # the stored slots only
    for t in range(nfull * g.group, n):
        out[t] = apply_rotation(tail[t % g.group], cache.sigma, g.variant) if rotated else tail[t % g.group]
    return (out, present) if with_mask else out


def dequantize(cache: Cache, max_tokens: int) -> tuple[np.ndarray, np.ndarray]:
    """K_hat, V_hat as fp64 [B][max_tokens][Hkv][D]; rows at or past a sequence's length are 0.
    Tile tokens: undo grid and scales, then rotate back by H_D^T ([AP] 3.2: the scaling
    is restored at dequantization). Tail tokens are returned as stored."""
    g = cache.g
    outs = []
    for s in range(2):
        o = np.zeros((g.batch, max_tokens, g.num_kv_heads, g.head_dim))
        for b in range(g.batch):
            for h in range(g.num_kv_heads):
                vals = stream_values(cache, b, h, s)[:max_tokens]
                o[b, :vals.shape[0], h] = vals
        outs.append(o)
    return outs[0], outs[1]


def attn_decode(cache: Cache, q_bits, num_q_heads: int, softmax_scale: float = 0.0,
                flags: int = 0, pairs=None) -> np.ndarray:
    """Single-query decode attention over the dequantized cache, by its definition:
    l_t = scale * (q . k_hat_t), p = softmax(l), out = sum_t p_t v_hat_t  (fp64 [B][Hq][D]).
    Query head g reads KV head g // (Hq / Hkv). Readings: scale defaults to 1/sqrt(D);
    with Q_PREROTATED the given query is q H_D and is mapped back by H_D^T ([AP] 3.1:
    (qH)(kH)^T = q k^T). An empty sequence gives 0. `pairs` optionally restricts the
    work to a list of (batch, kv head); other outputs stay 0."""
    g = cache.g
    d = g.head_dim
    scale = softmax_scale if softmax_scale > 0 else 1.0 / np.sqrt(d)
    q = bf16_to_f64(q_bits)                                     # [B][Hq][D]
    if flags & Q_PREROTATED:
        q = undo_rotation(q, cache.sigma, g.variant)
    grp = num_q_heads // g.num_kv_heads
    out = np.zeros((g.batch, num_q_heads, d))
    todo = pairs if pairs is not None else [(b, h) for b in range(g.batch) for h in range(g.num_kv_heads)]
    for b, h in todo:
        k, present = stream_values(cache, b, h, 0, with_mask=True)
        v = stream_values(cache, b, h, 1)
        k, v = k[present], v[present]                            # tiles without a page are skipped
        if k.shape[0] == 0:
            continue
        for gi in range(h * grp, (h + 1) * grp):
            logits = scale * (k @ q[b, gi])
            p = np.exp(logits - logits.max())
            p /= p.sum()
            out[b, gi] = p @ v
    return out


def append_attn_decode(cache: Cache, k_bits, v_bits, q_bits, num_q_heads: int, softmax_scale: float = 0.0,
                       flags: int = 0) -> np.ndarray:
    """One decode step: attend with q over the stored tokens plus the new one, then append it.
    The stored tokens are read as in attn_decode (tiles dequantized, the tail as stored);
    the new token is its canonical bf16 value, which is also what a group completed by
    this token holds before it is quantized ([AP] 3.2: the group being filled is kept
    until it is complete). A full sequence attends without the token, which the append
    then drops."""
    g = cache.g
    d = g.head_dim
    scale = softmax_scale if softmax_scale > 0 else 1.0 / np.sqrt(d)
    q = bf16_to_f64(q_bits)
    if flags & Q_PREROTATED:
        q = undo_rotation(q, cache.sigma, g.variant)
    kn = canonicalize(k_bits)[0]                                # [B][Hkv][D]
    vn = canonicalize(v_bits)[0]
    grp = num_q_heads // g.num_kv_heads
    out = np.zeros((g.batch, num_q_heads, d))
    for b in range(g.batch):
        for h in range(g.num_kv_heads):
            k, present = stream_values(cache, b, h, 0, with_mask=True)
            v = stream_values(cache, b, h, 1)
            k, v = k[present], v[present]
            if int(cache.lens[b, h, 0]) < g.capacity:
                k = np.vstack([k, kn[b, h][None]])
                v = np.vstack([v, vn[b, h][None]])
            if k.shape[0] == 0:
                continue
            for gi in range(h * grp, (h + 1) * grp):
                logits = scale * (k @ q[b, gi])
                p = np.exp(logits - logits.max())
                p /= p.sum()
                out[b, gi] = p @ v
    append_decode(cache, k_bits, v_bits)
    return out


# ----------------------------------------------------------------------------- diagnostics ([AP] section 2)
def error_split(x, xhat) -> tuple[np.ndarray, np.ndarray]:
    """Magnitude and direction parts of eps = xhat - x ([AP] section 2, error equation):
    E_M = (|xhat| - |x|) x/|x|,  E_D = |xhat| (xhat/|xhat| - x/|x|).
    Conventions: |x| = 0 gives E_M = 0, E_D = xhat; |xhat| = 0 gives E_D = 0."""
    x = np.asarray(x, dtype=np.float64)
    xh = np.asarray(xhat, dtype=np.float64)
    nx = np.linalg.norm(x, axis=-1, keepdims=True)
    nxh = np.linalg.norm(xh, axis=-1, keepdims=True)
    ux = np.where(nx > 0, x / np.where(nx > 0, nx, 1), 0.0)
    uxh = np.where(nxh > 0, xh / np.where(nxh > 0, nxh, 1), 0.0)
    e_m = np.where(nx > 0, (nxh - nx) * ux, 0.0)
    e_d = np.where(nx > 0, np.where(nxh > 0, nxh * (uxh - ux), 0.0), xh)
    return e_m, e_d


def axis_mean_squares(y) -> tuple[np.ndarray, np.ndarray]:
    """Per-token and per-channel mean squares of a normalized tile y[..., G, D]."""
    y = np.asarray(y, dtype=np.float64)
    return np.mean(y * y, axis=-1), np.mean(y * y, axis=-2)


def relative_token_error(x, xhat) -> np.ndarray:
    """|xhat - x|^2 / |x|^2 per token (tokens with |x| = 0 give 0)."""
    x = np.asarray(x, dtype=np.float64)
    num = np.sum((np.asarray(xhat) - x) ** 2, axis=-1)
    den = np.sum(x * x, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), 0.0)
