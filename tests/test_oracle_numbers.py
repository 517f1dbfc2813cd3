"""Pins of the oracle's number-format helpers against exact rational arithmetic.

fp16 rounding is the step that turns the oracle's fp64 scales into stored values,
so it is checked against an independent round-half-to-even written with Fractions
(IEEE 754 binary16: 10 fraction bits, emin = -14, subnormal spacing 2^-24).
"""
from fractions import Fraction
import math

import numpy as np

from oracle import kvarn_ref as R
from kv_cache_bit_amd import synth


def fp16_exact(x: float) -> float:
    """Round a double to binary16 with round-half-to-even using exact rationals."""
    if x == 0:
        return x
    sign = -1 if x < 0 else 1
    a = Fraction(abs(x))
    e = max(math.floor(math.log2(abs(x))), -14)
    # guard against log2 rounding at exact powers of two
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a and e >= -14:
        e += 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    n = a / ulp
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * ulp
    if v > 65504:
        return sign * math.inf
    return sign * float(v)


def test_fp16_round_against_rationals():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(2000) * np.exp(rng.uniform(-20, 12, 2000)))
    # exact ties at several binades, including the subnormal range
    for e in (-24, -20, -15, -14, -3, 0, 5, 14):
        ulp = 2.0 ** (max(e, -14) - 10) if e >= -14 else 2.0 ** -24
        for k in (1, 2, 3, 1023, 1024, 2047):
            vals += [(k + 0.5) * ulp * 2.0 ** 0, -(k + 0.5) * ulp]
    vals += [65504.0, 65519.0, 65519.999, 65520.0, 1e6, 2.0 ** -25, 2.0 ** -26 * 3, 5.960464477539063e-08]
    got = R.fp16_round(np.array(vals))
    want = np.array([fp16_exact(v) for v in vals])
    assert np.array_equal(got, want)


def test_fp16_saturate_flags():
    v, c = R.fp16_saturate(np.array([65504.0, 65505.0, -70000.0, 3.0]))
    assert v.tolist() == [65504.0, 65504.0, -65504.0, 3.0]
    assert c.tolist() == [False, True, True, False]


def test_bf16_decoding_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x4780, 0x477F, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    v = R.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 65536.0 and v[3] == 65280.0
    assert v[4] == 2.0 ** -133
    assert v[5] == (2 - 2 ** -7) * 2.0 ** 127
    assert v[6] == 0.0 and math.copysign(1, v[6]) == -1


def test_canonicalize_range_edges():
    # 2^16 = 0x4780 is kept; the next bf16 value, 2^16 (1 + 2^-7) = 0x4781, saturates to 2^16
    v, sat, _ = R.canonicalize(np.array([0x4780, 0xC780], dtype=np.uint16))
    assert v.tolist() == [65536.0, -65536.0] and not sat
    v, sat, _ = R.canonicalize(np.array([0x4781, 0xC7FF, 0x7F7F], dtype=np.uint16))
    assert v.tolist() == [65536.0, -65536.0, 65536.0] and sat
    v, sat, _ = R.canonicalize(np.array([0x477F, 0x3F80], dtype=np.uint16))
    assert v.tolist() == [65280.0, 1.0] and not sat
    # small values are kept as given, down to the smallest bf16 subnormal 2^-133 = 0x0001
    b = np.array([0x33C0, 0x0001, 0x8001, 0x0080, 0x0000, 0x8000], dtype=np.uint16)
    v, sat, nan = R.canonicalize(b)
    assert v.tolist() == [1.5 * 2.0 ** -24, 2.0 ** -133, -2.0 ** -133, 2.0 ** -126, 0.0, 0.0] and not sat and not nan
    assert math.copysign(1, v[5]) == -1
    # every finite bf16 value within +-2^16 is its own canonical value, and bf16_bits inverts
    rng = np.random.default_rng(2)
    b = synth.f32_to_bf16_bits((rng.standard_normal(5000) * np.exp(rng.uniform(-80, 10, 5000))).astype(np.float32))
    v = R.canonicalize(b)[0]
    assert np.array_equal(v, R.bf16_to_f64(b)) and np.array_equal(R.bf16_bits(v), b)


def test_synth_bf16_rounding_half_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even (1.0)
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    assert b.tolist() == [0x3F80, 0x3F82, 0xBF80]


def test_sign_vector_splitmix64_reference_values():
    # SplitMix64 seeded with 0: first outputs are published test values of the generator
    z = synth.splitmix64(0, 3)
    assert z == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    s = synth.sign_vector(0, 128)
    assert s.dtype == np.int8 and set(np.unique(s).tolist()) <= {-1, 1}
    assert s[0] == -1 and s[1] == 1 and s[2] == 1   # top bits of the three values above


def test_canonicalize_non_finite_inputs():
    """Infinities saturate like any value beyond +-2^16; a NaN (which the pages' finite
    tensors never hold) is stored as 0 and reported, so one NaN cannot poison a tile's
    scales: a prefill with a NaN raises FLAG_NAN and quantizes that element as a zero."""
    bits = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x3F80], dtype=np.uint16)  # +inf -inf nan -nan 1
    v, sat, nan = R.canonicalize(bits)
    assert v.tolist() == [65536.0, -65536.0, 0.0, 0.0, 1.0] and sat and nan
    v, sat, nan = R.canonicalize(np.array([0x3F80, 0xC000], dtype=np.uint16))
    assert not sat and not nan
    k, v2 = synth.kv_host(3, 1, 40, 1)
    k_nan = k.copy()
    k_nan[0, 5, 0, 17] = 0x7FC0
    k_zero = k.copy()
    k_zero[0, 5, 0, 17] = 0x0000
    a = R.Cache(R.Geom(1, 1, 128, 64, 32, 3, 2), synth.sign_vector(0))
    b = R.Cache(R.Geom(1, 1, 128, 64, 32, 3, 2), synth.sign_vector(0))
    R.quantize_prefill(a, k_nan, v2, 40)
    R.quantize_prefill(b, k_zero, v2, 40)
    assert a.flags == R.FLAG_NAN and b.flags == 0
    fl = R.FLAGS_OFFSET
    a.buf[fl:fl + 4] = 0
    assert np.array_equal(a.buf, b.buf)
