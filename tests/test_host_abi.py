"""Host-side checks of libkvarn that need no GPU: the library loads, exports every
entry point include/kvarn.h declares, sizes agree with the oracle's layout, and
every invalid argument is rejected with its status before any HIP call."""
import ctypes
import os
import re

import pytest

from kv_cache_bit_amd import kvarn as K
from oracle import kvarn_ref as R

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvarn.h")


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"KVARN_API\s+[\w\s\*]+?\b(kvarn_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 16
    for n in names:
        assert hasattr(K.lib, n), n
    assert sorted(K.EXPORTS) == names


def test_format_version_and_status_strings():
    assert K.kvarn_format_version() == R.VERSION == 3
    for s in range(7):
        assert K.status_str(s)
    assert K.status_str(99) == "unknown status"


@pytest.mark.parametrize("B,H,cap,G", [(1, 1, 32, 32), (2, 3, 96, 32), (1, 8, 32768, 32), (8, 8, 16384, 64),
                                       (32, 10, 17408, 32), (3, 5, 640, 64)])
def test_cache_bytes_match_oracle_layout(B, H, cap, G):
    assert K.kvarn_cache_bytes(K.geom(B, H, cap, G, 3)) == R.Geom(B, H, 128, cap, G, 3, 2).total


def test_bit_width_sizes_match_oracle():
    for bits in (2, 3, 4):
        for G in (32, 64):
            assert K.kvarn_cache_bytes(K.geom(2, 3, 256, G, 2, bits=bits)) == \
                R.Geom(2, 3, 128, 256, G, 2, bits).total


def test_paged_sizes_match_oracle():
    for B, H, cap, G, pages in [(2, 3, 256, 64, 7), (4, 8, 1024, 32, 100), (1, 1, 32, 32, 1)]:
        assert K.kvarn_cache_bytes(K.geom(B, H, cap, G, 2, num_pages=pages)) == \
            R.Geom(B, H, 128, cap, G, 2, 2, 0, pages).total


def test_variants_accepted():
    """Every combination of the four variant bits is a valid geometry, same size."""
    n0 = K.kvarn_cache_bytes(K.geom(2, 3, 256, 64, 2))
    for var in range(16):
        assert K.kvarn_cache_bytes(K.geom(2, 3, 256, 64, 2, variant=var)) == n0


def test_workspace_bytes():
    g = K.geom(32, 10, 17408, 32, 3)
    n = K.kvarn_attn_workspace_bytes(g, 40)
    # one partial (m, l, 2 pad, o[128]) per (b, q head, span); at this geometry a span holds
    # at most 4 waves x 16 tiles of the capacity, so 544 tiles give 9 spans; then len per
    # (b, kv head), 16-B padded
    assert n == 32 * 40 * 9 * (4 + 128) * 4 + 32 * 10 * 4
    with pytest.raises(K.KvarnError) as e:
        K.kvarn_attn_workspace_bytes(g, 41)
    assert e.value.status == K.KVARN_ERR_GEOM
    # any whole number of query heads per kv head: groups of 4 query heads per work-group
    assert K.kvarn_attn_workspace_bytes(K.geom(1, 1, 64, 32, 3), 9) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), K.KVARN_ERR_UNSUPPORTED),
    (dict(group=48), K.KVARN_ERR_UNSUPPORTED),
    (dict(bits=5), K.KVARN_ERR_UNSUPPORTED),
    (dict(bits=1), K.KVARN_ERR_UNSUPPORTED),
    (dict(varn_iters=9), K.KVARN_ERR_UNSUPPORTED),
    (dict(varn_iters=-1), K.KVARN_ERR_GEOM),
    (dict(capacity=100), K.KVARN_ERR_GEOM),
    (dict(capacity=0), K.KVARN_ERR_GEOM),
    (dict(batch=0), K.KVARN_ERR_GEOM),
    (dict(variant=16), K.KVARN_ERR_UNSUPPORTED),
    (dict(variant=-1), K.KVARN_ERR_UNSUPPORTED),
])
def test_geometry_rejected(kw, status):
    base = dict(batch=1, num_kv_heads=2, head_dim=128, capacity=128, group=32, varn_iters=3, bits=2, variant=0,
                num_pages=0)
    base.update(kw)
    g = K.geom(base.pop("batch"), base.pop("num_kv_heads"), base.pop("capacity"), **base)
    with pytest.raises(K.KvarnError) as e:
        K.kvarn_cache_bytes(g)
    assert e.value.status == status


def test_seven_field_geometry_is_the_base_of_the_extension():
    """kvarn_geom has exactly the seven int32 fields of the problem statement (28 bytes); the
    extension adds size, variant and num_pages after it, and is read only when the marker bit
    is set in bits. Without the bit, bytes past the seven fields are never read."""
    assert ctypes.sizeof(K.kvarn_geom) == 28
    assert [n for n, _ in K.kvarn_geom._fields_] == ["batch", "num_kv_heads", "head_dim", "capacity", "group",
                                                      "varn_iters", "bits"]
    assert ctypes.sizeof(K.kvarn_geom_ext) == 40 and K.kvarn_geom_ext.size.offset == 28
    plain = K.geom(2, 3, 256, 32, 3)
    assert isinstance(plain, K.kvarn_geom)
    # garbage after a plain struct does not matter: a buffer whose bytes 28.. say "paged"
    buf = (ctypes.c_int32 * 10)(2, 3, 128, 256, 32, 3, 2, 40, 0, 7)
    n = ctypes.c_size_t()
    assert K.lib.kvarn_cache_bytes(ctypes.addressof(buf), ctypes.byref(n)) == K.KVARN_OK
    assert n.value == K.kvarn_cache_bytes(plain) == R.Geom(2, 3, 128, 256, 32, 3, 2).total
    # the same bytes with the marker bit: read as an extension with 7 pages
    buf[6] = 2 | K.KVARN_GEOM_EXT
    assert K.lib.kvarn_cache_bytes(ctypes.addressof(buf), ctypes.byref(n)) == K.KVARN_OK
    assert n.value == R.Geom(2, 3, 128, 256, 32, 3, 2, 0, 7).total
    # an extension of the wrong size is refused
    buf[7] = 36
    assert K.lib.kvarn_cache_bytes(ctypes.addressof(buf), ctypes.byref(n)) == K.KVARN_ERR_GEOM
    ext = K.geom(2, 3, 256, 32, 3, variant=K.KVARN_VARIANT_CENTERED)
    assert isinstance(ext, K.kvarn_geom_ext) and ext.bits == 2 and ext.base.bits == 2 | K.KVARN_GEOM_EXT
    assert K.kvarn_cache_bytes(ext) == n.value - (R.Geom(2, 3, 128, 256, 32, 3, 2, 0, 7).total
                                                  - R.Geom(2, 3, 128, 256, 32, 3, 2).total)


# Fake device addresses: the calls below must fail validation before touching them.
A, A2, MIS = 0x10000, 0x20000, 0x10008


def _code(fn, *args):
    try:
        fn(*args)
    except K.KvarnError as e:
        return e.status
    return K.KVARN_OK


def test_argument_errors_return_before_any_launch():
    g = K.geom(1, 2, 128, 32, 3)
    signs = [1] * 128
    assert _code(K.kvarn_cache_init, g, 0, signs, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_cache_init, g, MIS, signs, 0) == K.KVARN_ERR_ALIGN
    assert _code(K.kvarn_cache_init, g, A, [1] * 127 + [0], 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_quantize_prefill, g, 0, A, A2, 10, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_quantize_prefill, g, A, 0, A2, 10, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_quantize_prefill, g, A, MIS, A2, 10, 0) == K.KVARN_ERR_ALIGN
    assert _code(K.kvarn_quantize_prefill, g, A, A, A2, 129, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_quantize_prefill, g, A, A, A2, -1, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_debug_prefill, g, A, A, A2, 64, MIS, None, None, None, 0) == K.KVARN_ERR_ALIGN
    assert _code(K.kvarn_append_decode, g, A, 0, A2, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_append_decode, g, A, A, MIS, 0) == K.KVARN_ERR_ALIGN
    assert _code(K.kvarn_dequantize, g, A, A, A2, 129, 0, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_dequantize, g, A, A, A2, 64, 7, 0) == K.KVARN_ERR_UNSUPPORTED
    assert _code(K.kvarn_dequantize, g, A, MIS, A2, 64, 0, 0) == K.KVARN_ERR_ALIGN
    # a geometry past the element-count limit (B * capacity * Hkv * D >= 2^40) is refused
    # before any launch, which also keeps every kernel's job count below 2^31
    huge = K.geom(1 << 16, 64, 1 << 16, 32, 3)
    assert _code(K.kvarn_dequantize, huge, A, A, A2, 1 << 16, 0, 0) == K.KVARN_ERR_RANGE
    ws = K.kvarn_attn_workspace_bytes(g, 4)
    assert _code(K.kvarn_attn_decode, g, A, A2, 4, 0.0, 0, A, ws - 1, A2, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_attn_decode, g, A, A2, 3, 0.0, 0, A, ws, A2, 0) == K.KVARN_ERR_GEOM
    assert _code(K.kvarn_attn_decode, g, A, A2, 4, 0.0, 8, A, ws, A2, 0) == K.KVARN_ERR_UNSUPPORTED
    assert _code(K.kvarn_attn_decode, g, A, A2, 4, float("nan"), 0, A, ws, A2, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_attn_decode, g, A, 0, 4, 0.0, 0, A, ws, A2, 0) == K.KVARN_ERR_NULL
    # multi-token append and the page map
    assert _code(K.kvarn_append_tokens, g, A, A, A2, 129, None, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_append_tokens, g, A, A, A2, -1, None, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_append_tokens, g, A, 0, A2, 3, None, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_append_tokens, g, A, MIS, A2, 3, None, 0) == K.KVARN_ERR_ALIGN
    assert _code(K.kvarn_append_tokens, g, A, A, A2, 3, A + 2, 0) == K.KVARN_ERR_ALIGN
    assert _code(K.kvarn_append_tokens, g, A, A, A2, 0, None, 0) == K.KVARN_OK   # nothing to do
    assert _code(K.kvarn_cache_set_pages, g, A, A2, 0, 1, 0) == K.KVARN_ERR_GEOM  # not paged
    gp = K.geom(2, 2, 128, 32, 3, num_pages=5)
    assert _code(K.kvarn_cache_set_pages, gp, A, A2, 3, 2, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_cache_set_pages, gp, A, A2, -1, 1, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_cache_set_pages, gp, A, 0, 0, 1, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_cache_set_pages, gp, A, A2 + 1, 0, 1, 0) == K.KVARN_ERR_ALIGN
    assert _code(K.kvarn_cache_set_pages, gp, A, A2, 4, 0, 0) == K.KVARN_OK
    assert _code(K.kvarn_cache_bytes, K.geom(2, 2, 128, 32, 3, num_pages=-1)) == K.KVARN_ERR_GEOM
    # fused decode step: the attention's checks plus the appended token's pointers
    assert _code(K.kvarn_append_attn_decode, g, A, A2, A2, A2, 4, 0.0, 0, A, ws - 1, A2, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_append_attn_decode, g, A, 0, A2, A2, 4, 0.0, 0, A, ws, A2, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_append_attn_decode, g, A, A2, MIS, A2, 4, 0.0, 0, A, ws, A2, 0) == K.KVARN_ERR_ALIGN
    assert _code(K.kvarn_append_attn_decode, g, 0, A2, A2, A2, 4, 0.0, 0, A, ws, A2, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_append_attn_decode, g, A, A2, A2, A2, 4, 0.0, 2, A, ws, A2, 0) == K.KVARN_ERR_UNSUPPORTED
    assert _code(K.kvarn_cache_flags, 0, 0) == K.KVARN_ERR_NULL
    # the no-allocation attention: its own size limit, then the attention's checks, all on the host
    big = K.geom(64, 8, 1 << 17, 32, 3)
    assert K.kvarn_attn_workspace_bytes(big, 64) > 32 << 20
    assert _code(K.kvarn_attn_decode_noalloc, big, A, A2, 64, 0.0, 0, A2, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_attn_decode_noalloc, g, 0, A2, 4, 0.0, 0, A2, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_attn_decode_noalloc, g, A, MIS, 4, 0.0, 0, A2, 0) == K.KVARN_ERR_ALIGN
    assert _code(K.kvarn_attn_decode_noalloc, g, A, A2, 3, 0.0, 0, A2, 0) == K.KVARN_ERR_GEOM
    assert _code(K.kvarn_attn_decode_noalloc, g, A, A2, 4, 0.0, 4, A2, 0) == K.KVARN_ERR_UNSUPPORTED
    bad = K.geom(1, 2, 100, 32, 3)
    assert _code(K.kvarn_quantize_prefill, bad, A, A, A2, 10, 0) == K.KVARN_ERR_GEOM
    # a launch of 2^32 or more work-items is refused (B * Hkv * T/G * 2 = 2^27 tiles)
    wide = K.geom(1024, 8, 1 << 18, 32, 3)
    assert _code(K.kvarn_quantize_prefill, wide, A, A, A2, 1 << 18, 0) == K.KVARN_ERR_RANGE
    # several layers in one call: the per-layer checks, the pointer arrays, distinct caches
    L3 = [A, A + 1024, A + 2048]
    assert _code(K.kvarn_quantize_prefill_layers, g, L3, [A2] * 3, [A2] * 3, 10, 0, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_quantize_prefill_layers, g, L3, [A2] * 3, [A2] * 3, 10, 0, 1025) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_quantize_prefill_layers, g, None, [A2] * 3, [A2] * 3, 10, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_quantize_prefill_layers, g, L3, None, [A2] * 3, 10, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_quantize_prefill_layers, g, [A, 0, A + 64], [A2] * 3, [A2] * 3, 10, 0) == K.KVARN_ERR_NULL
    assert _code(K.kvarn_quantize_prefill_layers, g, L3, [A2, MIS, A2], [A2] * 3, 10, 0) == K.KVARN_ERR_ALIGN
    assert _code(K.kvarn_quantize_prefill_layers, g, L3, [A2] * 3, [A2] * 3, 129, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_quantize_prefill_layers, g, [A, A + 1024, A], [A2] * 3, [A2] * 3, 10, 0) \
        == K.KVARN_ERR_GEOM
    assert _code(K.kvarn_quantize_prefill_layers, bad, L3, [A2] * 3, [A2] * 3, 10, 0) == K.KVARN_ERR_GEOM
    assert _code(K.kvarn_quantize_prefill_layers, wide, L3, [A2] * 3, [A2] * 3, 1 << 18, 0) == K.KVARN_ERR_RANGE
    assert _code(K.kvarn_cache_init, None if False else K.geom(1, 2, 128, 32, 3, head_dim=96), A, signs, 0) \
        == K.KVARN_ERR_UNSUPPORTED


def test_null_geometry():
    f = K.lib.kvarn_cache_bytes
    n = ctypes.c_size_t()
    assert f(None, ctypes.byref(n)) == K.KVARN_ERR_NULL


def test_one_hip_runtime_when_binding_loads_first():
    """Importing the binding before torch still leaves one HIP runtime in the process (the
    binding loads torch's before libkvarn): two runtimes make torch's own launches fail."""
    import subprocess
    import sys
    code = ("import kv_cache_bit_amd.kvarn, sys\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "paths = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
            "print(len(paths), 'torch' in sys.modules)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["1", "True"], out.stdout
