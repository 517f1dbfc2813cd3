"""ctypes binding of libkvarn (include/kvarn.h): same names, argument marshalling only.

Tensors are torch device tensors (memory and streams come from PyTorch); every
computation happens in the HIP kernels of libkvarn.so. If the library has not been
built, importing this module raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KVARN_LIB selects another build of the same library (the sanitized host build of the tests)
LIB_PATH = os.environ.get("KVARN_LIB") or os.path.join(HERE, "libkvarn.so")

KVARN_OK, KVARN_ERR_NULL, KVARN_ERR_ALIGN, KVARN_ERR_GEOM = 0, 1, 2, 3
KVARN_ERR_UNSUPPORTED, KVARN_ERR_RANGE, KVARN_ERR_DEVICE = 4, 5, 6
KVARN_OUT_F32, KVARN_OUT_BF16 = 0, 1
KVARN_Q_PREROTATED = 1
KVARN_FLAG_CAPACITY, KVARN_FLAG_SATURATED, KVARN_FLAG_SCALE_CLAMPED, KVARN_FLAG_UNMAPPED = 1, 2, 4, 8
KVARN_VARIANT_NO_ROTATION, KVARN_VARIANT_NO_CHANNEL_PASS, KVARN_VARIANT_NO_TOKEN_PASS = 1, 2, 4
KVARN_VARIANT_CENTERED = 8

EXPORTS = ("kvarn_format_version", "kvarn_cache_bytes", "kvarn_cache_init", "kvarn_quantize_prefill",
           "kvarn_append_decode", "kvarn_dequantize", "kvarn_attn_workspace_bytes", "kvarn_attn_decode",
           "kvarn_cache_flags", "kvarn_status_str", "kvarn_debug_prefill", "kvarn_append_attn_decode",
           "kvarn_append_tokens", "kvarn_cache_set_pages", "kvarn_attn_decode_noalloc",
           "kvarn_quantize_prefill_layers")
KVARN_MAX_PREFILL_LAYERS = 1024


class KvarnError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)} (status {status})")


KVARN_GEOM_EXT = 0x10000
KVARN_FLAG_NAN = 16
_BASE_FIELDS = ("batch", "num_kv_heads", "head_dim", "capacity", "group", "varn_iters", "bits")


class kvarn_geom(ctypes.Structure):
    """The seven-field geometry of include/kvarn.h (variant 0, records per sequence)."""
    _fields_ = [(n, ctypes.c_int32) for n in _BASE_FIELDS]
    variant = 0
    num_pages = 0

    def __repr__(self):
        return "kvarn_geom(" + ", ".join(f"{n}={getattr(self, n)}" for n in _BASE_FIELDS) + ")"


class kvarn_geom_ext(ctypes.Structure):
    """kvarn_geom plus the ablation variant and the page pool (KVARN_GEOM_EXT in base.bits)."""
    _fields_ = [("base", kvarn_geom), ("size", ctypes.c_uint32), ("variant", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]

    def __getattr__(self, name):  # batch, group, ... read through to the base fields
        if name in _BASE_FIELDS:
            v = getattr(self.base, name)
            return v & ~KVARN_GEOM_EXT if name == "bits" else v
        raise AttributeError(name)

    def __repr__(self):
        return (f"kvarn_geom_ext({self.base!r}, size={self.size}, variant={self.variant}, "
                f"num_pages={self.num_pages})")


def geom(batch, num_kv_heads, capacity, group=32, varn_iters=3, head_dim=128, bits=2, variant=0,
         num_pages=0):
    """A kvarn_geom, or a kvarn_geom_ext when a variant or a page pool is asked for."""
    base = kvarn_geom(batch, num_kv_heads, head_dim, capacity, group, varn_iters, bits)
    if variant == 0 and num_pages == 0:
        return base
    base.bits = bits | KVARN_GEOM_EXT
    return kvarn_geom_ext(base, ctypes.sizeof(kvarn_geom_ext), variant, num_pages)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -m kv_cache_bit_amd.build)")
    # torch ships its own HIP runtime (soname libamdhip64.so.7, file name without the .7):
    # loaded first, it is the one libkvarn binds to; loaded after libkvarn, a second runtime
    # comes in beside /opt/rocm's and torch's own kernels fail to launch.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, G, S, I32, U32, F32 = (ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                              ctypes.c_int32, ctypes.c_uint32, ctypes.c_float)
    sig = {
        "kvarn_format_version": ([], ctypes.c_int),
        "kvarn_cache_bytes": ([G, S], ctypes.c_int),
        "kvarn_cache_init": ([G, P, P, P], ctypes.c_int),
        "kvarn_quantize_prefill": ([G, P, P, P, I32, P], ctypes.c_int),
        "kvarn_quantize_prefill_layers": ([G, I32, P, P, P, I32, P], ctypes.c_int),
        "kvarn_append_decode": ([G, P, P, P, P], ctypes.c_int),
        "kvarn_dequantize": ([G, P, P, P, I32, I32, P], ctypes.c_int),
        "kvarn_attn_workspace_bytes": ([G, I32, S], ctypes.c_int),
        "kvarn_attn_decode": ([G, P, P, I32, F32, U32, P, ctypes.c_size_t, P, P], ctypes.c_int),
        "kvarn_append_attn_decode": ([G, P, P, P, P, I32, F32, U32, P, ctypes.c_size_t, P, P], ctypes.c_int),
        "kvarn_attn_decode_noalloc": ([G, P, P, I32, F32, U32, P, P], ctypes.c_int),
        "kvarn_append_tokens": ([G, P, P, P, I32, P, P], ctypes.c_int),
        "kvarn_cache_set_pages": ([G, P, P, I32, I32, P], ctypes.c_int),
        "kvarn_cache_flags": ([P, P, ctypes.POINTER(ctypes.c_uint32)], ctypes.c_int),
        "kvarn_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "kvarn_debug_prefill": ([G, P, P, P, I32, P, P, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


lib = _load()


# ----------------------------------------------------------------------------- marshalling helpers
def _g(g) -> int | None:
    """Address of a kvarn_geom or kvarn_geom_ext (both are passed as const kvarn_geom*)."""
    return None if g is None else ctypes.addressof(g)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, fn: str):
    if status != KVARN_OK:
        raise KvarnError(status, fn)


def status_str(status: int) -> str:
    return lib.kvarn_status_str(status).decode()


# ----------------------------------------------------------------------------- the C ABI, by name
def kvarn_format_version() -> int:
    return lib.kvarn_format_version()


def kvarn_cache_bytes(g: kvarn_geom) -> int:
    n = ctypes.c_size_t()
    _check(lib.kvarn_cache_bytes(_g(g), ctypes.byref(n)), "kvarn_cache_bytes")
    return n.value


def kvarn_cache_init(g: kvarn_geom, cache, signs, stream=None) -> None:
    import numpy as np
    s = np.ascontiguousarray(signs, dtype=np.int8)
    _check(lib.kvarn_cache_init(_g(g), _ptr(cache), s.ctypes.data, _stream(stream)), "kvarn_cache_init")


def kvarn_quantize_prefill(g: kvarn_geom, cache, k, v, num_tokens: int, stream=None) -> None:
    _check(lib.kvarn_quantize_prefill(_g(g), _ptr(cache), _ptr(k), _ptr(v), num_tokens, _stream(stream)),
           "kvarn_quantize_prefill")


def _ptr_array(items):
    """A host array of device pointers (void* const*), or None for None."""
    if items is None:
        return None
    return (ctypes.c_void_p * max(1, len(items)))(*[_ptr(t) for t in items])


def kvarn_quantize_prefill_layers(g: kvarn_geom, caches, ks, vs, num_tokens: int, stream=None,
                                  n_layers: int | None = None) -> None:
    """caches, ks, vs: sequences of device tensors (or addresses), one per layer; n_layers
    defaults to len(caches)."""
    if n_layers is None:
        n_layers = len(caches) if caches is not None else len(ks or vs or ())
    n = n_layers
    ca, ka, va = _ptr_array(caches), _ptr_array(ks), _ptr_array(vs)
    _check(lib.kvarn_quantize_prefill_layers(_g(g), n, ca, ka, va, num_tokens, _stream(stream)),
           "kvarn_quantize_prefill_layers")


def kvarn_debug_prefill(g: kvarn_geom, cache, k, v, num_tokens: int, w_k=None, w_v=None, y_k=None, y_v=None,
                        stream=None) -> None:
    _check(lib.kvarn_debug_prefill(_g(g), _ptr(cache), _ptr(k), _ptr(v), num_tokens, _ptr(w_k),
                                   _ptr(w_v), _ptr(y_k), _ptr(y_v), _stream(stream)), "kvarn_debug_prefill")


def kvarn_append_decode(g: kvarn_geom, cache, k, v, stream=None) -> None:
    _check(lib.kvarn_append_decode(_g(g), _ptr(cache), _ptr(k), _ptr(v), _stream(stream)),
           "kvarn_append_decode")


def kvarn_dequantize(g: kvarn_geom, cache, k_out, v_out, max_tokens: int, out_dtype: int = KVARN_OUT_F32,
                     stream=None) -> None:
    _check(lib.kvarn_dequantize(_g(g), _ptr(cache), _ptr(k_out), _ptr(v_out), max_tokens, out_dtype,
                                _stream(stream)), "kvarn_dequantize")


def kvarn_attn_workspace_bytes(g: kvarn_geom, num_q_heads: int) -> int:
    n = ctypes.c_size_t()
    _check(lib.kvarn_attn_workspace_bytes(_g(g), num_q_heads, ctypes.byref(n)),
           "kvarn_attn_workspace_bytes")
    return n.value


def kvarn_attn_decode(g: kvarn_geom, cache, q, num_q_heads: int, softmax_scale: float, flags: int, workspace,
                      workspace_bytes: int, out, stream=None) -> None:
    _check(lib.kvarn_attn_decode(_g(g), _ptr(cache), _ptr(q), num_q_heads, softmax_scale, flags,
                                 _ptr(workspace), workspace_bytes, _ptr(out), _stream(stream)), "kvarn_attn_decode")


def kvarn_attn_decode_noalloc(g: kvarn_geom, cache, q, num_q_heads: int, softmax_scale: float, flags: int, out,
                              stream=None) -> None:
    _check(lib.kvarn_attn_decode_noalloc(_g(g), _ptr(cache), _ptr(q), num_q_heads, softmax_scale, flags, _ptr(out),
                                         _stream(stream)), "kvarn_attn_decode_noalloc")


def kvarn_append_attn_decode(g: kvarn_geom, cache, k, v, q, num_q_heads: int, softmax_scale: float, flags: int,
                             workspace, workspace_bytes: int, out, stream=None) -> None:
    _check(lib.kvarn_append_attn_decode(_g(g), _ptr(cache), _ptr(k), _ptr(v), _ptr(q), num_q_heads,
                                        softmax_scale, flags, _ptr(workspace), workspace_bytes, _ptr(out),
                                        _stream(stream)), "kvarn_append_attn_decode")


def kvarn_append_tokens(g: kvarn_geom, cache, k, v, num_tokens: int, counts=None, stream=None) -> None:
    _check(lib.kvarn_append_tokens(_g(g), _ptr(cache), _ptr(k), _ptr(v), num_tokens, _ptr(counts),
                                   _stream(stream)), "kvarn_append_tokens")


def kvarn_cache_set_pages(g: kvarn_geom, cache, pages, tile_first: int, num_tiles: int, stream=None) -> None:
    _check(lib.kvarn_cache_set_pages(_g(g), _ptr(cache), _ptr(pages), tile_first, num_tiles,
                                     _stream(stream)), "kvarn_cache_set_pages")


def kvarn_cache_flags(cache, stream=None) -> int:
    f = ctypes.c_uint32()
    _check(lib.kvarn_cache_flags(_ptr(cache), _stream(stream), ctypes.byref(f)), "kvarn_cache_flags")
    return f.value


# ----------------------------------------------------------------------------- conveniences
def alloc_cache(g: kvarn_geom, signs, device="cuda", stream=None):
    """A torch uint8 buffer sized for g, with its header written."""
    import torch
    buf = torch.empty(kvarn_cache_bytes(g), dtype=torch.uint8, device=device)
    kvarn_cache_init(g, buf, signs, stream)
    return buf


def alloc_workspace(g: kvarn_geom, num_q_heads: int, device="cuda"):
    import torch
    n = kvarn_attn_workspace_bytes(g, num_q_heads)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device), n
