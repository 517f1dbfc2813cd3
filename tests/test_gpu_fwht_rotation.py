"""GPU parity of the butterfly-rotation build (libkvarn_fwht.so) against the CPU oracle.

That build differs from libkvarn.so only in the rotation of the write path: a 128-point
fast Walsh-Hadamard transform on the VALU (register stages, permlane swaps across lanes)
instead of the matrix cores. It exists to measure the one against the other, so it must
compute the same method: asserted here through the same parity chain as the main build
(W, Y, scales, codes and bytes against the oracle), on full tiles with a tail, at G = 32
and 64, on the edge rows that take the checked rotation, and with prefill(T) equal byte
for byte to T single-token appends of the same build. Run on an MI355X: pytest -m gpu.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth

from parity import GpuCache, check_prefill, from_u16
from test_gpu_edge_rows import edge_rows_kv

pytestmark = pytest.mark.gpu

FWHT_LIB = os.path.join(os.path.dirname(os.path.abspath(K.__file__)), "libkvarn_fwht.so")


@pytest.fixture(scope="module")
def fwht():
    lib = ctypes.CDLL(FWHT_LIB)  # built next to libkvarn.so by the package's build step
    for n in ("kvarn_quantize_prefill", "kvarn_debug_prefill", "kvarn_append_decode", "kvarn_format_version"):
        getattr(lib, n).restype = ctypes.c_int
    assert lib.kvarn_format_version() == K.kvarn_format_version()
    return lib


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def fwht_prefill(lib, gc, k_bits, v_bits, T):
    """Prefill through the butterfly build, with its debug W and Y: (w, y) fp64 [2][B][Tf][H][D]."""
    k, v = from_u16(k_bits[:, :T]), from_u16(v_bits[:, :T])
    B, H = gc.og.batch, gc.og.num_kv_heads
    tf = (T // gc.og.group) * gc.og.group
    w = torch.full((2, B, max(tf, 1), H, 128), float("nan"), device="cuda")
    y = torch.full((2, B, max(tf, 1), H, 128), float("nan"), device="cuda")
    st = lib.kvarn_debug_prefill(ctypes.byref(gc.g), _ptr(gc.buf), _ptr(k), _ptr(v), T, _ptr(w[0]), _ptr(w[1]),
                                 _ptr(y[0]), _ptr(y[1]), _stream())
    assert st == 0, st
    torch.cuda.synchronize()
    return w.cpu().numpy().astype(np.float64), y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("G,n_it,T", [(32, 3, 250), (64, 2, 300)])
def test_fwht_prefill_parity(fwht, G, n_it, T):
    print("[case] butterfly prefill", G, n_it, T, flush=True)
    B, H = 1, 2
    k, v = synth.kv_host(31, B, T, H)
    gc = GpuCache(B, H, (T // G + 1) * G, G, n_it)
    w, y = fwht_prefill(fwht, gc, k, v, T)
    check_prefill(gc, k, v, T, w, y)


@pytest.mark.parametrize("G,n_it", [(32, 3), (64, 2)])
def test_fwht_edge_rows_and_appends(fwht, G, n_it):
    """Zero rows, small rows and rows whose squares underflow fp32 (the checked rotation),
    then the same tokens through single-token appends of the same build: equal bytes."""
    print("[case] butterfly edge rows + appends", G, n_it, flush=True)
    B, H = 1, 2
    T = 2 * G + 5
    k, v = edge_rows_kv(11, B, T, H, 2 * G)
    cap = (T // G + 1) * G
    gc = GpuCache(B, H, cap, G, n_it)
    fwht_prefill(fwht, gc, k, v, T)
    check_prefill(gc, k, v, T)
    ap = GpuCache(B, H, cap, G, n_it)
    kd, vd = from_u16(k), from_u16(v)
    assert fwht.kvarn_quantize_prefill(ctypes.byref(ap.g), _ptr(ap.buf), _ptr(kd), _ptr(vd), 0, _stream()) == 0
    for t in range(T):
        assert fwht.kvarn_append_decode(ctypes.byref(ap.g), _ptr(ap.buf), _ptr(kd[:, t].contiguous()),
                                        _ptr(vd[:, t].contiguous()), _stream()) == 0
    ha, hb = gc.host_cache(), ap.host_cache()
    m = ha.defined_mask()
    assert np.array_equal(ha.buf[m], hb.buf[m])
