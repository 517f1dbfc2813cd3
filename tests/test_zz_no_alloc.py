"""kvarn_attn_decode_noalloc (the attention without a caller workspace, for callers that
cannot allocate) against kvarn_attn_decode on the same caches: two calls in a row, the
second with a smaller geometry, each bit-identical to the workspace entry point's output and
within the attention bar (2e-3 of max |ref|) of the oracle on the GPU-written bytes.
Run on an MI355X: pytest -m gpu."""
import numpy as np
import pytest
import torch

from kv_cache_bit_amd import kvarn as K
from kv_cache_bit_amd import synth

from parity import GpuCache, check_attention, from_u16, gpu_prefill

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_entry_point_twice():
    for (B, H, Hq, T, cap, G, seed) in [(4, 2, 8, 1000, 1056, 32, 41), (2, 1, 4, 300, 320, 64, 42)]:
        print("[case] noalloc attention", B, H, Hq, T, G, flush=True)
        k, v = synth.kv_host(seed, B, T, H)
        gc = GpuCache(B, H, cap, G, 3 if G == 32 else 2)
        gpu_prefill(gc, k, v, T)
        q = from_u16(synth.q_host(seed + 1, B, Hq))
        ws, n = K.alloc_workspace(gc.g, Hq)
        ref = torch.full((B, Hq, 128), float("nan"), device="cuda")
        got = torch.full((B, Hq, 128), float("nan"), device="cuda")
        K.kvarn_attn_decode(gc.g, gc.buf, q, Hq, 0.0, 0, ws, n, ref)
        K.kvarn_attn_decode_noalloc(gc.g, gc.buf, q, Hq, 0.0, 0, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        check_attention(got.cpu().numpy().astype(np.float64), gc.host_cache(), synth.q_host(seed + 1, B, Hq), Hq)
