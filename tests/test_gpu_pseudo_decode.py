"""The synthetic pseudo-decode harness on a small random decoder, through the library's
kernels. Asserted: every statistic is finite; while every token is still in the bf16 tail
(steps 0..30) the quantized runs match the exact one (KL below 1e-6, attention output
within 1e-4, the same top-1 token); at step 31, where the first group is quantized, the
attention output moves by more than 1e-3. The mean KL of the full method and of
Hadamard-only after step 64 is printed, not asserted: on this small random decoder the
full method is not reliably the closer one. The pairwise test asserts how VarN changes the
error of an outlier token (its docstring).
"""
import numpy as np
import pytest

from kv_cache_bit_amd import pseudo_decode as P

pytestmark = pytest.mark.gpu


def test_pseudo_decode_small():
    print("[case] pseudo-decode small", flush=True)
    stats, cfg = P.run(steps=192, B=2, layers=2, hq=8, hkv=2, group=32, seed=3,
                       variants=["kvarn", "hadamard_only"], log_every=0)
    for name, st in stats.items():
        for m, x in st.items():
            assert np.all(np.isfinite(x)), (name, m)
        # steps 0..30 read the bf16 tail only (the inputs as given); step 31
        # completes the first group, which the append quantizes before the attention
        assert st["pd_kl"][:31].max() < 1e-6, (name, st["pd_kl"][:31].max())
        assert st["pd_attn"][:31].max() < 1e-4, (name, st["pd_attn"][:31].max())
        assert np.all(st["pd_top1"][:31] == 1.0)
        assert st["pd_attn"][31] > 1e-3
    for mode in ("pd", "par"):
        a = stats["kvarn"][mode + "_kl"][64:].mean()
        b = stats["hadamard_only"][mode + "_kl"][64:].mean()
        print("[case]", mode, "kl kvarn", a, "hadamard only", b, flush=True)


def test_pairwise_small():
    """VarN makes the quantizer blind to a token's scale: the full method's relative
    errors do not move when one token per tile is made 32 times larger, while
    Hadamard-only keeps that token almost exact (it sets the grid's ends) and garbles the
    normal tokens (error above their own norm)."""
    print("[case] pairwise small", flush=True)
    res = P.pairwise(ratios=(1, 32), tiles=64, group=32, seed=1, variants=("kvarn", "hadamard_only"))
    print("[case]", res, flush=True)
    k1, k32 = res["kvarn"][1], res["kvarn"][32]
    h1, h32 = res["hadamard_only"][1], res["hadamard_only"][32]
    assert abs(k32["rel_err_normal"] / k1["rel_err_normal"] - 1) < 0.02
    assert abs(k32["rel_err_outlier"] / k1["rel_err_outlier"] - 1) < 0.1
    assert k32["rel_err_normal"] < 0.4 and k32["rel_err_outlier"] < 0.4
    assert h32["rel_err_normal"] > 1.0 > 0.5 > h1["rel_err_normal"]
    assert h32["rel_err_outlier"] < 0.05
