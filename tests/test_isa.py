"""The generated gfx950 code of libkvarn has no MFMA whose destination overlaps its
A or B operand (such an MFMA reads partially overwritten rows on this hardware).
Compiles the sources with hipcc (no GPU needed)."""
import shutil

import pytest

from kv_cache_bit_amd import isa_check


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="hipcc not installed")
def test_no_mfma_operand_aliasing():
    assert isa_check.main() == 0


def test_checker_flags_aliasing():
    bad = "k:\n  v_mfma_f32_16x16x32_f16 v[0:3], v[2:5], v[6:9], v[10:13]\n"
    good = "k:\n  v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], v[0:3]\n"
    assert isa_check.check_asm(bad) and not isa_check.check_asm(good)


def test_checker_flags_scratch_and_calls():
    spill = "k:\n  v_add_f32 v0, v1, v2\n; ScratchSize: 736\n"
    call = "k:\n  s_swappc_b64 s[30:31], s[4:5]\n; ScratchSize: 0\n"
    clean = "k:\n  v_add_f32 v0, v1, v2\n; ScratchSize: 0\n"
    assert isa_check.check_resources(spill) and isa_check.check_resources(call)
    assert not isa_check.check_resources(clean)
