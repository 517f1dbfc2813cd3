"""The boundary from C: tests/c_abi_check.c is compiled with gcc as strict C99 against
include/kvarn.h, linked to the built libkvarn.so and run (host-only calls: sizes, status
strings, argument checks). The sizes it prints match the oracle's layout."""
import os
import shutil
import subprocess

import pytest

from kv_cache_bit_amd import kvarn as K
from oracle import kvarn_ref as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def c_results(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_check")
    libdir = os.path.dirname(K.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
           "-L", libdir, "-l:libkvarn.so", f"-Wl,-rpath,{libdir}", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    out = {}
    for line in run.stdout.splitlines():
        k, v = line.split(" ", 1)
        out[k] = v
    return out


def test_c_caller_sees_every_entry_point(c_results):
    assert int(c_results["entry_points"]) == len(K.EXPORTS)
    assert int(c_results["format_version"]) == 3


def test_c_caller_sizes_match_oracle_and_binding(c_results):
    og = R.Geom(32, 10, 128, 17408, 32, 3, 2)
    assert int(c_results["cache_bytes_status"]) == K.KVARN_OK
    assert int(c_results["cache_bytes"]) == og.total
    assert int(c_results["workspace_status"]) == K.KVARN_OK
    assert int(c_results["workspace_bytes"]) == K.kvarn_attn_workspace_bytes(K.geom(32, 10, 17408), 40)


def test_c_caller_with_the_seven_field_struct(c_results):
    """A caller written to the seven-field geometry gets defined results: the struct is 28
    bytes, and the library reads no byte past it (the C caller surrounds it with a sentinel
    that would select a paged layout if it were read)."""
    assert int(c_results["sizeof_geom"]) == 28
    assert int(c_results["sizeof_geom_ext"]) == 40
    assert int(c_results["boxed_status"]) == K.KVARN_OK
    assert int(c_results["boxed_bytes"]) == R.Geom(32, 10, 128, 17408, 32, 3, 2).total
    assert int(c_results["ext_status"]) == K.KVARN_OK
    assert int(c_results["ext_bytes"]) == R.Geom(32, 10, 128, 17408, 32, 3, 2, 0, 100).total
    assert int(c_results["ext_badsize_status"]) == K.KVARN_ERR_GEOM


def test_c_caller_gets_host_side_errors(c_results):
    assert int(c_results["bits5_status"]) == K.KVARN_ERR_UNSUPPORTED
    assert int(c_results["group48_status"]) in (K.KVARN_ERR_GEOM, K.KVARN_ERR_UNSUPPORTED)
    assert int(c_results["null_geom_status"]) == K.KVARN_ERR_NULL
    assert int(c_results["null_out_status"]) == K.KVARN_ERR_NULL
    assert int(c_results["gqa_not_multiple_status"]) == K.KVARN_ERR_GEOM
    assert int(c_results["prefill_null_cache_status"]) == K.KVARN_ERR_NULL
    assert int(c_results["layers_null_status"]) == K.KVARN_ERR_NULL
    assert int(c_results["layers_duplicate_status"]) == K.KVARN_ERR_GEOM
    assert int(c_results["layers_count_status"]) == K.KVARN_ERR_RANGE
    assert c_results["status_str_ok"] == K.status_str(K.KVARN_OK)
    assert c_results["status_str_geom"] == K.status_str(K.KVARN_ERR_GEOM)
