"""The host path of libkvarn (argument validation, geometry and layout arithmetic, workspace
sizes, the extension struct) under AddressSanitizer and UndefinedBehaviorSanitizer: a build
with both on its host code runs every case of tests/test_host_abi.py in a child process that
preloads the sanitizer runtime. Any report aborts the child. No GPU is needed: every call the
cases make is refused on the host before any HIP call."""
import os
import subprocess
import sys

from kv_cache_bit_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_cases_under_asan_and_ubsan(tmp_path):
    lib = build.build_sanitized(str(tmp_path / "libkvarn_san.so"))
    env = dict(os.environ, KVARN_LIB=lib, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_host_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out
    assert " passed" in out
