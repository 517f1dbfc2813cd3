"""Build libkvarn.so in-tree with hipcc for gfx950.

Usage: python -m kv_cache_bit_amd.build   (or kv_cache_bit_amd.build.build())
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "quantize.hip", "dequant.hip", "attn.hip"]
LIB = os.path.join(HERE, "libkvarn.so")
# a measurement kernel of the benchmark (streaming reads and writes), kept out of libkvarn
BENCH_SOURCES = ["stream_mix.hip"]
BENCH_LIB = os.path.join(HERE, "libkvarn_bench.so")
# the same library with the rotation as a VALU butterfly instead of the matrix cores, built
# only to measure the one against the other (KVARN_LIB=<this file> selects it in the binding)
FWHT_LIB = os.path.join(HERE, "libkvarn_fwht.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared", "-fvisibility=hidden",
    # packed FP32 arithmetic off: plain v_fma_f32 / v_mul_f32 only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results straight into VGPRs: the VALU reads them without v_accvgpr_read copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(sources, lib, verbose, defines=()):
    tmp = lib + ".tmp"
    cmd = [hipcc(), *FLAGS, *defines, *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, lib)


SANITIZE = [  # host code only; the GPU code is built as usual
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-shared-libasan", "-g", "-O1",
]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime a process must preload to load a sanitized build."""
    import glob
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return hits[-1]


def build_sanitized(out: str, verbose: bool = False) -> str:
    """libkvarn with AddressSanitizer and UndefinedBehaviorSanitizer on its host code (argument
    validation, layout and workspace arithmetic), for the CPU tests of the host path."""
    cmd = [hipcc(), *[f for f in FLAGS if f != "-O3"], *SANITIZE, *[os.path.join(CSRC, s) for s in SOURCES],
           "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc (sanitized) failed ({res.returncode}):\n{res.stderr}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source into kv_cache_bit_amd/libkvarn.so (and the benchmark's
    measurement kernel into libkvarn_bench.so, the butterfly-rotation build into
    libkvarn_fwht.so); returns the library's path."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [(SOURCES, LIB, ()), (BENCH_SOURCES, BENCH_LIB, ()),
            (SOURCES, FWHT_LIB, ("-DKVARN_ROTATION_BUTTERFLY=1",))]
    with ThreadPoolExecutor(len(jobs)) as ex:  # independent hipcc processes
        for f in [ex.submit(_compile, s, lib, verbose, d) for s, lib, d in jobs]:
            f.result()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
