"""Build libhclrmix.so (HIP, gfx950) in-tree with hipcc.

Every translation unit is compiled with -ffp-contract=off (a multiply and an
add stay separately rounded unless written as fmaf), without packed-fp32
instructions, and for gfx950 only.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhclrmix.so")
# Measurement kernels (achievable HBM and matrix-core peaks), loaded by bench.py only.
PEAKS_LIB = os.path.join(HERE, "libhcpeaks.so")
PEAKS_SOURCES = ["hc_peaks.hip"]

SOURCES = ["hc_api.cpp", "hc_generic.hip", "hc_decode.hip", "hc_prefill.hip", "hc_invrms.hip", "hc_pad.hip"]
HEADERS = ["hc_device.h", "hc_internal.h", "hc_mfma_common.h"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wshadow", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(c) and os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err and verbose:
        print(err)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Builds libhclrmix.so and the measurement library libhcpeaks.so; returns the former's path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PEAKS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
