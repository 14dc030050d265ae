"""Builds the in-tree HIP libraries for gfx950: overlap_attention_amd/libmkra.so (the
ring-attention path and the AllGather+GEMM path) and libmkra_probes.so (measurement
probes that bench.py runs).

Usage: python -m overlap_attention_amd.build   (or overlap_attention_amd.build.build())
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmkra.so")
SOURCES = [os.path.join(HERE, "csrc", n) for n in ("mkra_kernel.hip", "mkra_api.cpp", "mkag_kernel.hip", "mkag_api.cpp")]
KERNEL_SOURCES = [SOURCES[0], SOURCES[2]]
PROBES_LIB = os.path.join(HERE, "libmkra_probes.so")
PROBES_SOURCES = [os.path.join(HERE, "csrc", "mkra_probes.hip")]

# All HIP code is built without packed-FP32 instructions.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _build_one(sources, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc()] + FLAGS + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("building %s failed" % os.path.basename(lib))
    os.replace(tmp, lib)


def device_asm(out_path: str, source: str = SOURCES[0]) -> str:
    """gfx950 assembly of one HIP source (device code only), for build checks."""
    flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [hipcc()] + flags + ["--cuda-device-only", "-S", source, "-o", out_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("assembling %s failed" % os.path.basename(source))
    return open(out_path).read()


def build(verbose: bool = False) -> str:
    _build_one(SOURCES, LIB, verbose)
    _build_one(PROBES_SOURCES, PROBES_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
