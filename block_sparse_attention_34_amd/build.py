"""Builds libabsa.so (the HIP kernels and the C ABI) for gfx950 in-tree.

Usage: ``python -m block_sparse_attention_34_amd.build`` or ``build()``.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["absa_api.hip", "absa_select.hip", "absa_attend.hip", "absa_attend_pp.hip", "absa_fp8.hip"]
LIB = os.path.join(PKG, "libabsa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms stay off: plain fp32 code is what the kernels rely on
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # a kernel whose host-side launch stub went missing fails here, not at load time
    "-Wl,--no-undefined",
]


def hipcc_path() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; ROCm is required to build libabsa.so")
    return p


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libabsa.so next to this file; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc_path()] + HIPCC_FLAGS + ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                                          "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr[-8000:])
    os.replace(tmp, LIB)
    return LIB


def build_test_probe(src: str, out: str) -> str:
    """Compile one test-support HIP source (not part of the library) into a shared object."""
    tmp = out + ".tmp"
    cmd = [hipcc_path()] + HIPCC_FLAGS + ["-o", tmp, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr[-8000:])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
