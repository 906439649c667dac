"""Compile libtreeverify.so for gfx950 with hipcc (runs on a machine without a GPU too)."""

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libtreeverify.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # M0 is written only by the LDS-DMA inline asm in attn.hip (see lds_dma16)
    "-Wno-inline-asm",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


# the same sources with TV_PLAN_VARIANT=1: another work partition and order, the same
# results (tests compare the two builds bit for bit)
LIB_VARIANT = os.path.join(PKG, "libtreeverify_variant.so")


def _compile(out, extra, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), tmp, out


def build(verbose=False):
    """Compile every HIP source into the in-tree shared library (and its plan-variant
    twin); returns the library's path."""
    jobs = [_compile(LIB, [], verbose), _compile(LIB_VARIANT, ["-DTV_PLAN_VARIANT=1"], verbose)]
    for proc, tmp, out in jobs:
        _, err = proc.communicate()
        if proc.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + err[-8000:])
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
