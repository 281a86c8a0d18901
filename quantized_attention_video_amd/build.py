"""Build libsattn.so (the C-ABI library of include/sattn.h) in-tree with hipcc for gfx950.

Usage: python -m quantized_attention_video_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsattn.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("api.hip", "quant.hip", "attn.hip")]
FLAGS = [
    "-O3",
    "--offload-arch=gfx950",
    "-std=c++20",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-ffp-contract=off",  # every FP32 rounding step is written out; FMAs are explicit
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",  # no packed FP32 VALU ops
    "-Wall",
]


def build(verbose=False):
    """Compile every HIP source into LIB (atomically replaced); raises on failure."""
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"), *SOURCES,
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln and "--hip-link" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


C_DRIVER_SRC = os.path.join(ROOT, "tests", "c_abi_driver.cpp")
C_DRIVER = os.path.join(ROOT, "tests", "c_abi_driver")


def build_c_driver(verbose=False):
    """Compile the test program that calls the library through include/sattn.h alone (host
    code, linked against LIB with a path relative to itself)."""
    tmp = C_DRIVER + ".tmp"
    cmd = ["hipcc", "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"), C_DRIVER_SRC, "-L", HERE,
           "-lsattn", "-Wl,-rpath,$ORIGIN/../quantized_attention_video_amd", "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "--hip-link" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc (C ABI test driver) failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, C_DRIVER)
    return C_DRIVER


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_driver(verbose=True))
