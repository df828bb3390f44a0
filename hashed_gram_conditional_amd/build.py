"""Build step of libengram.so (the layer) and libengram_calibrate.so (the
benchmark's MFMA calibration): compiles the HIP sources for gfx950 in-tree.

Run ``python hashed_gram_conditional_amd/build.py`` (or ``__graft_entry__.build()``).
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = ["hash.hip", "gather.hip", "hash_gather.hip", "gemm.hip", "gemm_mx.hip", "gate.hip",
           "conv.hip", "layout.hip", "engram_api.hip"]
LIB = os.path.join(PKG, "libengram.so")
CALIB_SOURCE = "calibrate.hip"
CALIB_LIB = os.path.join(PKG, "libengram_calibrate.so")

# Packed-fp32 instructions are disabled for every HIP translation unit.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C-ABI's host
# code (argument validation, prime search, workspace arithmetic); the device
# code is built as usual. Each -fsanitize= applies to the host pass only.
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-shared-libsan", "-g",
]


def sources():
    return [os.path.join(PKG, "csrc", s) for s in SOURCES]


def build_library(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    srcs = sources()
    tmp = out + ".tmp"
    flags = [f for f in HIP_FLAGS if not (sanitize and f == "-O3")]
    if sanitize:
        flags += ["-O1", *SANITIZE_FLAGS]
    cmd = [hipcc(), *flags, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {LIB}")
    os.replace(tmp, out)
    return out


def build_calibration(verbose: bool = False, out: str = CALIB_LIB) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-o", tmp, os.path.join(PKG, "csrc", CALIB_SOURCE)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {out}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_calibration(verbose=True))
