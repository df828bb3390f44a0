"""Build step of libworkloads.so, the device twin of the table generator."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libworkloads.so")


def build_generator(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = LIB + ".tmp"
    cmd = [os.path.join(rocm, "bin", "hipcc"), "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-fPIC", "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", tmp, os.path.join(HERE, "csrc", "table_gen.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {LIB}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_generator(verbose=True))
