"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
a copy of the library whose host pass is instrumented (device code as usual)
runs the host-only ABI tests and a randomized sweep of the host entry points
(argument validation, the prime search, the token-map check, workspace sizes)
in a child process that preloads the sanitizer runtime. Any report fails it."""
import glob
import hashlib
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT_DIR = os.path.join(ROOT, "_build", "asan")
OUT = os.path.join(OUT_DIR, "libengram.so")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def _runtime():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


pytestmark = [
    pytest.mark.skipif(_gpu_visible(), reason="host-only: fake device pointers"),
    pytest.mark.skipif(_runtime() is None, reason="no clang ASan runtime in this ROCm"),
]


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_engram_build_asan", os.path.join(ROOT, "hashed_gram_conditional_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def sanitized_library():
    b = _build_module()
    h = hashlib.sha256()
    for src in b.sources() + [os.path.join(ROOT, "include", "engram.h"),
                              os.path.join(ROOT, "hashed_gram_conditional_amd", "build.py")]:
        h.update(open(src, "rb").read())
    stamp = os.path.join(OUT_DIR, "sources.sha256")
    if not (os.path.exists(OUT) and os.path.exists(stamp) and
            open(stamp).read() == h.hexdigest()):
        os.makedirs(OUT_DIR, exist_ok=True)
        b.build_library(out=OUT, sanitize=True)
        with open(stamp, "w") as f:
            f.write(h.hexdigest())
    return OUT


def _env(lib):
    env = dict(os.environ)
    env.update(LD_PRELOAD=_runtime(), ENGRAM_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=97",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=98")
    return env


SWEEP = r'''
import ctypes, numpy as np
import hashed_gram_conditional_amd as E
L = E.LIB
rng = np.random.default_rng(7)
assert "_build/asan" in E.LIB_PATH
for _ in range(300):
    base = int(rng.integers(-5, 1 << 33))
    count = int(rng.integers(-3, 60))
    try:
        E.engram_make_primes(base, count)
    except (E.EngramError, ValueError, OverflowError):
        pass
    try:
        E.engram_make_layer_primes(max(base, 2) % (1 << 31), int(rng.integers(-1, 6)),
                                   int(rng.integers(-1, 30)))
    except (E.EngramError, ValueError, OverflowError):
        pass
for _ in range(200):
    V = int(rng.integers(1, 3000))
    Vp = int(rng.integers(1, V + 5))
    tm = rng.integers(-3, Vp + 3, V).astype(np.int32)
    E.engram_check_token_map(tm, V, Vp)
tm = np.arange(97, dtype=np.int32)
for _ in range(400):
    B, T = int(rng.integers(-2, 1 << 20)), int(rng.integers(-2, 1 << 20))
    hc, dim = int(rng.integers(-1, 10)), int(rng.integers(-8, 9000))
    p, off, _ = E.engram_make_primes(1009, 6)
    params = E.hash_params(97, 97, 4, 2, 0, 0x1000, [1, 3, 5, 7], p, off)
    d = E.forward_desc(B, T, hc, dim, int(rng.integers(-1, 1 << 40)), int(rng.integers(0, 3)),
                       int(rng.integers(0, 300)), 1e-6, 0.0,
                       wkv_ld=int(rng.integers(-8, 1 << 21)))
    L.engram_forward_workspace_size(ctypes.byref(params), ctypes.byref(d))
    L.engram_forward_static(ctypes.byref(params), ctypes.byref(d), 0x1000, None, None, 0x2000,
                            0x3000, 0x4000, 0x5000, 0x6000, None, None)
    L.engram_gate_conv_workspace_size(ctypes.byref(d))
    L.engram_transpose(0x1000, 1 << 44, int(rng.integers(-2, 1 << 40)),
                       int(rng.integers(-2, 1 << 30)), int(rng.integers(-2, 1 << 62)),
                       int(rng.integers(0, 6)), None)
    L.engram_project(0x1000, 0x2000, 0x3000, int(rng.integers(-1, 3)) * 0,
                     int(rng.integers(-64, 1 << 21)), int(rng.integers(-8, 1 << 16)),
                     int(rng.integers(-8, 1 << 22)), int(rng.integers(0, 2)), None, 0, None)
print("sweep ok")
'''


def test_host_abi_tests_under_sanitizers(sanitized_library):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=_env(sanitized_library), capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr


def test_randomized_host_calls_under_sanitizers(sanitized_library):
    r = subprocess.run([sys.executable, "-c", SWEEP], cwd=ROOT, env=_env(sanitized_library),
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "sweep ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
