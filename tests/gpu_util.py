"""Shared helpers of the GPU parity tests (comparison rules and tolerances)."""
import sys

import numpy as np

import oracle as O

# Tolerance of bf16 outputs and gates: |gpu - oracle| <= ATOL + RTOL |oracle|.
ATOL = 1e-3
RTOL = 2e-2
U32 = 2.0 ** -24          # fp32 unit roundoff


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_setup(w):
    primes = O.primes_from(w.prime_base, w.segments)
    offs, R = O.segment_offsets(primes)
    return primes, offs, R


def oracle_rows(gw, ids=None, hist=None, use_hist=True):
    w = gw.w
    primes, offs, _ = oracle_setup(w)
    ids = gw.ids_np if ids is None else ids
    if use_hist and hist is None:
        hist = gw.hist_np
    return O.hash_rows(ids, gw.token_map_np, w.compressed_vocab, gw.pad, gw.mult, primes, offs,
                       w.max_ngram, w.heads, hist=hist)


def assert_close(got, exp, what, atol=ATOL, rtol=RTOL, extra=None):
    got = np.asarray(got, dtype=np.float64)
    exp = np.asarray(exp, dtype=np.float64)
    tol = atol + rtol * np.abs(exp)
    if extra is not None:
        tol = tol + extra
    err = np.abs(got - exp)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at {idx.tolist()}: "
            f"got {got[bad][:5]}, expected {exp[bad][:5]}, max excess {(err - tol).max():.3g}")


def gemm_tolerance(e: np.ndarray, wkv: np.ndarray, kv_exact: np.ndarray, bf16_out: bool):
    """Per-element bound on |kv_gpu - kv_exact| for an fp32-accumulated product:
    rounding of the stored value (half an ulp, 2^-8 relative for bf16) plus a
    16-sigma bound on the accumulation error, u * sqrt(K) * ||e_k w_k||_2."""
    e = np.asarray(e, dtype=np.float64)
    w = np.asarray(wkv, dtype=np.float64)
    K = e.shape[1]
    norm = np.sqrt((e * e) @ (w * w).T)
    acc = 16.0 * U32 * np.sqrt(K) * norm
    rnd = (2.0 ** -8 if bf16_out else 2.0 ** -23) * np.abs(kv_exact)
    return acc + rnd


def gemm_tolerance_mx(e: np.ndarray, w: np.ndarray, kv_exact: np.ndarray):
    """Bound on |kv_gpu - kv_exact| for the block-scaled FP8 MFMA product: the
    instruction sums its 64 exact products with less than fp32 precision (single
    -instruction probes on gfx950 stayed below 2e-4 of the products' absolute sum
    on random data including subnormal codes), so 2^-11 of sum |e_k w_k| plus the
    fp32 accumulation across instructions and the bf16 rounding of the output."""
    e = np.asarray(e, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return 2.0 ** -11 * (np.abs(e) @ np.abs(w).T) + gemm_tolerance(e, w, kv_exact, True)
