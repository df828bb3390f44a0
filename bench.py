"""Benchmark of the Engram layer forward on one MI355X.

Workload: the full prefill layer forward at the pages' shape -- 4 sequences x
8192 Zipf(1.1) tokens with 2 DEAD spans of 256 per sequence, the 24 (order,
head) segments of primes from 1,000,000 (24,003,916 rows x 264 B = 6.34 GB,
generated on the device), wkv bf16 [25600, 6144] with its rows 6208 elements
apart (engram_wkv_row_stride), hc = 4 streams of width 5120.
All inputs are seeded synthetic data already resident in HBM when timing
starts.

One step = one pass of the whole hot path over the batch: engram_hash ->
engram_gather -> engram_fold_gate_weights -> engram_project_gate_sums ->
engram_gate_sums, the launches engram_forward makes at this size (its
projection fills the CUs with whole tiles, so the key side of the gate runs in
the projection's epilogue), called through the C ABI on torch's current stream.
W untimed warmup steps, then K timed steps bracketed by torch.cuda.synchronize(),
with HIP events around each step's projection only (the roofline's kernel); a
per-stage breakdown follows in steps of its own. Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Engram layer tokens/s (hash+gather+gate) and gather GB/s vs HBM peak, 1 GPU"
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0         # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0          # MI355X dense fp8 MFMA
# Algorithmic bytes per token of the gather: 24 row ids (int64) read, 24 rows of
# 264 B read, 6144 bf16 written.
GATHER_BYTES_PER_TOKEN = 24 * 8 + 24 * 264 + 6144 * 2


# The sources the bf16 projection kernel is built from; its committed traffic
# figures hold while these hash to the recorded value.
GEMM_BF16_SOURCES = ("hashed_gram_conditional_amd/csrc/gemm.hip",
                     "hashed_gram_conditional_amd/csrc/gemm_tiles.h",
                     "hashed_gram_conditional_amd/csrc/common.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(kernel: str, sources):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 PMC summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the counter's reading for a copy of
    known size), or None when no summary matches the current kernel sources (the
    sha256 of their concatenated bytes, in the order given)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for src in sources:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    sha = h.hexdigest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            f = line.split()
            if len(f) >= 3 and f[0] == "traffic" and f[1] == kernel:
                kv = dict(x.split("=", 1) for x in f[2:])
                if kv.get("sha256") != sha:
                    continue
                fetch = float(kv["fetch_kib"]) * 1024 * float(kv["fetch_scale"])
                write = float(kv["write_kib"]) * 1024 * float(kv["write_scale"])
                return {"bytes": round(fetch + write), "read": round(fetch), "written": round(write),
                        "source": os.path.relpath(path, ROOT)}
    return None


def cpu_baseline(gw, host_table, target_s: float = 10.0, max_tokens: int = 8192):
    """The oracle as it stands, timed on the host on a bounded sample: all five
    steps for the first n tokens of sequence 0 (table rows materialised in host
    RAM beforehand, so the gather reads memory rather than regenerating rows),
    then each stage on its own workload (cpu_stages). ``host_table`` is the
    6.34 GB table as a host numpy array."""
    import oracle as O
    from workloads import gen

    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = int(blas[0]["num_threads"]) if blas else 1
    except Exception:
        cores = os.cpu_count() or 1
    w = gw.w
    primes = O.primes_from(w.prime_base, w.segments)
    offs, R = O.segment_offsets(primes)
    wkv = O.bf16_bits_to_f64(gw.dense_np["wkv"])
    q_w, k_w = gw.dense_np["q_w"], gw.dense_np["k_w"]
    h_seq0 = gw.dense_np["h"][0]
    ids0 = gw.ids_np[:1]
    dead0 = (ids0[0] < 0) | (ids0[0] >= w.raw_vocab)

    def run(n):
        ids = np.ascontiguousarray(ids0[:, :n])
        rid_all, _ = O.hash_rows(ids, gw.token_map_np, w.compressed_vocab, gw.pad, gw.mult,
                                 primes, offs, w.max_ngram, w.heads)
        need = np.unique(rid_all)
        host_rows = gen.table_rows(w.table_seed, need)

        def fetch(r):
            return host_rows[np.searchsorted(need, r)]

        h = O.bf16_bits_to_f64(h_seq0[:n])
        t0 = time.perf_counter()
        rid, _ = O.hash_rows(ids, gw.token_map_np, w.compressed_vocab, gw.pad, gw.mult,
                             primes, offs, w.max_ngram, w.heads)
        O.forward_tokens(np.arange(n), rid, dead0[:n], fetch_rows=fetch, table_rows=R,
                         wkv=wkv, q_w=q_w, k_w=k_w, h=h, hc=w.hc, dim=w.dim, eps=w.eps,
                         clamp=w.gate_clamp, bf16=True)
        return time.perf_counter() - t0

    def grow(target, cap):
        n = 64
        dt = run(n)
        while dt < target / 4 and n < cap:
            n = min(cap, int(n * max(2.0, min(16.0, target / max(dt, 1e-3)))))
            dt = run(n)
        return n, dt

    n, dt = grow(target_s, max_tokens)
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            n1, dt1 = grow(target_s / 2, max_tokens // 8)
        single = {"value": round(n1 / dt1, 3), "unit": "tokens/s", "cores": 1,
                  "sample": f"first {n1} tokens, {dt1:.2f} s with BLAS limited to one thread"}
    except Exception as exc:                        # threadpoolctl missing or refused
        log(f"single-thread oracle run skipped: {exc}")
    stages = cpu_stages(gw, host_table)
    host = host_description()
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} tokens of sequence 0 of the same prefill workload, all five "
                      f"steps in fp64 numpy, table rows pre-read into host RAM; {dt:.2f} s "
                      f"with BLAS on {cores} threads",
            "cpu_model": host["cpu_model"], "host": host, "single_thread": single,
            "stages": stages}


def host_description():
    """nproc, the CPUs this process may run on, and /proc/cpuinfo's description of
    the first CPU (model name, family, model, stepping, cache size)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break
                k, _, v = line.partition(":")
                info[k.strip()] = v.strip()
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"nproc": os.cpu_count(), "usable_cpus": affinity,
            "cpu_model": info.get("model name", ""),
            "cpu_family": info.get("cpu family"), "cpu_model_number": info.get("model"),
            "stepping": info.get("stepping"), "cache_size": info.get("cache size"),
            "vendor": info.get("vendor_id")}


def _grow(run, target_s, start, cap):
    """Double the sample until one run takes a quarter of target_s (or cap)."""
    n = start
    dt = run(n)
    while dt < target_s / 4 and n < cap:
        n = min(cap, int(n * max(2.0, min(16.0, target_s / max(dt, 1e-3)))))
        dt = run(n)
    return n, dt


def cpu_stages(gw, host_table):
    """The oracle's stages on their own workloads, all cores and one thread:
    the hash over all 8 x 4096 tokens of the hash workload (C1 setup, primes from
    16,000,000); the gather over the gather workload's tokens reading the 6.34 GB
    table materialised in host RAM (a random row gather from memory, then the
    dequantisation); the decode step (256 tokens with history against the
    101.4 GB table), whose rows are regenerated from the counter generator since
    that table does not fit host RAM. Parallel runs give each worker thread its
    own contiguous range of tokens (tokens are independent)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle as O
    from threadpoolctl import threadpool_limits
    from workloads import C1, C2, C4, gen

    workers = min(16, os.cpu_count() or 1)
    out = {}
    # hash: C1
    tm, mult = gen.hash_setup(C1)
    primes = O.primes_from(C1.prime_base, C1.segments)
    offs, _ = O.segment_offsets(primes)
    ids, _ = gen.token_ids(C1)
    t0 = time.perf_counter()
    O.hash_rows(ids, tm, C1.compressed_vocab, int(tm[0]), mult, primes, offs, C1.max_ngram,
                C1.heads)
    dt = time.perf_counter() - t0
    out["hash"] = {"tokens_per_s": round(C1.tokens / dt, 1),
                   "GBps": round(C1.tokens * 196 / dt / 1e9, 4), "cores": 1,
                   "sample": f"all {C1.tokens} tokens of the 8 x 4096 hash workload, {dt:.3f} s"}
    # gather: C2 over the materialised table
    w = gw.w
    R = gw.rows
    ids2, _ = gen.token_ids(C2)
    rid2, _ = O.hash_rows(ids2, gw.token_map_np, w.compressed_vocab, gw.pad, gw.mult,
                          O.primes_from(C2.prime_base, C2.segments),
                          O.segment_offsets(O.primes_from(C2.prime_base, C2.segments))[0],
                          C2.max_ngram, C2.heads)
    fetch = lambda r: host_table[r]

    def gather_run(n, threads):
        chunk = max(1, -(-n // threads))
        t0 = time.perf_counter()
        if threads == 1:
            O.gather_e4m3(fetch, rid2[:n], R)
        else:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(lambda lo: O.gather_e4m3(fetch, rid2[lo:min(n, lo + chunk)], R),
                            range(0, n, chunk)))
        return time.perf_counter() - t0

    g = {}
    for label, threads in (("all_cores", workers), ("single_thread", 1)):
        n, dt = _grow(lambda k: gather_run(k, threads), 4.0, 256, C2.tokens)
        g[label] = {"tokens_per_s": round(n / dt, 1),
                    "GBps": round(n * GATHER_BYTES_PER_TOKEN / dt / 1e9, 4), "cores": threads,
                    "sample": f"first {n} tokens of the 16 x 8192 gather workload ({n * 24} "
                              f"rows), {dt:.2f} s"}
    g["table"] = "24,003,916 x 264 B (6.34 GB) in host RAM, rows read by fancy indexing"
    out["gather"] = g
    # decode: C4, rows regenerated
    tm4, mult4 = gen.hash_setup(C4)
    p4 = O.primes_from(C4.prime_base, C4.segments)
    o4, R4 = O.segment_offsets(p4)
    ids4, _ = gen.token_ids(C4)
    hist4 = gen.history(C4, tm4)
    d4 = gen.dense_inputs(C4)
    wkv4 = O.bf16_bits_to_f64(d4["wkv"])
    h4 = O.bf16_bits_to_f64(d4["h"].reshape(C4.tokens, C4.hc, C4.dim))
    dead4 = ids4.reshape(-1) < 0

    def decode_run():
        t0 = time.perf_counter()
        rid4, _ = O.hash_rows(ids4, tm4, C4.compressed_vocab, int(tm4[0]), mult4, p4, o4,
                              C4.max_ngram, C4.heads, hist=hist4)
        O.forward_tokens(np.arange(C4.tokens), rid4, dead4,
                         fetch_rows=lambda r: gen.table_rows(C4.table_seed, r), table_rows=R4,
                         wkv=wkv4, q_w=d4["q_w"], k_w=d4["k_w"], h=h4, hc=C4.hc, dim=C4.dim,
                         eps=C4.eps, clamp=C4.gate_clamp, bf16=True)
        return time.perf_counter() - t0

    dt = decode_run()
    with threadpool_limits(limits=1):
        dt1 = decode_run()
    out["decode"] = {"tokens_per_s": round(C4.tokens / dt, 1), "cores": workers,
                     "single_thread_tokens_per_s": round(C4.tokens / dt1, 1),
                     "sample": f"one decode step, 256 tokens with history, all five steps; "
                               f"{dt:.2f} s with BLAS on all threads, {dt1:.2f} s on one",
                     "note": "rows regenerated from the counter generator (the 101.4 GB "
                             "table does not fit host RAM)"}
    del wkv4, h4, d4
    return out


def copy_calibration(mib: int):
    """One device-to-device copy of ``mib`` MiB: the counter reading of a copy of
    known size scales FETCH_SIZE and WRITE_SIZE to bytes."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _calibration_lib():
    import ctypes
    path = os.path.join(ROOT, "hashed_gram_conditional_amd", "libengram_calibrate.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.engram_calibrate_mfma_bf16.argtypes = [P, P, I64, P, I32, I32, P]
    lib.engram_calibrate_mfma_fp8.argtypes = [P, P, I64, P, P, I64, P, I32, I32, P]
    for f in (lib.engram_calibrate_mfma_flop, lib.engram_calibrate_mfma_fp8_flop):
        f.argtypes = [I32, I32]
        f.restype = ctypes.c_double
    return lib


def _time_stream(call, flop_of, iters: int):
    import torch
    stream = torch.cuda.current_stream()
    call(2000)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    call(iters)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    return flop_of(iters) / (ms * 1e-3) / 1e12, ms


def mfma_ceiling(a, b, iters: int = 40000):
    """The rate of a pure v_mfma_f32_32x32x16_bf16 stream (libengram_calibrate.so,
    no memory traffic in its loop) on fragments of the projection's own operands:
    a the gathered e, b the weight. On random bits the power limit holds the clock
    below the one the published peak assumes; this is the ceiling of any kernel
    computing that product on this GPU."""
    import ctypes
    import torch
    lib = _calibration_lib()
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    n_frag = min(a.numel(), b.numel()) // 8
    stream = torch.cuda.current_stream()

    def call(n):
        rc = lib.engram_calibrate_mfma_bf16(a.data_ptr(), b.data_ptr(), n_frag, out.data_ptr(),
                                            blocks, n, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"engram_calibrate_mfma_bf16 failed: {rc}")

    tflops, ms = _time_stream(call, lambda n: lib.engram_calibrate_mfma_flop(blocks, n), iters)
    return {"what": "pure v_mfma_f32_32x32x16_bf16 stream on fragments of the step's e and "
                    "wkv, one wave per SIMD, no memory traffic",
            "achieved": round(tflops, 1), "unit": "TFLOP/s", "ms": round(ms, 2),
            "frac_of_peak": round(tflops / BF16_PEAK_TFLOPS, 4)}


def mfma_ceiling_fp8(a, b, sa, sb, iters: int = 20000):
    """mfma_ceiling for the FP8 projection: v_mfma_scale_f32_32x32x64_f8f6f4 on
    32-byte fragments of the step's E4M3 codes (a: e's, b: the weight's) with
    their E8M0 scale bytes (sa, sb)."""
    import ctypes
    import torch
    lib = _calibration_lib()
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    n_frag = min(a.numel(), b.numel()) // 32
    n_scale = min(sa.numel(), sb.numel())
    stream = torch.cuda.current_stream()

    def call(n):
        rc = lib.engram_calibrate_mfma_fp8(a.data_ptr(), b.data_ptr(), n_frag, sa.data_ptr(),
                                           sb.data_ptr(), n_scale, out.data_ptr(), blocks, n,
                                           ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"engram_calibrate_mfma_fp8 failed: {rc}")

    tflops, ms = _time_stream(call, lambda n: lib.engram_calibrate_mfma_fp8_flop(blocks, n),
                              iters)
    return {"what": "pure v_mfma_scale_f32_32x32x64_f8f6f4 stream on fragments of the step's "
                    "e and weight codes and scales, one wave per SIMD, no memory traffic",
            "achieved": round(tflops, 1), "unit": "TFLOP/s", "ms": round(ms, 2),
            "frac_of_peak": round(tflops / FP8_PEAK_TFLOPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-step measurement on the 101 GB table")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode-step measurement (profiling its kernels)")
    ap.add_argument("--gather-only", action="store_true",
                    help="only the gather workload's measurement (profiling its kernel)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--wkv-ld", type=int, default=None,
                    help="row stride of wkv in elements (0: dense rows; default: "
                         "engram_wkv_row_stride)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the layer is measured on one GPU only; no multi-GPU run is made.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import hashed_gram_conditional_amd as E
    from workloads import C3
    from workloads.harness import GpuWorkload

    torch.cuda.set_device(0)
    if args.decode_only:
        if args.copy_calibration_mib:
            copy_calibration(args.copy_calibration_mib)
        print(json.dumps({"decode": decode_bench(args.steps, args.warmup, args.wkv_ld)}),
              flush=True)
        return
    if args.gather_only:
        from workloads import C2
        if args.copy_calibration_mib:
            copy_calibration(args.copy_calibration_mib)
        print(json.dumps({"gather_c2": gather_c2_bench(GpuWorkload(C2), args.steps)}),
              flush=True)
        return
    t_setup = time.perf_counter()
    gw = GpuWorkload(C3, wkv_ld=args.wkv_ld)
    w = gw.w
    T, S = w.tokens, w.segments
    K_in, N_out = S * w.row_dim, (w.hc + 1) * w.dim
    rows = torch.empty((T, S), dtype=torch.int64, device="cuda")
    e = torch.empty((T, K_in), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((T, N_out), dtype=torch.bfloat16, device="cuda")
    gates = torch.empty((T, w.hc), dtype=torch.float32, device="cuda")
    qk_w = torch.empty((w.hc, w.dim), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s: {T} tokens, table {gw.rows} rows")

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)

    stream = torch.cuda.current_stream()

    # Events only where a figure needs them: an event recorded between two
    # launches leaves the GPU idle for about 6 us on this stack. The timed
    # steps bracket the projection (the roofline's kernel); the per-stage
    # breakdown comes from steps of its own afterwards.
    def step(evs, marks):
        if evs and 0 in marks:
            evs[0].record(stream)
        E.engram_hash(gw.params, gw.ids, w.batch, w.seq, None, None, rows)
        if evs and 1 in marks:
            evs[1].record(stream)
        E.engram_gather(gw.table, gw.rows, gw.row_format, w.row_dim, rows, T * S, e)
        if evs and 2 in marks:
            evs[2].record(stream)
        E.engram_fold_gate_weights(gw.q_w, gw.k_w, w.hc, w.dim, qk_w)
        if evs and 3 in marks:
            evs[3].record(stream)
        E.engram_project_gate_sums(gw.desc, e, K_in, gw.wkv, gw.h, qk_w, kv)
        if evs and 4 in marks:
            evs[4].record(stream)
        E.engram_gate_sums(gw.desc, gw.ids, w.raw_vocab, kv, gw.h, gates)
        if evs and 5 in marks:
            evs[5].record(stream)

    for _ in range(args.warmup):
        step(None, ())
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i], (3, 4))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    project_ms = float(np.mean([s[3].elapsed_time(s[4]) for s in ev]))
    # hash, gather, fold, projection, gate: events around every stage
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(sev[i], (0, 1, 2, 3, 4, 5))
    torch.cuda.synchronize()
    stage_ms = np.mean([[s[j].elapsed_time(s[j + 1]) for j in range(5)] for s in sev], axis=0)

    # the separate stages for comparison: the projection storing every key,
    # then the gate reading them (engram_forward's path for calls that do not
    # fill the CUs with whole tiles)
    sep = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps + 2):
        evs = sep[i - 2] if i >= 2 else None
        if evs:
            evs[0].record(stream)
        E.engram_project(e, gw.wkv, kv, T, K_in, N_out, gw.wkv_ld, 0)
        if evs:
            evs[1].record(stream)
        E.engram_gate_folded(gw.desc, gw.ids, w.raw_vocab, kv, qk_w, gw.h, gates)
        if evs:
            evs[2].record(stream)
    torch.cuda.synchronize()
    sep_ms = np.mean([[s[j].elapsed_time(s[j + 1]) for j in range(2)] for s in sep], axis=0)

    # the fused entry point, for comparison (the same launches, one call)
    ws, nws = gw.workspace()
    fe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(2):
        E.engram_forward(gw.params, gw.desc, gw.ids, None, None, gw.table, gw.wkv, gw.q_w,
                         gw.k_w, gw.h, gates, ws, nws)
    fe[0].record(stream)
    for _ in range(args.steps):
        E.engram_forward(gw.params, gw.desc, gw.ids, None, None, gw.table, gw.wkv, gw.q_w,
                         gw.k_w, gw.h, gates, ws, nws)
    fe[1].record(stream)
    torch.cuda.synchronize()
    forward_ms = fe[0].elapsed_time(fe[1]) / args.steps
    ceiling = mfma_ceiling(e, gw.wkv[:1024, :K_in].contiguous())

    flops = 2.0 * T * N_out * K_in
    gemm_tflops = flops / (project_ms * 1e-3) / 1e12
    gather_gbps = GATHER_BYTES_PER_TOKEN * T / (stage_ms[1] * 1e-3) / 1e9
    tokens_per_s = T / (ms_per_step * 1e-3)
    traffic = measured_traffic("gemm_bf16_sums_kernel", GEMM_BF16_SOURCES)
    ceiling["projection_frac_of_ceiling"] = round(gemm_tflops / ceiling["achieved"], 4)
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill layer forward: 4 x 8192 Zipf tokens, 24 segments of "
                               "primes from 1,000,000 (24,003,916 x 264 B rows), wkv "
                               "6144 -> 5 x 5120, hc 4 x 5120",
                   "batch": w.batch, "seq": w.seq, "segments": S, "hc": w.hc, "dim": w.dim,
                   "table_rows": gw.rows, "wkv_row_stride": gw.wkv_ld},
        "roofline": {"bound": "mfma",
                     "kernel": "gemm_bf16_sums_kernel (engram_project_gate_sums)",
                     "achieved": round(gemm_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic["bytes"] if traffic else None,
                     "traffic_detail": traffic,
                     "algorithmic_flop": flops},
        "mfma_ceiling": ceiling,
        "gather": {"kernel": "gather_e4m3_kernel (engram_gather)",
                   "achieved": round(gather_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                   "frac": round(gather_gbps / HBM_PEAK_GBPS, 4),
                   "bytes_per_token": GATHER_BYTES_PER_TOKEN},
        "project_ms": round(project_ms, 4),
        "stages_ms": {"hash": round(stage_ms[0], 4), "gather": round(stage_ms[1], 4),
                      "fold": round(stage_ms[2], 4), "project_gate_sums": round(stage_ms[3], 4),
                      "gate_sums": round(stage_ms[4], 4),
                      "method": "steps of their own after the timed ones, events around every "
                                "stage (each adds ~6 us of idle GPU)"},
        "separate_stages_ms": {"project": round(sep_ms[0], 4), "gate": round(sep_ms[1], 4),
                               "what": "engram_project storing every key, then "
                                       "engram_gate_folded reading them"},
        "engram_forward_ms": round(forward_ms, 4),
    }
    detail, hash_steady = gather_detail(gw, rows, e, max(args.steps // 2, 5))
    out["gather"].update(detail)
    out["gather"]["frac_of_torch_copy"] = round(gather_gbps / detail["torch_copy_GBps"], 4)
    out["hash_steady"] = hash_steady
    out["gather_c2"] = gather_c2_bench(gw, max(args.steps, 10))
    out["gather_c2"]["frac_of_torch_copy_cold"] = round(
        out["gather_c2"]["cold"]["achieved"] / detail["torch_copy_GBps"], 4)
    out["short_conv"] = conv_prefill_bench(gw, rows, e, kv, gates, args.steps, args.warmup)
    t_pin = time.perf_counter()
    host = torch.empty(gw.table.shape, dtype=torch.uint8, pin_memory=True)
    host.copy_(gw.table)
    torch.cuda.synchronize()
    log(f"host table pinned and filled in {time.perf_counter() - t_pin:.1f} s")
    out["host_tier"] = host_tier_bench(gw, host, rows, e, kv, gates, args.steps, args.warmup)
    out["hash_layers"] = hash_layers_bench(max(args.steps, 20))
    out["fp8_wkv"] = fp8_prefill_bench(gw, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on bounded samples ...")
        out["cpu_baseline"] = cpu_baseline(gw, host.numpy())
    del host
    if not args.no_decode:
        del rows, e, kv, gates, ws
        gw.free()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["decode"] = decode_bench(args.steps, args.warmup, args.wkv_ld)
    print(json.dumps(out), flush=True)


def conv_prefill_bench(gw, rows, e, kv, gates, steps: int, warmup: int):
    """The prefill layer with the papers' short convolution branch after the gate
    (4 taps at dilation 3, RMSNorm, SiLU; random filters and norm weights):
    engram_hash -> engram_gather -> engram_fold_gate_weights ->
    engram_project_gate_sums -> engram_gate_conv_sums (engram_forward_conv's
    launches at this size), the last also writing the 9-position history of
    every sequence. The gate-and-branch stage runs two kernels over the token
    stream; its algorithmic bytes per token are those of both: h, v and the key
    sums read and the gates and mean square written by the first, then h read
    and written, v and the statistics read by the second."""
    import torch
    import hashed_gram_conditional_amd as E

    w = gw.w
    T, S = w.tokens, w.segments
    K_in, N_out = S * w.row_dim, (w.hc + 1) * w.dim
    g = torch.Generator(device="cuda").manual_seed(77)
    cw = 0.3 * torch.randn((w.hc, w.dim, 4), generator=g, device="cuda")
    nw = 1 + 0.1 * torch.randn((w.hc, w.dim), generator=g, device="cuda")
    sv = torch.zeros((w.batch, 9, w.dim), dtype=torch.bfloat16, device="cuda")
    ss = torch.zeros((w.batch, 9, w.hc + 1), dtype=torch.float32, device="cuda")
    conv = E.short_conv(cw, 4, 3, 1e-6, nw, None, None, sv, ss)
    n_ws = E.engram_gate_conv_workspace_size(gw.desc)
    cws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
    qk_w = torch.empty((w.hc, w.dim), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]

    def step(evs):
        if evs:
            evs[0].record(stream)
        E.engram_hash(gw.params, gw.ids, w.batch, w.seq, None, None, rows)
        if evs:
            evs[1].record(stream)
        E.engram_gather(gw.table, gw.rows, gw.row_format, w.row_dim, rows, T * S, e)
        if evs:
            evs[2].record(stream)
        E.engram_fold_gate_weights(gw.q_w, gw.k_w, w.hc, w.dim, qk_w)
        if evs:
            evs[3].record(stream)
        E.engram_project_gate_sums(gw.desc, e, K_in, gw.wkv, gw.h, qk_w, kv)
        if evs:
            evs[4].record(stream)
        E.engram_gate_conv_sums(gw.desc, conv, gw.ids, w.raw_vocab, kv, gw.h, gates, cws, n_ws)
        if evs:
            evs[5].record(stream)

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # hash, gather, fold, projection, gate and branch
    st = np.mean([[s_[j].elapsed_time(s_[j + 1]) for j in range(5)] for s_ in ev], axis=0)
    ms = 1e3 * wall / steps
    d = w.dim
    bytes_per_token = (w.hc * d * 2 + d * 2 + w.hc * (d // 128) * 8 + (w.hc + 1) * 4) + \
                      (2 * w.hc * d * 2 + d * 2 + (w.hc + 1) * 4)
    gbps = bytes_per_token * T / (st[4] * 1e-3) / 1e9
    del cws, sv, ss, cw, nw, qk_w
    return {"workload": "prefill layer forward as above with the short convolution branch "
                        "(4 taps, dilation 3) and its history written",
            "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "stages_ms": {"hash": round(st[0], 4), "gather": round(st[1], 4),
                          "fold": round(st[2], 4), "project_gate_sums": round(st[3], 4),
                          "gate_conv_sums": round(st[4], 4)},
            "gate_conv": {"kernels": "gate_sums_kernel (gates, mean(v^2)) + "
                                     "short_conv_window_kernel + conv_state_kernel",
                          "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(gbps / HBM_PEAK_GBPS, 4),
                          "bytes_per_token": bytes_per_token}}


def host_tier_bench(gw, host, rows, e, kv, gates, steps: int, warmup: int):
    """The prefill layer with its table (6.34 GB) in pinned host memory. The
    gather kernels read the rows over the host link. (1) Lookups alone: all
    32768 tokens' rows (raw and dequantised) and one 256-token decode-sized
    batch. (2) The pipelined step: while step i's projection and gate run on the
    compute stream, a second stream hashes and gathers step i+1's rows from the
    host table into the other of two e buffers; events order the buffers. The
    fetch is hidden when it takes less than the projection (stall =
    max(0, T_fetch - T_window))."""
    import torch
    import hashed_gram_conditional_amd as E

    w = gw.w
    T, S = w.tokens, w.segments
    K_in, N_out = S * w.row_dim, (w.hc + 1) * w.dim
    main = torch.cuda.current_stream()
    raw = torch.empty((T, S, 264), dtype=torch.uint8, device="cuda")

    def timed(fn, reps):
        for _ in range(2):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(main)
        for _ in range(reps):
            fn()
        b.record(main)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    E.engram_hash(gw.params, gw.ids, w.batch, w.seq, None, None, rows)
    rows_ms = timed(lambda: E.engram_gather_rows(host, gw.rows, rows, T * S, raw), 10)
    deq_ms = timed(lambda: E.engram_gather(host, gw.rows, gw.row_format, w.row_dim, rows, T * S,
                                           e), 10)
    dec_ms = timed(lambda: E.engram_gather(host, gw.rows, gw.row_format, w.row_dim, rows,
                                           256 * S, e), 50)
    row_bytes = T * S * 264

    # pipelined steps, two e / row-id buffers
    e_buf = [e, torch.empty_like(e)]
    r_buf = [rows, torch.empty_like(rows)]
    side = torch.cuda.Stream()
    ready = [torch.cuda.Event(), torch.cuda.Event()]
    free = [torch.cuda.Event(), torch.cuda.Event()]

    qk_w = torch.empty((w.hc, w.dim), dtype=torch.float32, device="cuda")

    def fetch(slot):
        side.wait_event(free[slot])
        E.engram_hash(gw.params, gw.ids, w.batch, w.seq, None, None, r_buf[slot], stream=side)
        E.engram_gather(host, gw.rows, gw.row_format, w.row_dim, r_buf[slot], T * S, e_buf[slot],
                        stream=side)
        ready[slot].record(side)

    def compute(slot):
        main.wait_event(ready[slot])
        E.engram_fold_gate_weights(gw.q_w, gw.k_w, w.hc, w.dim, qk_w, stream=main)
        E.engram_project_gate_sums(gw.desc, e_buf[slot], K_in, gw.wkv, gw.h, qk_w, kv,
                                   stream=main)
        E.engram_gate_sums(gw.desc, gw.ids, w.raw_vocab, kv, gw.h, gates, stream=main)
        free[slot].record(main)

    for ev in free:
        ev.record(main)
    fetch(0)

    def run(n, first):
        for i in range(first, first + n):
            fetch((i + 1) % 2)
            compute(i % 2)
        return first + n

    nxt = run(warmup, 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    nxt = run(steps, nxt)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    del raw, e_buf, r_buf
    return {"workload": "prefill layer forward as above with the 6.34 GB table in pinned host "
                        "memory: each step's rows are gathered over the host link by the GPU "
                        "during the previous step's projection (two buffers, two streams)",
            "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "fetch_rows_ms": round(rows_ms, 4),
            "fetch_rows_GBps": round(row_bytes / (rows_ms * 1e-3) / 1e9, 1),
            "fetch_dequant_ms": round(deq_ms, 4),
            "fetch_dequant_rows_GBps": round(row_bytes / (deq_ms * 1e-3) / 1e9, 1),
            "decode_fetch_256_tokens_us": round(dec_ms * 1e3, 1)}


def gather_detail(gw, rows, e, reps: int):
    """Beside the warm (back-to-back) gather: torch's device-to-device copy rate, the
    same gather with the L2s and the 256 MB Infinity Cache flushed before every
    rep by reading a 1 GiB buffer, and engram_hash over 32 x the prefill
    ids in one call (the steady-state hash rate, free of launch latency)."""
    import statistics
    import torch
    import hashed_gram_conditional_amd as E

    w = gw.w
    T, S = w.tokens, w.segments
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed_once(fn):
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    copy_ms = statistics.median(timed_once(lambda: dst.copy_(src)) for _ in range(5))
    copy_gbps = 2 * n / (copy_ms * 1e-3) / 1e9
    del src
    sink = torch.empty((), dtype=torch.uint8, device="cuda")
    cold = []
    for _ in range(reps):
        torch.amax(dst, dim=0, out=sink)
        cold.append(timed_once(lambda: E.engram_gather(gw.table, gw.rows, gw.row_format,
                                                        w.row_dim, rows, T * S, e)))
    del dst, sink
    cold_ms = statistics.median(cold)
    cold_gbps = GATHER_BYTES_PER_TOKEN * T / (cold_ms * 1e-3) / 1e9

    ids32 = gw.ids.repeat(32, 1).contiguous()
    B32 = ids32.shape[0]
    rows32 = torch.empty((B32 * w.seq, S), dtype=torch.int64, device="cuda")
    hash32 = lambda: E.engram_hash(gw.params, ids32, B32, w.seq, None, None, rows32)
    for _ in range(3):
        hash32()
    torch.cuda.synchronize()
    hash_ms = statistics.median(timed_once(hash32) for _ in range(max(reps, 10)))
    tokens = B32 * w.seq
    hash_bytes = 4 + 8 * S
    del ids32, rows32
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return ({"torch_copy_GBps": round(copy_gbps, 1),
             "torch_copy": "tensor.copy_ of 1 GiB on the device: read + write bytes over the median "
                           "of 5 (a reference rate, not the HBM peak)",
             "cold": {"ms": round(cold_ms, 4), "achieved": round(cold_gbps, 1),
                      "frac": round(cold_gbps / HBM_PEAK_GBPS, 4),
                      "flush": "1 GiB read before each rep (caches evicted, clean)"}},
            {"workload": f"engram_hash over 32 x the prefill ids ({B32} x {w.seq} = {tokens} "
                         f"tokens) in one call",
             "us": round(hash_ms * 1e3, 1), "tokens_per_s": round(tokens / (hash_ms * 1e-3), 1),
             "bytes_per_token": hash_bytes,
             "achieved_GBps": round(hash_bytes * tokens / (hash_ms * 1e-3) / 1e9, 1)})


def gather_c2_bench(gw, reps: int):
    """engram_gather at the gather workload's own size: 16 x 8192 Zipf tokens
    hashed against the same 24,003,916-row table (the gather workload and the
    prefill share the table's seed and primes), 3,145,728 rows of 264 B read
    and 1.61 GB of bf16 written per call. Warm: back-to-back calls. Cold: a
    1 GiB buffer read before every call (a max-reduction), which evicts the L2s
    and the 256 MB Infinity Cache and leaves them holding clean lines. Cold,
    dirty caches: the same buffer written instead, so the caches hold up to
    ~0.27 GB of another kernel's dirty lines that the timed call must write back
    to HBM. Each figure is the median over ``reps`` calls timed with HIP events
    on the launch stream."""
    import statistics
    import torch
    import hashed_gram_conditional_amd as E
    from workloads import C2, C3, gen
    from workloads.device import to_device

    assert (C2.table_seed, C2.prime_base, C2.setup_seed) == \
        (C3.table_seed, C3.prime_base, C3.setup_seed)
    w = C2
    T, S = w.tokens, w.segments
    ids_np, _ = gen.token_ids(w)
    ids = to_device(ids_np)
    rows = torch.empty((T, S), dtype=torch.int64, device="cuda")
    out = torch.empty((T * S, 256), dtype=torch.bfloat16, device="cuda")
    E.engram_hash(gw.params, ids, w.batch, w.seq, None, None, rows)
    torch.cuda.synchronize()
    distinct = int(torch.unique(rows).numel())
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    run = lambda: E.engram_gather(gw.table, gw.rows, gw.row_format, w.row_dim, rows, T * S, out)

    def timed_once():
        a.record(stream)
        run()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    warm = statistics.median(timed_once() for _ in range(reps))
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(3)
    sink = torch.empty((), dtype=torch.uint8, device="cuda")
    cold, dirty = [], []
    for _ in range(reps):
        torch.amax(flush, dim=0, out=sink)
        cold.append(timed_once())
    for i in range(reps):
        flush.fill_(i & 7)
        dirty.append(timed_once())
    cold_ms = statistics.median(cold)
    dirty_ms = statistics.median(dirty)
    del flush, sink, out, rows, ids
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    nbytes = GATHER_BYTES_PER_TOKEN * T
    gw_ = lambda ms: nbytes / (ms * 1e-3) / 1e9
    return {"workload": "gather + dequant: 16 x 8192 Zipf tokens with 2 DEAD spans of 256 per "
                        "sequence, 24 rows each from the 24,003,916 x 264 B table (6.34 GB), "
                        "bf16 [131072, 6144] written",
            "kernel": "gather_e4m3_kernel (engram_gather)", "bytes_per_token": GATHER_BYTES_PER_TOKEN,
            "algorithmic_bytes": nbytes, "distinct_rows": distinct, "lookups": T * S,
            "warm": {"ms": round(warm, 4), "achieved": round(gw_(warm), 1),
                     "frac": round(gw_(warm) / HBM_PEAK_GBPS, 4)},
            "cold": {"ms": round(cold_ms, 4), "achieved": round(gw_(cold_ms), 1),
                     "frac": round(gw_(cold_ms) / HBM_PEAK_GBPS, 4),
                     "flush": "1 GiB read before each call (caches evicted, clean)"},
            "cold_dirty_caches": {"ms": round(dirty_ms, 4), "achieved": round(gw_(dirty_ms), 1),
                                  "frac": round(gw_(dirty_ms) / HBM_PEAK_GBPS, 4),
                                  "flush": "1 GiB written before each call (its dirty lines "
                                           "are written back during the call)"},
            "peak": HBM_PEAK_GBPS, "unit": "GB/s"}


def fp8_prefill_bench(gw, steps: int, warmup: int):
    """The same prefill layer with the projection weight in block-scaled FP8 (E4M3
    values, one E8M0 scale per 32 inputs, quantised from the bf16 run's N(0, 0.02)
    distribution): engram_hash -> engram_gather_mx -> engram_fold_gate_weights ->
    engram_project_mx_gate_sums -> engram_gate_sums (engram_forward_mx's launches
    at this size), per-stage HIP events as in the bf16 run."""
    import torch
    import hashed_gram_conditional_amd as E
    from workloads import gen
    from workloads.device import to_device

    w = gw.w
    T, S = w.tokens, w.segments
    N_out = (w.hc + 1) * w.dim
    codes, scales = gen.wkv_mx(w)
    wc, wsc = to_device(codes), to_device(scales)
    rows = torch.empty((T, S), dtype=torch.int64, device="cuda")
    e_codes = torch.empty((T, S * 256), dtype=torch.uint8, device="cuda")
    e_scales = torch.empty((T, S * 8), dtype=torch.uint8, device="cuda")
    kv = torch.empty((T, N_out), dtype=torch.bfloat16, device="cuda")
    gates = torch.empty((T, w.hc), dtype=torch.float32, device="cuda")
    qk_w = torch.empty((w.hc, w.dim), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]

    def step(evs):
        if evs:
            evs[0].record(stream)
        E.engram_hash(gw.params, gw.ids, w.batch, w.seq, None, None, rows)
        if evs:
            evs[1].record(stream)
        E.engram_gather_mx(gw.table, gw.rows, rows, T * S, e_codes, e_scales)
        if evs:
            evs[2].record(stream)
        E.engram_fold_gate_weights(gw.q_w, gw.k_w, w.hc, w.dim, qk_w)
        if evs:
            evs[3].record(stream)
        E.engram_project_mx_gate_sums(gw.desc, e_codes, e_scales, S, wc, wsc, gw.h, qk_w, kv)
        if evs:
            evs[4].record(stream)
        E.engram_gate_sums(gw.desc, gw.ids, w.raw_vocab, kv, gw.h, gates)
        if evs:
            evs[5].record(stream)

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # hash, gather_mx, fold, projection, gate
    st = np.mean([[s[j].elapsed_time(s[j + 1]) for j in range(5)] for s in ev], axis=0)
    ms = 1e3 * wall / steps
    tflops = 2.0 * T * N_out * S * 256 / (st[3] * 1e-3) / 1e12
    ceiling = mfma_ceiling_fp8(e_codes, wc, e_scales, wsc)
    ceiling["projection_frac_of_ceiling"] = round(tflops / ceiling["achieved"], 4)
    # the decode-sized projection: the first 256 tokens' rows against the same
    # weight (engram_project_mx alone, back-to-back calls between two events)
    dec = 256
    kv_dec = torch.empty((dec, N_out), dtype=torch.bfloat16, device="cuda")
    n_dec = E.engram_project_mx_workspace_size(dec, S, N_out)
    ws_dec = torch.empty(n_dec, dtype=torch.uint8, device="cuda") if n_dec else None
    for _ in range(3):
        E.engram_project_mx(e_codes[:dec], e_scales[:dec], S, wc, wsc, kv_dec, dec, N_out,
                            ws_dec, n_dec)
    dev_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    dev_ev[0].record(stream)
    for _ in range(20):
        E.engram_project_mx(e_codes[:dec], e_scales[:dec], S, wc, wsc, kv_dec, dec, N_out,
                            ws_dec, n_dec)
    dev_ev[1].record(stream)
    torch.cuda.synchronize()
    dec_us = 1e3 * dev_ev[0].elapsed_time(dev_ev[1]) / 20
    w_bytes = N_out * S * 256 * (1 + 1 / 32)
    del rows, e_codes, e_scales, kv, gates, wc, wsc, kv_dec, ws_dec
    return {"workload": "prefill layer forward as above, projection weight in block-scaled FP8 "
                        "(E4M3 + one E8M0 scale per 32 inputs), rows fed to the FP8 MFMA "
                        "without dequantisation",
            "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "stages_ms": {"hash": round(st[0], 4), "gather_mx": round(st[1], 4),
                          "fold": round(st[2], 4), "project_mx_gate_sums": round(st[3], 4),
                          "gate_sums": round(st[4], 4)},
            "project_mx": {"achieved": round(tflops, 2), "peak": FP8_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tflops / FP8_PEAK_TFLOPS, 4)},
            "mfma_ceiling": ceiling,
            "decode_projection": {"tokens": dec, "us": round(dec_us, 2),
                                  "weight_GBps": round(w_bytes / (dec_us * 1e-6) / 1e9, 1),
                                  "what": "engram_project_mx on 256 tokens' rows (the decode "
                                          "size), 20 back-to-back calls between two events"}}


def hash_layers_bench(reps: int):
    """Row ids of the two Engram layers (the pages' layer-1 and layer-14 primes,
    each layer with its own multipliers) for 8 x 4096 tokens: one
    engram_hash_layers pass against one engram_hash call per layer. Each figure
    is the mean over ``reps`` back-to-back launches between two HIP events."""
    import torch
    import hashed_gram_conditional_amd as E
    from workloads import C1, gen
    from workloads.harness import GpuWorkload

    gw = GpuWorkload(C1, table=False, dense=False)
    w = gw.w
    L, T, S = 2, w.tokens, w.segments
    mults = gen.layer_multipliers(w, L)
    primes, offs, table_rows = E.engram_make_layer_primes(w.prime_base, L, S)
    params = [E.hash_params(w.raw_vocab, w.compressed_vocab, w.max_ngram, w.heads, gw.pad,
                            gw.token_map, mults[i], primes[i], offs[i]) for i in range(L)]
    rows = torch.empty((L, T, S), dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / reps

    one = timed(lambda: E.engram_hash_layers(params, gw.ids, w.batch, w.seq, None, None, rows))
    two = timed(lambda: [E.engram_hash(params[i], gw.ids, w.batch, w.seq, None, None, rows[i])
                         for i in range(L)])
    nbytes = T * (4 + L * S * 8)
    del rows
    gw.free()
    return {"workload": "two Engram layers hashed in one pass: 8 x 4096 Zipf tokens with DEAD "
                        "spans, 2 x 24 segments, primes from 16,000,000 (tables of "
                        f"{table_rows[0]:,} and {table_rows[1]:,} rows)",
            "one_pass_us": round(one, 2), "one_call_per_layer_us": round(two, 2),
            "bytes_per_token": 4 + L * S * 8,
            "achieved_GBps": round(nbytes / (one * 1e-6) / 1e9, 1)}


def decode_bench(steps: int, warmup: int, wkv_ld=None):
    """Decode step on the full-size table: 256 sequences x 1 new token with a
    3-token history, 384,006,168 rows (101.4 GB) in HBM; engram_forward per step
    with the history carried in place."""
    import torch
    import hashed_gram_conditional_amd as E
    from workloads import C4
    from workloads.harness import GpuWorkload

    t0 = time.perf_counter()
    gw = GpuWorkload(C4, wkv_ld=wkv_ld)
    w = gw.w
    ws, nws = gw.workspace()
    gates = torch.empty((w.tokens, w.hc), dtype=torch.float32, device="cuda")
    hist = gw.hist_in.clone()
    torch.cuda.synchronize()
    log(f"decode setup {time.perf_counter() - t0:.1f} s: table {gw.rows} rows")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        E.engram_forward(gw.params, gw.desc, gw.ids, hist, hist, gw.table, gw.wkv, gw.q_w,
                         gw.k_w, gw.h, gates, ws, nws)
    torch.cuda.synchronize()
    # Two events around the whole run: an event recorded between two launches
    # leaves the GPU idle for about 6 us on this stack, 5 % of a decode step.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for i in range(steps):
        E.engram_forward(gw.params, gw.desc, gw.ids, hist, hist, gw.table, gw.wkv, gw.q_w,
                         gw.k_w, gw.h, gates, ws, nws)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    # the same step captured once in a HIP graph and replayed (no launch gaps
    # between its kernels; the history advances in place on every replay)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        E.engram_forward(gw.params, gw.desc, gw.ids, hist, hist, gw.table, gw.wkv, gw.q_w,
                         gw.k_w, gw.h, gates, ws, nws)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    gev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    gev[0].record(stream)
    for _ in range(steps):
        graph.replay()
    gev[1].record(stream)
    torch.cuda.synchronize()
    graph_ms = gev[0].elapsed_time(gev[1]) / steps
    del graph
    # per-stage breakdown through the stage entry points
    T, S = w.tokens, w.segments
    K_in, N_out = S * w.row_dim, (w.hc + 1) * w.dim
    rows = torch.empty((T, S), dtype=torch.int64, device="cuda")
    e = torch.empty((T, K_in), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((T, N_out), dtype=torch.bfloat16, device="cuda")
    pws_n = E.engram_project_workspace_size(T, K_in, N_out, 0)
    pws = torch.empty(max(pws_n, 1), dtype=torch.uint8, device="cuda")
    # each stage alone, `steps` back-to-back calls between two events (an event
    # between every launch would add its idle gap to every stage)
    def per_stage(fn):
        for _ in range(2):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    st = [per_stage(lambda: E.engram_hash(gw.params, gw.ids, w.batch, w.seq, hist, None, rows)),
          per_stage(lambda: E.engram_gather(gw.table, gw.rows, gw.row_format, w.row_dim, rows,
                                            T * S, e)),
          per_stage(lambda: E.engram_project(e, gw.wkv, kv, T, K_in, N_out, gw.wkv_ld, 0, pws,
                                             pws_n)),
          per_stage(lambda: E.engram_gate(gw.desc, gw.ids, w.raw_vocab, kv, gw.q_w, gw.k_w,
                                          gw.h, gates))]
    wkv_bytes = N_out * K_in * 2
    # the same decode step with the short convolution branch: each sequence's
    # 9-position history is read and shifted in place every step
    g = torch.Generator(device="cuda").manual_seed(78)
    cw = 0.3 * torch.randn((w.hc, w.dim, 4), generator=g, device="cuda")
    sv = torch.zeros((w.batch, 9, w.dim), dtype=torch.bfloat16, device="cuda")
    ss = torch.zeros((w.batch, 9, w.hc + 1), dtype=torch.float32, device="cuda")
    conv = E.short_conv(cw, 4, 3, 1e-6, None, sv, ss, sv, ss)
    ncw = E.engram_forward_conv_workspace_size(gw.params, gw.desc)
    cws = torch.empty(ncw, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        E.engram_forward_conv(gw.params, gw.desc, conv, gw.ids, hist, hist, gw.table, gw.wkv,
                              gw.q_w, gw.k_w, gw.h, gates, cws, ncw)
    torch.cuda.synchronize()
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record(stream)
    for i in range(steps):
        E.engram_forward_conv(gw.params, gw.desc, conv, gw.ids, hist, hist, gw.table, gw.wkv,
                              gw.q_w, gw.k_w, gw.h, gates, cws, ncw)
    ce[1].record(stream)
    torch.cuda.synchronize()
    conv_ms = ce[0].elapsed_time(ce[1]) / steps
    del cws, sv, ss, cw
    # the same decode step with the block-scaled FP8 weight (quantised from the
    # same wkv): engram_forward_mx, the history in place
    from workloads import gen
    from workloads.device import to_device
    codes, scales = gen.wkv_mx(w)
    wc, wsc = to_device(codes), to_device(scales)
    del codes, scales
    nmx = E.engram_forward_mx_workspace_size(gw.params, gw.desc)
    mws = torch.empty(max(nmx, 1), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        E.engram_forward_mx(gw.params, gw.desc, gw.ids, hist, hist, gw.table, wc, wsc, gw.q_w,
                            gw.k_w, gw.h, gates, mws, nmx)
    torch.cuda.synchronize()
    me = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    me[0].record(stream)
    for i in range(steps):
        E.engram_forward_mx(gw.params, gw.desc, gw.ids, hist, hist, gw.table, wc, wsc, gw.q_w,
                            gw.k_w, gw.h, gates, mws, nmx)
    me[1].record(stream)
    torch.cuda.synchronize()
    mx_ms = me[0].elapsed_time(me[1]) / steps
    del wc, wsc, mws
    res = {"workload": "decode: 256 sequences x 1 token with a 3-token history, 24 segments of "
                       "primes from 16,000,000 (384,006,168 x 264 B = 101.4 GB table), hc 4 x 5120, "
                       f"wkv rows {gw.wkv_ld} elements apart",
           "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
           "graph_replay": {"tokens_per_s": round(T / (graph_ms * 1e-3), 1),
                            "ms_per_step": round(graph_ms, 4)},
           "stages_ms": {"hash": round(st[0], 4), "gather": round(st[1], 4),
                         "project": round(st[2], 4), "gate": round(st[3], 4)},
           "stages_method": "each stage alone, back-to-back calls between two events; the "
                            "hash and gather kernels (5-6 us, profiles/decode_c4_kernel_stats.md) "
                            "are shorter than one call through the binding (about 10 us), so "
                            "their figures are the host's issue rate",
           "project_weight_stream": {"achieved": round(wkv_bytes / (st[2] * 1e-3) / 1e9, 1),
                                     "peak": HBM_PEAK_GBPS, "unit": "GB/s"},
           "short_conv": {"workload": "the same step through engram_forward_conv (4 taps, "
                                      "dilation 3, 9-position history in place)",
                          "tokens_per_s": round(T / (conv_ms * 1e-3), 1),
                          "ms_per_step": round(conv_ms, 4)},
           "fp8_wkv": {"workload": "the same step through engram_forward_mx, the projection "
                                   "weight in block-scaled FP8 (E4M3 + one E8M0 scale per 32 "
                                   "inputs)",
                       "tokens_per_s": round(T / (mx_ms * 1e-3), 1),
                       "ms_per_step": round(mx_ms, 4)}}
    gw.free()
    return res


if __name__ == "__main__":
    main()
