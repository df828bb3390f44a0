"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/engram.h declares, and rejects bad arguments before
launching anything (no compute call reaches the device here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from workloads import C0, C1, gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

E = pytest.importorskip("hashed_gram_conditional_amd")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# The validation tests hand the library made-up device addresses that every
# check must reject before any launch; they only run where no GPU is visible.
host_only = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: host-only test")


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(engram_[a-z_0-9]+)\s*\(",
                                src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 11, names
    lib = ctypes.CDLL(E.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layouts_match():
    assert E.LIB.engram_sizeof_hash_params() == ctypes.sizeof(E.HashParams)
    assert E.LIB.engram_sizeof_forward_desc() == ctypes.sizeof(E.ForwardDesc)


@pytest.mark.parametrize("base,count", [(1009, 6), (1_000_000, 24), (16_000_000, 48),
                                        (2, 30), (4_294_967_000, 3)])
def test_library_primes_equal_oracle_primes(base, count):
    p, off, tot = E.engram_make_primes(base, count)
    po = O.primes_from(base, count)
    oo, to = O.segment_offsets(po)
    assert p == po and off == oo and tot == to


@pytest.mark.parametrize("base,layers,per_layer", [(16_000_000, 2, 24), (1009, 3, 6),
                                                    (1_000_000, 4, 24), (2, 1, 5)])
def test_library_layer_primes_equal_oracle(base, layers, per_layer):
    assert E.engram_make_layer_primes(base, layers, per_layer) == \
        O.layer_primes(base, layers, per_layer)


def test_make_primes_rejects_beyond_32_bits():
    with pytest.raises(E.EngramError):
        E.engram_make_primes(4_294_967_290, 2)


def test_token_map_check():
    tm, _ = gen.hash_setup(C1)
    assert E.engram_check_token_map(tm, C1.raw_vocab, C1.compressed_vocab) == E.OK
    assert E.engram_check_token_map(tm, C1.raw_vocab, C1.compressed_vocab + 1) == E.EVOCAB
    bad = tm.copy()
    bad[5] = C1.compressed_vocab
    assert E.engram_check_token_map(bad, C1.raw_vocab, C1.compressed_vocab) == E.EVOCAB


def _params(w=C0, **kw):
    tm, mult = gen.hash_setup(w)
    p, off, _ = E.engram_make_primes(w.prime_base, w.segments)
    args = dict(raw_vocab=w.raw_vocab, compressed_vocab=w.compressed_vocab,
                max_ngram=w.max_ngram, heads=w.heads, pad_id=int(tm[0]), token_map=0x1000,
                multipliers=mult, primes=p, offsets=off)
    args.update(kw)
    return E.hash_params(**args)


def _hash_status(params, ids=0x2000, B=1, T=4, rows=0x3000):
    return E.LIB.engram_hash(ctypes.byref(params), ids, B, T, None, None, rows, None)


@host_only
def test_hash_argument_validation():
    _, mult = gen.hash_setup(C0)
    lim = O.multiplier_limit(C0.compressed_vocab)
    assert _hash_status(_params(multipliers=[mult[0] + 1] + mult[1:])) == E.EMULT   # even
    assert _hash_status(_params(multipliers=[lim + 2] + mult[1:])) == E.EMULT       # too big
    assert _hash_status(_params(multipliers=[-1] + mult[1:])) == E.EMULT
    p, off, _ = E.engram_make_primes(C0.prime_base, C0.segments)
    assert _hash_status(_params(offsets=[0] + off[2:] + [0])) == E.EPRIMES
    assert _hash_status(_params(primes=[1] + p[1:])) == E.EPRIMES
    assert _hash_status(_params(pad_id=C0.compressed_vocab)) == E.EINVAL
    assert _hash_status(_params(token_map=0)) == E.EINVAL
    assert _hash_status(_params(max_ngram=9)) == E.ESHAPE
    assert _hash_status(_params(max_ngram=1)) == E.ESHAPE
    assert _hash_status(_params(heads=0)) == E.ESHAPE
    assert _hash_status(_params(), ids=0x2001) == E.EINVAL          # misaligned
    assert _hash_status(_params(), ids=None) == E.EINVAL
    assert _hash_status(_params(), B=-1) == E.ESHAPE
    # B * T beyond int64 must not wrap into an accepted token count
    assert _hash_status(_params(), B=1 << 40, T=1 << 40) == E.ESHAPE
    assert _hash_status(_params(), B=1 << 31, T=1 << 32) == E.ESHAPE


def _hash_layers_status(params, layers=None, ids=0x2000, B=1, T=4, rows=0x3000):
    arr = (E.HashParams * len(params))(*params)
    n = len(params) if layers is None else layers
    return E.LIB.engram_hash_layers(ctypes.addressof(arr), n, ids, B, T, None, None, rows, None)


@host_only
def test_hash_layers_validation():
    w = C1
    tm, _ = gen.hash_setup(w)
    mults = gen.layer_multipliers(w, 4)
    primes, offs, _ = E.engram_make_layer_primes(w.prime_base, 4, w.segments)

    def layer(li, **kw):
        args = dict(raw_vocab=w.raw_vocab, compressed_vocab=w.compressed_vocab,
                    max_ngram=w.max_ngram, heads=w.heads, pad_id=int(tm[0]), token_map=0x1000,
                    multipliers=mults[li], primes=primes[li], offsets=offs[li])
        args.update(kw)
        return E.hash_params(**args)

    two = [layer(0), layer(1)]
    assert _hash_layers_status(two, ids=None) == E.EINVAL         # shapes fine, ids null
    assert _hash_layers_status(two, layers=0) == E.ESHAPE
    assert _hash_layers_status(two * 3, layers=5) == E.ESHAPE
    assert _hash_layers_status([layer(0), layer(1, token_map=0x1100)]) == E.EINVAL
    assert _hash_layers_status([layer(0), layer(1, pad_id=int(tm[0]) + 1)]) == E.EINVAL
    assert _hash_layers_status([layer(0), layer(1, compressed_vocab=w.compressed_vocab - 1)]) \
        == E.EINVAL
    assert _hash_layers_status([layer(0), layer(1, multipliers=[2] + mults[1][1:])]) == E.EMULT
    assert _hash_layers_status([layer(0), layer(1, offsets=[0] * w.segments)]) == E.EPRIMES
    # 4 layers of 24 segments fit; 3 layers of 56 (N = 8, K = 8) exceed 128
    assert _hash_layers_status([layer(i) for i in range(4)], ids=None) == E.EINVAL
    big = E.engram_make_layer_primes(w.prime_base, 3, 56)
    wide = [E.hash_params(w.raw_vocab, w.compressed_vocab, 8, 8, int(tm[0]), 0x1000,
                          [1] * 8, big[0][i], big[1][i]) for i in range(3)]
    assert _hash_layers_status(wide) == E.ESHAPE


@host_only
def test_gather_project_gate_validation():
    L = E.LIB
    assert L.engram_gather(0x1000, 10, 0, 128, 0x2000, 4, 0x3000, None) == E.ESHAPE
    assert L.engram_gather(0x1000, 10, 7, 256, 0x2000, 4, 0x3000, None) == E.EINVAL
    assert L.engram_gather(0x1000, 10, 0, 256, 0x2004, 4, 0x3000, None) == E.EINVAL
    assert L.engram_gather(0x1000, 10, 1, 30, 0x2000, 4, 0x3000, None) == E.ESHAPE
    assert L.engram_gather(None, 0, 0, 256, None, 0, None, None) == E.OK      # empty
    assert L.engram_project(0x1000, 0x2000, 0x3000, 4, 100, 64, 0, 0, None, 0, None) == E.ESHAPE
    assert L.engram_project(0x1000, 0x2000, 0x3000, 4, 128, 60, 0, 0, None, 0, None) == E.ESHAPE
    assert L.engram_project(0x1000, 0x2000, 0x3000, 4, 128, 64, 0, 2, None, 0, None) == E.EINVAL
    assert L.engram_project(0x1008, 0x2000, 0x3000, 4, 128, 64, 0, 0, None, 0, None) == E.EINVAL
    assert L.engram_project(0x1000, 0x2000, 0x3000, 4, 128, 64, 0, 0, 0x4010, 1 << 30, None) \
        == E.EWORKSPACE                                              # not 256-aligned
    d = E.forward_desc(1, 4, 4, 5120, 100, 0, 256)
    bad = E.forward_desc(1, 4, 9, 5120, 100, 0, 256)
    assert L.engram_gate(ctypes.byref(bad), 0x1000, 10, 0x2000, 0x3000, 0x4000, 0x5000, None,
                         None) == E.ESHAPE
    bad = E.forward_desc(1, 4, 4, 5124, 100, 0, 256)
    assert L.engram_gate(ctypes.byref(bad), 0x1000, 10, 0x2000, 0x3000, 0x4000, 0x5000, None,
                         None) == E.ESHAPE
    assert L.engram_gate(ctypes.byref(d), None, 10, 0x2000, 0x3000, 0x4000, 0x5000, None,
                         None) == E.EINVAL


@host_only
def test_forward_validation_and_workspace_size():
    p = _params(C1)
    d = E.forward_desc(4, 8192, 4, 5120, 384_006_168, 0, 256)
    n = E.engram_forward_workspace_size(p, d)
    T = 4 * 8192
    assert n == T * 24 * 8 + T * 6144 * 2 + T * 25600 * 2 + 4 * 5120 * 4   # + folded scales
    L = E.LIB
    args = [0x1000, None, None, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None]
    assert L.engram_forward(ctypes.byref(p), ctypes.byref(d), *args, 0x10000, n - 1,
                            None) == E.EWORKSPACE
    assert L.engram_forward(ctypes.byref(p), ctypes.byref(d), *args, 0x10010, n,
                            None) == E.EWORKSPACE                   # not 256-aligned
    small = E.forward_desc(4, 8192, 4, 5120, 384_006_167, 0, 256)   # rows < sum of primes
    assert L.engram_forward(ctypes.byref(p), ctypes.byref(small), *args, 0x10000, n,
                            None) == E.EPRIMES
    assert E.status_string(E.EPRIMES).startswith("bad primes")
    for B, T in [(1 << 40, 1 << 40), (1 << 31, 2), (-1, 4)]:       # wraps, > 2^31 - 1, < 0
        big = E.forward_desc(B, T, 4, 5120, 384_006_168, 0, 256)
        assert E.engram_forward_workspace_size(p, big) == 0
        assert L.engram_forward(ctypes.byref(p), ctypes.byref(big), *args, 0x10000, n,
                                None) == E.ESHAPE


def test_one_hip_runtime_whatever_the_import_order():
    # torch carries its own HIP runtime; the library must bind to that one even
    # when it is imported first, or the process holds two runtimes and the
    # library's sees no device.
    import subprocess
    import sys
    code = ("import hashed_gram_conditional_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_gate_mode_and_short_conv_validation():
    """Bad gate modes and convolution descriptors fail before any launch."""
    L = E.LIB
    d = E.forward_desc(2, 16, 4, 64, 1 << 20, 0, 256)
    ptrs = [0x1000, 8, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000]     # ids, V, kv, qw, kw, h, gate
    ws = E.engram_gate_conv_workspace_size(d)
    assert ws == 2 * 16 * 5 * 4 + (-(2 * 16 * 5 * 4) % 256)

    def gc(desc, conv, wsp=0x10000, wsb=ws):
        return L.engram_gate_conv(ctypes.byref(desc), ctypes.byref(conv), *ptrs, wsp, wsb, None)

    ok = E.short_conv(0x7000)
    bad_mode = E.forward_desc(2, 16, 4, 64, 1 << 20, 0, 256, gate_mode=2)
    assert gc(bad_mode, ok) == E.EINVAL
    assert L.engram_gate(ctypes.byref(bad_mode), *ptrs, None) == E.EINVAL
    d_res = E.forward_desc(2, 16, 4, 64, 1 << 20, 0, 256, wkv_ld=-1)
    assert gc(d_res, ok) == E.ESHAPE
    assert gc(d, E.short_conv(0x7000, taps=0)) == E.ESHAPE
    assert gc(d, E.short_conv(0x7000, taps=9)) == E.ESHAPE
    assert gc(d, E.short_conv(0x7000, dilation=0)) == E.ESHAPE
    assert gc(d, E.short_conv(0x7000, taps=8, dilation=10)) == E.ESHAPE    # history 70 > 64
    assert gc(d, E.short_conv(0x7000, eps=0.0)) == E.EINVAL
    assert gc(d, E.short_conv(None)) == E.EINVAL
    assert gc(d, E.short_conv(0x7004)) == E.EINVAL                         # weight misaligned
    assert gc(d, E.short_conv(0x7000, state_v_in=0x8000)) == E.EINVAL     # half a history
    assert gc(d, E.short_conv(0x7000, state_v_out=0x8000)) == E.EINVAL
    assert gc(d, E.short_conv(0x7000, state_v_in=0x8008, state_s_in=0x9000)) == E.EINVAL
    res = E.short_conv(0x7000)
    res.reserved = 3
    assert gc(d, res) == E.EINVAL
    assert gc(d, ok, wsb=ws - 1) == E.EWORKSPACE
    assert gc(d, ok, wsp=0x10040) == E.EWORKSPACE
    assert gc(d, ok, wsp=None) == E.EWORKSPACE
    assert L.engram_gate_conv(ctypes.byref(d), None, *ptrs, 0x10000, ws, None) == E.EINVAL


def test_forward_conv_workspace_and_validation():
    p = _params(C1)
    d = E.forward_desc(4, 8192, 4, 5120, 384_006_168, 0, 256)
    T = 4 * 8192
    n = E.engram_forward_conv_workspace_size(p, d)
    assert n == E.engram_forward_workspace_size(p, d) + T * 5 * 4
    L = E.LIB
    args = [0x1000, None, None, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None]
    conv = E.short_conv(0x7000)
    assert L.engram_forward_conv(ctypes.byref(p), ctypes.byref(d), ctypes.byref(conv), *args,
                                 0x10000, n - 1, None) == E.EWORKSPACE
    assert L.engram_forward_conv(ctypes.byref(p), ctypes.byref(d), None, *args, 0x10000, n,
                                 None) == E.EINVAL
    bad = E.short_conv(0x7000, taps=0)
    assert L.engram_forward_conv(ctypes.byref(p), ctypes.byref(d), ctypes.byref(bad), *args,
                                 0x10000, n, None) == E.ESHAPE


def test_binding_rejects_tensors_the_kernels_cannot_read():
    import torch
    from hashed_gram_conditional_amd import _binding as B
    t = torch.zeros(8, 4, dtype=torch.int32)
    with pytest.raises(ValueError, match="pinned"):
        B._ptr(t)                                   # pageable host memory
    with pytest.raises(ValueError, match="contiguous"):
        B._ptr(t.t())
    with pytest.raises(ValueError, match="contiguous"):
        B._table_ptr(t.t())
    assert B._table_ptr(t) == t.data_ptr()          # the library checks tables itself
    assert B._ptr(None) is None and B._ptr(0x1000) == 0x1000


@host_only
def test_fold_and_folded_gate_validation():
    L = E.LIB
    assert L.engram_fold_gate_weights(0x1000, 0x2000, 0, 64, 0x3000, None) == E.ESHAPE
    assert L.engram_fold_gate_weights(0x1000, 0x2000, 4, 60, 0x3000, None) == E.ESHAPE
    assert L.engram_fold_gate_weights(0x1000, 0x2000, 9, 64, 0x3000, None) == E.ESHAPE
    assert L.engram_fold_gate_weights(None, 0x2000, 4, 64, 0x3000, None) == E.EINVAL
    assert L.engram_fold_gate_weights(0x1000, 0x2000, 4, 64, None, None) == E.EINVAL
    assert L.engram_fold_gate_weights(0x1004, 0x2000, 4, 64, 0x3000, None) == E.EINVAL
    d = E.forward_desc(2, 8, 4, 64, 100, 0, 256)
    gf = lambda desc, qk: L.engram_gate_folded(ctypes.byref(desc), 0x1000, 100, 0x2000, qk,
                                               0x4000, None, None)
    assert gf(d, None) == E.EINVAL
    assert gf(d, 0x3008) == E.EINVAL                                 # misaligned scales
    assert gf(E.forward_desc(2, 8, 9, 64, 100, 0, 256), 0x3000) == E.ESHAPE
    assert L.engram_gate_folded(ctypes.byref(d), 0x1000, 0, 0x2000, 0x3000, 0x4000, None,
                                None) == E.EINVAL                    # raw_vocab < 1


@host_only
def test_gate_sums_validation():
    """engram_project_gate_sums / engram_project_mx_gate_sums / engram_gate_sums /
    engram_gate_conv_sums: bf16 rows and dim % 256 only, the projections' shape
    rules, every pointer present and aligned, the convolution's workspace."""
    L = E.LIB
    bf16 = E.ROW_E4M3_E8M0_264
    d = E.forward_desc(2, 300, 4, 512, 100, bf16, 256, wkv_ld=1032)
    ps = lambda desc, k=1024, e=0x1000, w=0x2000, h=0x3000, qk=0x4000, kv=0x5000: \
        L.engram_project_gate_sums(ctypes.byref(desc), e, k, w, h, qk, kv, None)
    for bad_k in (0, 1000, -64):
        assert ps(d, k=bad_k) == E.ESHAPE
    assert ps(E.forward_desc(2, 300, 4, 320, 100, bf16, 256)) == E.ESHAPE     # dim % 256
    assert ps(E.forward_desc(2, 300, 4, 512, 100, E.ROW_F32, 32)) == E.EINVAL
    assert ps(E.forward_desc(2, 300, 4, 512, 100, bf16, 256, wkv_ld=1000)) == E.ESHAPE
    assert ps(E.forward_desc(2, 300, 4, 512, 100, bf16, 256, wkv_ld=1028)) == E.ESHAPE
    assert ps(E.forward_desc(0, 300, 4, 512, 100, bf16, 256), e=None) == E.OK  # no tokens
    for name in ("e", "w", "h", "qk", "kv"):
        assert ps(d, **{name: None}) == E.EINVAL, name
        assert ps(d, **{name: 0x6008}) == E.EINVAL, name
    big = E.forward_desc(1 << 15, 1 << 15, 4, 512, 100, bf16, 256)
    assert ps(big) == E.ESHAPE                            # beyond the tile bound
    gs = lambda desc, ids=0x1000, vocab=100, kv=0x2000, h=0x3000, g=None: \
        L.engram_gate_sums(ctypes.byref(desc), ids, vocab, kv, h, g, None)
    assert gs(E.forward_desc(2, 8, 4, 320, 100, bf16, 256)) == E.ESHAPE
    assert gs(E.forward_desc(2, 8, 4, 512, 100, E.ROW_F32, 32)) == E.EINVAL
    assert gs(d, vocab=0) == E.EINVAL
    assert gs(E.forward_desc(2, 8, 9, 512, 100, bf16, 256)) == E.ESHAPE     # hc > 8
    for kw in ({"ids": None}, {"kv": None}, {"h": None}, {"ids": 0x1002}, {"kv": 0x2008},
               {"h": 0x3008}, {"g": 0x4002}):
        assert gs(d, **kw) == E.EINVAL, kw
    assert gs(E.forward_desc(0, 8, 4, 512, 100, bf16, 256), ids=None) == E.OK
    pm = lambda desc, segs=4, ec=0x1000, es=0x2000, wc=0x3000, wsc=0x4000, h=0x5000, qk=0x6000, \
        kv=0x7000: L.engram_project_mx_gate_sums(ctypes.byref(desc), ec, es, segs, wc, wsc, h, qk,
                                                 kv, None)
    for segs in (0, 65):
        assert pm(d, segs=segs) == E.ESHAPE
    assert pm(E.forward_desc(2, 300, 4, 320, 100, bf16, 256)) == E.ESHAPE
    assert pm(E.forward_desc(2, 300, 4, 512, 100, E.ROW_F32, 32)) == E.EINVAL
    assert pm(big) == E.ESHAPE
    for name, bad in (("ec", 0x1008), ("es", 0x2002), ("wc", 0x3008), ("wsc", 0x4002),
                      ("h", 0x5008), ("qk", 0x6008), ("kv", 0x7008)):
        assert pm(d, **{name: None}) == E.EINVAL, name
        assert pm(d, **{name: bad}) == E.EINVAL, name
    assert pm(E.forward_desc(0, 300, 4, 512, 100, bf16, 256), ec=None) == E.OK
    conv = E.short_conv(0x8000, 4, 3, 1e-6)
    ws_need = E.engram_gate_conv_workspace_size(d)
    gc = lambda desc, ids=0x1000, kv=0x2000, h=0x3000, g=None, ws=0x10000, n=ws_need, cv=conv: \
        L.engram_gate_conv_sums(ctypes.byref(desc), ctypes.byref(cv), ids, 100, kv, h, g, ws, n,
                                None)
    assert gc(E.forward_desc(2, 300, 4, 320, 100, bf16, 256)) == E.ESHAPE
    assert gc(E.forward_desc(2, 300, 4, 512, 100, E.ROW_F32, 32)) == E.EINVAL
    for kw in ({"ids": None}, {"kv": None}, {"h": None}, {"kv": 0x2008}, {"g": 0x4002}):
        assert gc(d, **kw) == E.EINVAL, kw
    assert gc(d, ws=None) == E.EWORKSPACE
    assert gc(d, n=ws_need - 1) == E.EWORKSPACE
    assert gc(d, ws=0x10010) == E.EWORKSPACE
    bad_conv = E.short_conv(0x8000, 9, 3, 1e-6)
    assert gc(d, cv=bad_conv) == E.ESHAPE


def test_forward_static_refuses_calls_beyond_its_array():
    """engram_forward_static checks its scratch need on the host, before it
    looks up the array or launches anything."""
    p = _params(C1)
    L = E.LIB
    cap = E.engram_forward_static_max_bytes()
    assert cap == 64 << 20
    per_token = 24 * 8 + 6144 * 2 + 25600 * 2
    args = [0x1000, None, None, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, None]
    fits = cap // per_token - 4
    big = E.forward_desc(fits + 64, 1, 4, 5120, 384_006_168, 0, 256)
    assert L.engram_forward_static(ctypes.byref(p), ctypes.byref(big), *args) == E.ESCRATCH
    assert "static array" in E.status_string(E.ESCRATCH)
    bad = E.forward_desc(4, 8192, 9, 5120, 384_006_168, 0, 256)      # hc > 8
    assert L.engram_forward_static(ctypes.byref(p), ctypes.byref(bad), *args) == E.ESHAPE


@host_only
def test_projection_shapes_beyond_32_bit_offsets_are_refused():
    """The bf16 kernels address a 256-row panel with 32-bit byte counts: in_dim
    above 2^20, or a grid beyond 2^32 threads, is refused before any launch
    (rather than wrapping the record and returning zeros or garbage)."""
    L = E.LIB
    ok = L.engram_project(0x1000, 0x2000, 0x3000, 4, 1 << 20, 64, 0, 0, None, 0, None)
    assert ok != E.ESHAPE                     # fake pointers: any later status but ESHAPE
    assert L.engram_project(0x1000, 0x2000, 0x3000, 4, (1 << 20) + 64, 64, 0, 0, None, 0,
                            None) == E.ESHAPE
    assert L.engram_project(0x1000, 0x2000, 0x3000, 4, 1 << 23, 64, 0, 0, None, 0, None) \
        == E.ESHAPE
    big_m, big_n = (1 << 31) - 1, 1 << 20     # 8.4 M x 8192 tiles
    assert L.engram_project(0x1000, 0x2000, 0x3000, big_m, 6144, big_n, 0, 0, None, 0,
                            None) == E.ESHAPE
    assert L.engram_project_mx(0x1000, 0x2000, 24, 0x3000, 0x4000, 0x5000, big_m, big_n,
                               None, 0, None) == E.ESHAPE
    # the fp32 kernel indexes with 64-bit offsets: no in_dim limit of its own
    assert L.engram_project(0x1000, 0x2000, 0x3000, 0, (1 << 21), 64, 0, 1, None, 0,
                            None) == E.OK


@host_only
def test_transpose_validation():
    L = E.LIB
    assert L.engram_transpose(0x1000, 0x2000, 4, 8, 0, 3, None) == E.EINVAL      # 3-byte elements
    assert L.engram_transpose(0x1000, 0x1010, 4, 8, 0, 2, None) == E.EINVAL      # overlap
    assert L.engram_transpose(0x1001, 0x9000, 4, 8, 0, 2, None) == E.EINVAL      # misaligned
    assert L.engram_transpose(None, None, 0, 5, 0, 2, None) == E.OK              # empty
    assert L.engram_transpose(0x1000, 0x9000, -1, 5, 0, 2, None) == E.ESHAPE
    assert L.engram_transpose(0x1000, 1 << 44, 1 << 30, 1 << 20, 0, 2, None) == E.ESHAPE
    # a strided destination: dst_ld below rows, an extent beyond 2^62 bytes,
    # and an overlap that only the strided extent reaches
    assert L.engram_transpose(0x1000, 0x9000, 4, 8, 3, 2, None) == E.ESHAPE
    assert L.engram_transpose(0x1000, 0x9000, 4, 8, 1 << 61, 2, None) == E.ESHAPE
    assert L.engram_transpose(0x1100, 0x1000, 4, 8, 64, 2, None) == E.EINVAL


@host_only
def test_weight_row_stride_validation():
    """wkv_ld: 0 or >= in_dim, 16-byte multiples, at most 2^20 for bf16; the same
    rule through engram_forward_desc. Bad strides fail before any launch."""
    L = E.LIB
    args = (0x1000, 0x2000, 0x3000, 4, 128, 64)
    for ld in (64, 120, 132, (1 << 20) + 8, -8):
        assert L.engram_project(*args, ld, 0, None, 0, None) == E.ESHAPE, ld
    assert L.engram_project(0x1000, 0x2000, 0x3000, 4, 128, 64, 130, 1, None, 0, None) \
        == E.ESHAPE                                                  # fp32: 4-element rows
    assert L.engram_project(0x1000, 0x2000, 0x3000, 0, 128, 64, 136, 0, None, 0, None) == E.OK
    assert L.engram_project(0x1000, 0x2000, 0x3000, 0, 128, 64, 132, 1, None, 0, None) == E.OK
    p = _params(C1)
    fw = [0x1000, None, None, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None, 0x10000, 1 << 40,
          None]
    for ld in (-1, 6000, 6148):
        d = E.forward_desc(4, 8192, 4, 5120, 384_006_168, 0, 256, wkv_ld=ld)
        assert L.engram_forward(ctypes.byref(p), ctypes.byref(d), *fw) == E.ESHAPE, ld


def test_recommended_stride():
    assert E.engram_wkv_row_stride(6144, 2) == 6208      # 12 KiB rows -> 97 lines of 128 B
    assert E.engram_wkv_row_stride(1024, 2) == 1024      # 2 KiB rows stay dense
    assert E.engram_wkv_row_stride(6144, 4) == 6176
    assert E.engram_wkv_row_stride(100, 2) == 128        # rounded up to 128 bytes
    assert E.engram_wkv_row_stride(0, 2) == 0 and E.engram_wkv_row_stride(64, 3) == 0


def test_calibration_library_exports():
    """The benchmark's MFMA calibration library loads and exports its
    functions; bad arguments are refused before any launch."""
    path = os.path.join(ROOT, "hashed_gram_conditional_amd", "libengram_calibrate.so")
    if not os.path.exists(path):
        pytest.skip("libengram_calibrate.so not built")
    lib = ctypes.CDLL(path)
    lib.engram_calibrate_mfma_flop.restype = ctypes.c_double
    lib.engram_calibrate_mfma_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    assert lib.engram_calibrate_mfma_flop(256, 10) == 256 * 4 * 10 * 128 * 32768
    f = lib.engram_calibrate_mfma_bf16
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert f(None, 0x2000, 64, 0x3000, 1, 1, None) == -1
    assert f(0x1008, 0x2000, 64, 0x3000, 1, 1, None) == -1      # misaligned
    assert f(0x1000, 0x2000, 4, 0x3000, 1, 1, None) == -1        # fewer than 8 fragments
    assert f(0x1000, 0x2000, 64, 0x3000, 0, 1, None) == -1
    lib.engram_calibrate_mfma_fp8_flop.restype = ctypes.c_double
    lib.engram_calibrate_mfma_fp8_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    assert lib.engram_calibrate_mfma_fp8_flop(256, 10) == 256 * 4 * 10 * 128 * 131072
    f8 = lib.engram_calibrate_mfma_fp8
    f8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_void_p]
    assert f8(0x1010, 0x2000, 64, 0x4000, 0x5000, 8, 0x3000, 1, 1, None) == -1   # misaligned
    assert f8(0x1000, 0x2000, 64, None, 0x5000, 8, 0x3000, 1, 1, None) == -1
    assert f8(0x1000, 0x2000, 64, 0x4000, 0x5000, 0, 0x3000, 1, 1, None) == -1
