"""ctypes binding of libengram.so (include/engram.h).

Argument marshalling only: torch tensors are passed as raw device pointers and
every step runs in the library's HIP kernels. There is no fallback: importing
this module fails loudly when the built library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

# ENGRAM_LIBRARY selects another build of the same library (the host-sanitized
# one the CPU tests run); by default the in-tree libengram.so is loaded.
_LIB_PATH = os.environ.get("ENGRAM_LIBRARY") or \
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "libengram.so")

DEAD = -1
MAX_NGRAM = 8
MAX_SEGMENTS = 64
MAX_LAYERS = 4
MAX_TOTAL_SEGMENTS = 128
ROW_BYTES = 264
ROW_E4M3_E8M0_264 = 0
ROW_F32 = 1
GATE_SIGNED_SQRT = 0
GATE_PLAIN = 1
MAX_CONV_TAPS = 8
MAX_CONV_HISTORY = 64

OK, EINVAL, EVOCAB, EMULT, ESHAPE, EWORKSPACE, EHIP, EPRIMES, ESCRATCH = \
    0, -1, -2, -3, -4, -5, -6, -7, -8


class EngramError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {status_string(status)} (status {status})"
        if status == EHIP:
            msg += f": {LIB.engram_last_hip_error().decode()}"
        super().__init__(msg)


class HashParams(ctypes.Structure):
    _fields_ = [
        ("raw_vocab", ctypes.c_int32),
        ("compressed_vocab", ctypes.c_int32),
        ("max_ngram", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("pad_id", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("token_map", ctypes.c_void_p),
        ("multipliers", ctypes.c_int64 * MAX_NGRAM),
        ("primes", ctypes.c_int64 * MAX_SEGMENTS),
        ("offsets", ctypes.c_int64 * MAX_SEGMENTS),
    ]


class ForwardDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seq", ctypes.c_int64),
        ("hc", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("table_rows", ctypes.c_int64),
        ("row_format", ctypes.c_int32),
        ("row_dim", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("gate_clamp", ctypes.c_float),
        ("gate_mode", ctypes.c_int32),
        ("wkv_ld", ctypes.c_int32),
    ]


class ShortConv(ctypes.Structure):
    _fields_ = [
        ("taps", ctypes.c_int32),
        ("dilation", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("weight", ctypes.c_void_p),
        ("norm_weight", ctypes.c_void_p),
        ("state_v_in", ctypes.c_void_p),
        ("state_s_in", ctypes.c_void_p),
        ("state_v_out", ctypes.c_void_p),
        ("state_s_out", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python hashed_gram_conditional_amd/build.py)")
    # The library needs libamdhip64.so.7. torch ships its own HIP runtime under
    # that soname and loads it by another name; if the library were loaded
    # first, the process would end up with two HIP runtimes and the library's
    # would see no device. Importing torch first makes the dynamic linker bind
    # the library to torch's runtime, the one that owns the device memory and
    # streams the library is handed.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "engram_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "engram_last_hip_error": (ctypes.c_char_p, []),
        "engram_sizeof_hash_params": (SZ, []),
        "engram_sizeof_forward_desc": (SZ, []),
        "engram_sizeof_short_conv": (SZ, []),
        "engram_gate_conv_workspace_size": (SZ, [P]),
        "engram_gate_conv": (ctypes.c_int, [P, P, P, I32, P, P, P, P, P, P, SZ, P]),
        "engram_forward_conv_workspace_size": (SZ, [P, P]),
        "engram_forward_conv": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "engram_make_primes": (ctypes.c_int, [I64, I32, P, P, P]),
        "engram_make_layer_primes": (ctypes.c_int, [I64, I32, I32, P, P, P]),
        "engram_hash_layers": (ctypes.c_int, [P, I32, P, I64, I64, P, P, P, P]),
        "engram_check_token_map": (ctypes.c_int, [P, I32, I32]),
        "engram_hash": (ctypes.c_int, [P, P, I64, I64, P, P, P, P]),
        "engram_gather": (ctypes.c_int, [P, I64, I32, I32, P, I64, P, P]),
        "engram_project": (ctypes.c_int, [P, P, P, I64, I64, I64, I64, I32, P, SZ, P]),
        "engram_wkv_row_stride": (I64, [I64, I32]),
        "engram_project_workspace_size": (SZ, [I64, I64, I64, I32]),
        "engram_gate": (ctypes.c_int, [P, P, I32, P, P, P, P, P, P]),
        "engram_fold_gate_weights": (ctypes.c_int, [P, P, I32, I32, P, P]),
        "engram_gate_folded": (ctypes.c_int, [P, P, I32, P, P, P, P, P]),
        "engram_project_gate_sums": (ctypes.c_int, [P, P, I64, P, P, P, P, P]),
        "engram_gate_sums": (ctypes.c_int, [P, P, I32, P, P, P, P]),
        "engram_project_mx_gate_sums": (ctypes.c_int, [P, P, P, I32, P, P, P, P, P, P]),
        "engram_gate_conv_sums": (ctypes.c_int, [P, P, P, I32, P, P, P, P, SZ, P]),
        "engram_forward_workspace_size": (SZ, [P, P]),
        "engram_gather_rows": (ctypes.c_int, [P, I64, P, I64, P, P]),
        "engram_project_mx": (ctypes.c_int, [P, P, I32, P, P, P, I64, I64, P, SZ, P]),
        "engram_gather_mx": (ctypes.c_int, [P, I64, P, I64, P, P, P]),
        "engram_project_mx_workspace_size": (SZ, [I64, I32, I64]),
        "engram_forward_mx_workspace_size": (SZ, [P, P]),
        "engram_forward_mx": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "engram_forward": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "engram_forward_static": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P, P, P]),
        "engram_forward_static_max_bytes": (SZ, []),
        "engram_transpose": (ctypes.c_int, [P, P, I64, I64, I64, I32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.engram_sizeof_hash_params() != ctypes.sizeof(HashParams):
        raise ImportError("engram_hash_params layout mismatch between binding and library")
    if lib.engram_sizeof_forward_desc() != ctypes.sizeof(ForwardDesc):
        raise ImportError("engram_forward_desc layout mismatch between binding and library")
    if lib.engram_sizeof_short_conv() != ctypes.sizeof(ShortConv):
        raise ImportError("engram_short_conv layout mismatch between binding and library")
    return lib


LIB = _load()
LIB_PATH = _LIB_PATH


def status_string(status: int) -> str:
    return LIB.engram_status_string(int(status)).decode()


def _table_ptr(t) -> Optional[int]:
    """Address of a table argument: device memory or pinned host memory (the
    library checks which and rejects pageable memory with ENGRAM_EINVAL)."""
    if t is None or isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("engram: a table tensor must be contiguous")
    return t.data_ptr()


def _ptr(t) -> Optional[int]:
    """Address of a tensor the kernels read or write in place: contiguous, and in
    device memory or pinned host memory (a pageable host tensor would fault)."""
    if t is None or isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("engram: tensors must be contiguous")
    if not t.is_cuda and not t.is_pinned():
        raise ValueError("engram: a host tensor must be pinned for the GPU to reach it")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != OK:
        raise EngramError(status, where)


def hash_params(raw_vocab: int, compressed_vocab: int, max_ngram: int, heads: int,
                pad_id: int, token_map, multipliers: Sequence[int], primes: Sequence[int],
                offsets: Sequence[int]) -> HashParams:
    """Fill an engram_hash_params (token_map: device int32 tensor or pointer)."""
    p = HashParams()
    p.raw_vocab, p.compressed_vocab = raw_vocab, compressed_vocab
    p.max_ngram, p.heads, p.pad_id, p.reserved = max_ngram, heads, pad_id, 0
    p.token_map = _ptr(token_map)
    for i, m in enumerate(multipliers):
        p.multipliers[i] = int(m)
    for j, (pr, off) in enumerate(zip(primes, offsets)):
        p.primes[j] = int(pr)
        p.offsets[j] = int(off)
    return p


def forward_desc(batch: int, seq: int, hc: int, dim: int, table_rows: int, row_format: int,
                 row_dim: int, eps: float = 1e-6, gate_clamp: float = 0.0,
                 gate_mode: int = GATE_SIGNED_SQRT, wkv_ld: int = 0) -> ForwardDesc:
    d = ForwardDesc()
    d.batch, d.seq, d.hc, d.dim = batch, seq, hc, dim
    d.table_rows, d.row_format, d.row_dim = table_rows, row_format, row_dim
    d.eps, d.gate_clamp, d.gate_mode, d.wkv_ld = eps, gate_clamp, gate_mode, wkv_ld
    return d


def short_conv(weight, taps: int = 4, dilation: int = 3, eps: float = 1e-6, norm_weight=None,
               state_v_in=None, state_s_in=None, state_v_out=None,
               state_s_out=None) -> ShortConv:
    """The short convolution branch's descriptor; tensors are kept by the caller."""
    c = ShortConv()
    c.taps, c.dilation, c.eps = taps, dilation, eps
    c.weight, c.norm_weight = _ptr(weight), _ptr(norm_weight)
    c.state_v_in, c.state_s_in = _ptr(state_v_in), _ptr(state_s_in)
    c.state_v_out, c.state_s_out = _ptr(state_v_out), _ptr(state_s_out)
    return c


def engram_make_primes(base: int, count: int):
    """[host] (primes, offsets, total_rows) of the first ``count`` primes >= base."""
    pr = (ctypes.c_int64 * max(count, 1))()
    off = (ctypes.c_int64 * max(count, 1))()
    tot = ctypes.c_int64()
    _check(LIB.engram_make_primes(base, count, ctypes.addressof(pr), ctypes.addressof(off),
                                  ctypes.addressof(tot)), "engram_make_primes")
    return list(pr)[:count], list(off)[:count], tot.value


def engram_make_layer_primes(base: int, layers: int, per_layer: int):
    """[host] (primes, offsets, rows), each a list per layer: one ascending prime
    sequence from ``base`` dealt to the layers, offsets restarting per layer."""
    n = max(layers * per_layer, 1)
    pr = (ctypes.c_int64 * n)()
    off = (ctypes.c_int64 * n)()
    rows = (ctypes.c_int64 * max(layers, 1))()
    _check(LIB.engram_make_layer_primes(base, layers, per_layer, ctypes.addressof(pr),
                                        ctypes.addressof(off), ctypes.addressof(rows)),
           "engram_make_layer_primes")
    cut = lambda a: [list(a)[l * per_layer:(l + 1) * per_layer] for l in range(layers)]
    return cut(pr), cut(off), list(rows)[:layers]


def engram_check_token_map(token_map, raw_vocab: int, compressed_vocab: int) -> int:
    """[host] status of the start-up check of a host int32 map (numpy array)."""
    import numpy as np
    arr = np.ascontiguousarray(token_map, dtype=np.int32)
    return LIB.engram_check_token_map(arr.ctypes.data, raw_vocab, compressed_vocab)


def engram_hash(params: HashParams, ids, batch: int, seq: int, hist_in, hist_out, row_ids,
                stream=None):
    _check(LIB.engram_hash(ctypes.byref(params), _ptr(ids), batch, seq, _ptr(hist_in),
                           _ptr(hist_out), _ptr(row_ids), _stream(stream)), "engram_hash")


def engram_hash_layers(params: Sequence[HashParams], ids, batch: int, seq: int, hist_in,
                       hist_out, row_ids, stream=None):
    """Row ids of len(params) layers into row_ids [layers, batch*seq, S]."""
    arr = (HashParams * len(params))(*params)
    _check(LIB.engram_hash_layers(ctypes.addressof(arr), len(params), _ptr(ids), batch, seq,
                                  _ptr(hist_in), _ptr(hist_out), _ptr(row_ids), _stream(stream)),
           "engram_hash_layers")


def engram_gather(table, table_rows: int, row_format: int, row_dim: int, row_ids, n_ids: int,
                  out, stream=None):
    _check(LIB.engram_gather(_table_ptr(table), table_rows, row_format, row_dim, _ptr(row_ids),
                             n_ids, _ptr(out), _stream(stream)), "engram_gather")


def engram_project_workspace_size(tokens: int, in_dim: int, out_dim: int, act_f32: int) -> int:
    return LIB.engram_project_workspace_size(tokens, in_dim, out_dim, act_f32)


def engram_project(e, wkv, kv, tokens: int, in_dim: int, out_dim: int, wkv_ld: int,
                   act_f32: int, workspace=None, workspace_bytes: int = 0, stream=None):
    _check(LIB.engram_project(_ptr(e), _ptr(wkv), _ptr(kv), tokens, in_dim, out_dim, wkv_ld,
                              act_f32,
                              _ptr(workspace), workspace_bytes, _stream(stream)),
           "engram_project")


def engram_gate(desc: ForwardDesc, ids, raw_vocab: int, kv, q_w, k_w, h, gate_out,
                stream=None):
    _check(LIB.engram_gate(ctypes.byref(desc), _ptr(ids), raw_vocab, _ptr(kv), _ptr(q_w),
                           _ptr(k_w), _ptr(h), _ptr(gate_out), _stream(stream)), "engram_gate")


def engram_fold_gate_weights(q_w, k_w, hc: int, dim: int, qk_w, stream=None):
    """qk_w [hc, dim] = q_w * k_w (fp32), the gate's scales folded once."""
    _check(LIB.engram_fold_gate_weights(_ptr(q_w), _ptr(k_w), hc, dim, _ptr(qk_w),
                                        _stream(stream)), "engram_fold_gate_weights")


def engram_gate_folded(desc: ForwardDesc, ids, raw_vocab: int, kv, qk_w, h, gate_out,
                       stream=None):
    _check(LIB.engram_gate_folded(ctypes.byref(desc), _ptr(ids), raw_vocab, _ptr(kv),
                                  _ptr(qk_w), _ptr(h), _ptr(gate_out), _stream(stream)),
           "engram_gate_folded")


def engram_project_gate_sums(desc: ForwardDesc, e, in_dim: int, wkv, h, qk_w, kv, stream=None):
    """The projection with the gate's key-side sums in kv's key columns."""
    _check(LIB.engram_project_gate_sums(ctypes.byref(desc), _ptr(e), in_dim, _ptr(wkv), _ptr(h),
                                        _ptr(qk_w), _ptr(kv), _stream(stream)),
           "engram_project_gate_sums")


def engram_project_mx_gate_sums(desc: ForwardDesc, e_codes, e_scales, segments: int, w_codes,
                                w_scales, h, qk_w, kv, stream=None):
    """engram_project_gate_sums with the block-scaled FP8 weight."""
    _check(LIB.engram_project_mx_gate_sums(ctypes.byref(desc), _ptr(e_codes), _ptr(e_scales),
                                           segments, _ptr(w_codes), _ptr(w_scales), _ptr(h),
                                           _ptr(qk_w), _ptr(kv), _stream(stream)),
           "engram_project_mx_gate_sums")


def engram_gate_conv_sums(desc: ForwardDesc, conv: ShortConv, ids, raw_vocab: int, kv, h,
                          gate_out, workspace, workspace_bytes: int, stream=None):
    """engram_gate_conv from engram_project_gate_sums' kv."""
    _check(LIB.engram_gate_conv_sums(ctypes.byref(desc), ctypes.byref(conv), _ptr(ids), raw_vocab,
                                     _ptr(kv), _ptr(h), _ptr(gate_out), _ptr(workspace),
                                     workspace_bytes, _stream(stream)), "engram_gate_conv_sums")


def engram_gate_sums(desc: ForwardDesc, ids, raw_vocab: int, kv, h, gate_out, stream=None):
    """The gate and residual update from engram_project_gate_sums' kv."""
    _check(LIB.engram_gate_sums(ctypes.byref(desc), _ptr(ids), raw_vocab, _ptr(kv), _ptr(h),
                                _ptr(gate_out), _stream(stream)), "engram_gate_sums")


def engram_forward_workspace_size(params: HashParams, desc: ForwardDesc) -> int:
    return int(LIB.engram_forward_workspace_size(ctypes.byref(params), ctypes.byref(desc)))


def engram_forward(params: HashParams, desc: ForwardDesc, ids, hist_in, hist_out, table, wkv,
                   q_w, k_w, h, gate_out, workspace, workspace_bytes: int, stream=None):
    _check(LIB.engram_forward(ctypes.byref(params), ctypes.byref(desc), _ptr(ids),
                              _ptr(hist_in), _ptr(hist_out), _table_ptr(table), _ptr(wkv),
                              _ptr(q_w), _ptr(k_w), _ptr(h), _ptr(gate_out),
                              _ptr(workspace), workspace_bytes, _stream(stream)),
           "engram_forward")


def engram_forward_static(params: HashParams, desc: ForwardDesc, ids, hist_in, hist_out, table,
                          wkv, q_w, k_w, h, gate_out, stream=None):
    _check(LIB.engram_forward_static(ctypes.byref(params), ctypes.byref(desc), _ptr(ids),
                                     _ptr(hist_in), _ptr(hist_out), _table_ptr(table),
                                     _ptr(wkv), _ptr(q_w), _ptr(k_w), _ptr(h), _ptr(gate_out),
                                     _stream(stream)),
           "engram_forward_static")


def engram_transpose(src, dst, rows: int, cols: int, dst_ld: int, elem_bytes: int, stream=None):
    _check(LIB.engram_transpose(_ptr(src), _ptr(dst), rows, cols, dst_ld, elem_bytes,
                                _stream(stream)), "engram_transpose")


def engram_wkv_row_stride(in_dim: int, elem_bytes: int) -> int:
    return int(LIB.engram_wkv_row_stride(in_dim, elem_bytes))


def engram_forward_static_max_bytes() -> int:
    return int(LIB.engram_forward_static_max_bytes())


def engram_gather_rows(table, table_rows: int, row_ids, n_ids: int, out, stream=None):
    _check(LIB.engram_gather_rows(_table_ptr(table), table_rows, _ptr(row_ids), n_ids, _ptr(out),
                                  _stream(stream)), "engram_gather_rows")


def engram_project_mx_workspace_size(tokens: int, segments: int, out_dim: int) -> int:
    return LIB.engram_project_mx_workspace_size(tokens, segments, out_dim)


def engram_gather_mx(table, table_rows: int, row_ids, n_ids: int, codes, scales, stream=None):
    _check(LIB.engram_gather_mx(_table_ptr(table), table_rows, _ptr(row_ids), n_ids, _ptr(codes),
                                _ptr(scales), _stream(stream)), "engram_gather_mx")


def engram_project_mx(e_codes, e_scales, segments: int, w_codes, w_scales, kv, tokens: int,
                      out_dim: int, workspace=None, workspace_bytes: int = 0, stream=None):
    _check(LIB.engram_project_mx(_ptr(e_codes), _ptr(e_scales), segments, _ptr(w_codes),
                                 _ptr(w_scales), _ptr(kv), tokens, out_dim, _ptr(workspace),
                                 workspace_bytes, _stream(stream)), "engram_project_mx")


def engram_forward_mx_workspace_size(params: HashParams, desc: ForwardDesc) -> int:
    return LIB.engram_forward_mx_workspace_size(ctypes.byref(params), ctypes.byref(desc))


def engram_forward_mx(params: HashParams, desc: ForwardDesc, ids, hist_in, hist_out, table,
                      w_codes, w_scales, q_w, k_w, h, gate_out, workspace, workspace_bytes: int,
                      stream=None):
    _check(LIB.engram_forward_mx(ctypes.byref(params), ctypes.byref(desc), _ptr(ids),
                                 _ptr(hist_in), _ptr(hist_out), _table_ptr(table), _ptr(w_codes),
                                 _ptr(w_scales), _ptr(q_w), _ptr(k_w), _ptr(h), _ptr(gate_out),
                                 _ptr(workspace), workspace_bytes, _stream(stream)),
           "engram_forward_mx")


def engram_gate_conv_workspace_size(desc: ForwardDesc) -> int:
    return int(LIB.engram_gate_conv_workspace_size(ctypes.byref(desc)))


def engram_gate_conv(desc: ForwardDesc, conv: ShortConv, ids, raw_vocab: int, kv, q_w, k_w, h,
                     gate_out, workspace, workspace_bytes: int, stream=None):
    _check(LIB.engram_gate_conv(ctypes.byref(desc), ctypes.byref(conv), _ptr(ids), raw_vocab,
                                _ptr(kv), _ptr(q_w), _ptr(k_w), _ptr(h), _ptr(gate_out),
                                _ptr(workspace), workspace_bytes, _stream(stream)),
           "engram_gate_conv")


def engram_forward_conv_workspace_size(params: HashParams, desc: ForwardDesc) -> int:
    return int(LIB.engram_forward_conv_workspace_size(ctypes.byref(params), ctypes.byref(desc)))


def engram_forward_conv(params: HashParams, desc: ForwardDesc, conv: ShortConv, ids, hist_in,
                        hist_out, table, wkv, q_w, k_w, h, gate_out, workspace,
                        workspace_bytes: int, stream=None):
    _check(LIB.engram_forward_conv(ctypes.byref(params), ctypes.byref(desc), ctypes.byref(conv),
                                   _ptr(ids), _ptr(hist_in), _ptr(hist_out), _table_ptr(table),
                                   _ptr(wkv), _ptr(q_w), _ptr(k_w), _ptr(h), _ptr(gate_out),
                                   _ptr(workspace), workspace_bytes, _stream(stream)),
           "engram_forward_conv")
