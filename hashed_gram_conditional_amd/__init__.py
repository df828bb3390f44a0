"""Engram conditional-memory layer forward for MI355X (gfx950).

The computation runs in the HIP kernels of ``libengram.so`` behind the C ABI of
``include/engram.h``; this package is its thin Python binding (torch tensors
in, raw pointers out). Importing it fails if the library is not built.
"""
from ._binding import (  # noqa: F401
    DEAD, MAX_NGRAM, MAX_SEGMENTS, MAX_LAYERS, MAX_TOTAL_SEGMENTS, ROW_BYTES, ROW_E4M3_E8M0_264, ROW_F32,
    GATE_SIGNED_SQRT, GATE_PLAIN, MAX_CONV_TAPS, MAX_CONV_HISTORY,
    OK, EINVAL, EVOCAB, EMULT, ESHAPE, EWORKSPACE, EHIP, EPRIMES, ESCRATCH,
    EngramError, HashParams, ForwardDesc, ShortConv, LIB, LIB_PATH,
    status_string, hash_params, forward_desc, short_conv,
    engram_make_primes, engram_make_layer_primes, engram_check_token_map, engram_hash,
    engram_hash_layers, engram_gather,
    engram_project, engram_project_workspace_size, engram_gate, engram_fold_gate_weights,
    engram_gate_folded, engram_project_gate_sums, engram_gate_sums,
    engram_project_mx_gate_sums, engram_gate_conv_sums, engram_forward_workspace_size,
    engram_forward, engram_forward_static, engram_forward_static_max_bytes, engram_transpose,
    engram_wkv_row_stride,
    engram_gather_rows, engram_gather_mx, engram_project_mx, engram_project_mx_workspace_size,
    engram_forward_mx, engram_forward_mx_workspace_size,
    engram_gate_conv, engram_gate_conv_workspace_size, engram_forward_conv,
    engram_forward_conv_workspace_size,
)
