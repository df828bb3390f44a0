"""Device-side input generation (the table twin) and upload helpers."""
import ctypes
import os

import numpy as np

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libworkloads.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.workloads_fill_table.restype = ctypes.c_int
        lib.workloads_fill_table.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_uint64, ctypes.c_void_p]
        _LIB = lib
    return _LIB


def fill_table(table, seed: int, row_begin: int = 0, stream=None):
    """Fill a device uint8 tensor [rows, 264] with the counter-based table rows."""
    import torch
    assert table.dtype == torch.uint8 and table.dim() == 2 and table.shape[1] == 264
    assert table.is_contiguous()
    st = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = _lib().workloads_fill_table(table.data_ptr(), table.shape[0], row_begin,
                                     ctypes.c_uint64(seed & (2 ** 64 - 1)), st)
    if rc != 0:
        raise RuntimeError(f"workloads_fill_table failed: hip error {rc}")


def to_device(arr: np.ndarray, device="cuda"):
    """numpy -> torch device tensor; uint16 arrays become bfloat16 (bit copy)."""
    import torch
    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def bf16_bits(t) -> np.ndarray:
    """device bfloat16 tensor -> numpy uint16 bit patterns."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
