"""Device-side set-up of a workload for the tests, the benchmark and the smoke
check: uploads the seeded inputs, generates the table on the device and fills
the C-ABI argument structs through the library binding. Holds none of the
layer's arithmetic (the primes come from the library's own prime search)."""
from __future__ import annotations

import numpy as np

from . import gen
from .configs import EngramWorkload, ROW_F32
from .device import fill_table, to_device


class GpuWorkload:
    def __init__(self, w: EngramWorkload, device: str = "cuda", table: bool = True,
                 dense: bool = True, wkv_mx: bool = False, wkv_ld: int | None = None):
        """wkv_ld: row stride of the device wkv in elements; None takes the
        library's recommended stride (engram_wkv_row_stride), 0 dense rows. The
        gaps between rows hold NaN, which no kernel may read."""
        import torch
        import hashed_gram_conditional_amd as E

        self.w = w
        self.E = E
        self.device = device
        self.token_map_np, self.mult = gen.hash_setup(w)
        self.pad = int(self.token_map_np[0])
        self.primes, self.offsets, self.rows = E.engram_make_primes(w.prime_base, w.segments)
        self.ids_np, self.spans = gen.token_ids(w)
        self.hist_np = gen.history(w, self.token_map_np) if w.decode_history else None
        self.token_map = to_device(self.token_map_np, device)
        self.ids = to_device(self.ids_np, device)
        self.hist_in = to_device(self.hist_np, device) if self.hist_np is not None else None
        self.params = E.hash_params(w.raw_vocab, w.compressed_vocab, w.max_ngram, w.heads,
                                    self.pad, self.token_map, self.mult, self.primes,
                                    self.offsets)
        self.f32 = w.row_format == ROW_F32
        self.row_format = E.ROW_F32 if self.f32 else E.ROW_E4M3_E8M0_264
        self.table = None
        self.dense_np = None
        self.wkv_ld = 0
        if dense and w.has_forward:
            self.dense_np = gen.dense_inputs(w, table_rows_f32=self.rows if self.f32 else 0)
            self.wkv = self._strided_wkv(self.dense_np["wkv"], wkv_ld, device)
            self.q_w = to_device(self.dense_np["q_w"], device)
            self.k_w = to_device(self.dense_np["k_w"], device)
            self.h = to_device(self.dense_np["h"], device)
        if table and w.has_table:
            if self.f32:
                if self.dense_np is None:
                    self.dense_np = gen.dense_inputs(w, table_rows_f32=self.rows)
                self.table = to_device(self.dense_np["table"], device)
            else:
                self.table = torch.empty((self.rows, gen.ROW_BYTES), dtype=torch.uint8,
                                         device=device)
                fill_table(self.table, w.table_seed)
        self.desc = E.forward_desc(w.batch, w.seq, w.hc, w.dim, self.rows, self.row_format,
                                   w.row_dim, w.eps, w.gate_clamp,
                                   wkv_ld=self.wkv_ld)
        # the projection weight in block-scaled FP8 (codes, scales), host and device
        self.wkv_mx_np = None
        if wkv_mx:
            self.wkv_mx_np = gen.wkv_mx(w)
            self.w_codes = to_device(self.wkv_mx_np[0], device)
            self.w_scales = to_device(self.wkv_mx_np[1], device)

    def _strided_wkv(self, wkv: np.ndarray, wkv_ld, device):
        n, k = wkv.shape
        ld = self.E.engram_wkv_row_stride(k, wkv.itemsize) if wkv_ld is None else (wkv_ld or k)
        assert ld >= k
        self.wkv_ld = ld
        if ld == k:
            return to_device(wkv, device)
        nan = np.uint16(0x7FC0) if wkv.dtype == np.uint16 else np.float32("nan")
        padded = np.full((n, ld), nan, dtype=wkv.dtype)
        padded[:, :k] = wkv
        return to_device(padded, device)

    @property
    def tokens(self) -> int:
        return self.w.tokens

    def dead_np(self) -> np.ndarray:
        ids = self.ids_np.reshape(-1)
        return (ids < 0) | (ids >= self.w.raw_vocab)

    def fetch_rows(self, rows: np.ndarray) -> np.ndarray:
        """Host twin of the device table: the bytes of the given rows."""
        return gen.table_rows(self.w.table_seed, rows)

    def workspace(self):
        import torch
        n = self.E.engram_forward_workspace_size(self.params, self.desc)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device), n

    def workspace_mx(self):
        import torch
        n = self.E.engram_forward_mx_workspace_size(self.params, self.desc)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device), n

    def free(self):
        for name in ("table", "wkv", "q_w", "k_w", "h", "ids", "token_map", "hist_in",
                     "w_codes", "w_scales"):
            if hasattr(self, name):
                setattr(self, name, None)
