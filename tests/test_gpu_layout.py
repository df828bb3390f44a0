"""Weights held with the other dimension innermost -- wkv as [S row_dim,
(hc+1) dim] (inputs outer, outputs inner) and q_w / k_w as [dim, hc] -- turned
into the kernels' layout by engram_transpose give the same layer bits."""
import numpy as np
import pytest

from tests.gpu_util import say
from workloads import C3, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hashed_gram_conditional_amd as E  # noqa: E402
from workloads.device import bf16_bits, to_device  # noqa: E402
from workloads.harness import GpuWorkload  # noqa: E402
from tests.test_gpu_parity import S_A, S_B  # noqa: E402

DEV = "cuda"


@pytest.mark.parametrize("rows,cols,dt", [(1, 1, np.uint16), (3, 200, np.uint16),
                                          (65, 129, np.float32), (130, 63, np.uint16),
                                          (5120, 4, np.float32), (4, 5120, np.float32)])
def test_transpose_bit_exact(rows, cols, dt):
    rng = np.random.default_rng(rows * 1000 + cols)
    a = rng.integers(0, 2 ** 16 if dt == np.uint16 else 2 ** 32, (rows, cols)).astype(
        np.uint16 if dt == np.uint16 else np.uint32)
    if dt == np.float32:
        a = a.view(np.float32)
    src = to_device(a)
    dst = torch.empty((cols, rows), dtype=src.dtype, device=DEV)
    E.engram_transpose(src, dst, rows, cols, 0, a.dtype.itemsize)
    torch.cuda.synchronize()
    got = bf16_bits(dst) if dt == np.uint16 else dst.cpu().numpy().view(np.uint32)
    raw = a if dt == np.uint16 else a.view(np.uint32)           # compare bits, NaNs included
    assert np.array_equal(got, np.ascontiguousarray(raw.T))


def test_transpose_full_wkv_shape():
    """The prefill weight in the [6144, 25600] orientation comes back as the
    [25600, 6144] array the kernels read, bit for bit, with dense rows and with
    rows 6208 elements apart."""
    say("transpose wkv [6144, 25600] -> [25600, 6144] and [25600, 6208]")
    w = gen.dense_inputs(C3)["wkv"]                       # [25600, 6144] bf16 bits
    src = to_device(np.ascontiguousarray(w.T))
    dst = torch.empty((C3.kv_cols, C3.mem_dim), dtype=torch.bfloat16, device=DEV)
    E.engram_transpose(src, dst, C3.mem_dim, C3.kv_cols, 0, 2)
    ld = E.engram_wkv_row_stride(C3.mem_dim, 2)
    spread = torch.empty((C3.kv_cols, ld), dtype=torch.bfloat16, device=DEV)
    E.engram_transpose(src, spread, C3.mem_dim, C3.kv_cols, ld, 2)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(dst), w)
    assert np.array_equal(bf16_bits(spread)[:, :C3.mem_dim], w)


@pytest.mark.parametrize("w", [S_A, S_B], ids=lambda w: w.name)
def test_forward_with_weights_in_the_other_layout(w):
    gw = GpuWorkload(w)
    d = gw.dense_np
    K, N = w.mem_dim, w.kv_cols
    wkv_in_out = to_device(np.ascontiguousarray(d["wkv"].T))          # [K, N]
    qw_dh = to_device(np.ascontiguousarray(d["q_w"].T))               # [dim, hc]
    kw_dh = to_device(np.ascontiguousarray(d["k_w"].T))
    # the transposed weight goes into rows K + 72 apart, unlike the harness's
    ld = K + 72
    wkv = torch.full((N, ld), float("nan"), dtype=torch.bfloat16, device=DEV)
    q_w = torch.empty((w.hc, w.dim), dtype=torch.float32, device=DEV)
    k_w = torch.empty_like(q_w)
    E.engram_transpose(wkv_in_out, wkv, K, N, ld, 2)
    E.engram_transpose(qw_dh, q_w, w.dim, w.hc, 0, 4)
    E.engram_transpose(kw_dh, k_w, w.dim, w.hc, 0, 4)
    desc = E.forward_desc(w.batch, w.seq, w.hc, w.dim, gw.rows, gw.row_format, w.row_dim,
                          w.eps, w.gate_clamp, wkv_ld=ld)
    ws, n = gw.workspace()
    outs = []
    for d, ww, qq, kk in ((gw.desc, gw.wkv, gw.q_w, gw.k_w), (desc, wkv, q_w, k_w)):
        h = gw.h.clone()
        g = torch.empty((w.tokens, w.hc), dtype=torch.float32, device=DEV)
        E.engram_forward(gw.params, d, gw.ids, None, None, gw.table, ww, qq, kk, h, g, ws, n)
        torch.cuda.synchronize()
        outs.append((h, g))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    gw.free()
