"""The weight's row stride (wkv_ld). Every projection path gives the same bits
with the rows of wkv spread apart as with dense rows, and reads none of the
gaps, which hold NaN here (a NaN read would reach kv). The fused forward and a
transpose into a strided buffer follow."""
import numpy as np
import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hashed_gram_conditional_amd as E  # noqa: E402
from workloads.device import bf16_bits, to_device  # noqa: E402
from workloads.harness import GpuWorkload  # noqa: E402
from tests.test_gpu_parity import S_A, S_B  # noqa: E402

DEV = "cuda"


def _spread(w: torch.Tensor, ld: int) -> torch.Tensor:
    n, k = w.shape
    nan = float("nan")
    out = torch.full((n, ld), nan, dtype=w.dtype, device=DEV)
    out[:, :k] = w
    return out


def _project(e, w, M, K, N, ld, f32, with_ws):
    n = E.engram_project_workspace_size(M, K, N, int(f32)) if with_ws else 0
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=DEV) if n else None
    kv = torch.empty((M, N), dtype=e.dtype, device=DEV)
    E.engram_project(e, w, kv, M, K, N, ld, int(f32), ws, n)
    torch.cuda.synchronize()
    return kv


# decode shape (columns dealt to the CUs), wide tiles filling the chip, split-K
# with a workspace and 128-wide tiles without one, a ragged edge, fp32
@pytest.mark.parametrize("M,K,N,pad,f32,with_ws", [
    (256, 6144, 25600, 64, False, False),
    (100, 768, 16384, 8, False, False),
    (4096, 128, 4096, 8, False, False),
    (300, 512, 1032, 8, False, True),
    (300, 512, 1032, 64, False, False),
    (37, 192, 40, 4, True, False),
])
def test_project_strided_weight_same_bits(M, K, N, pad, f32, with_ws):
    say(f"project M={M} K={K} N={N} ld={K + pad} f32={f32} ws={with_ws}")
    g = torch.Generator(device="cpu").manual_seed(M + K + N)
    dt = torch.float32 if f32 else torch.bfloat16
    e = torch.randn((M, K), generator=g).to(dt).to(DEV)
    w = (0.02 * torch.randn((N, K), generator=g)).to(dt).to(DEV)
    dense = _project(e, w, M, K, N, 0, f32, with_ws)
    spread = _project(e, _spread(w, K + pad), M, K, N, K + pad, f32, with_ws)
    assert not torch.isnan(spread).any()
    view = (lambda t: t.view(torch.int32)) if f32 else (lambda t: t.view(torch.int16))
    assert torch.equal(view(dense), view(spread))


@pytest.mark.parametrize("w", [S_A, S_B], ids=lambda w: w.name)
def test_forward_strided_weight_same_bits(w):
    """engram_forward and engram_forward_static with desc.wkv_ld set give the
    bits of dense rows. The two entry points may differ from each other in kv's last bits (split K
    against 128-wide tiles), so each is compared with itself."""
    dense = GpuWorkload(w, wkv_ld=0)
    assert dense.wkv_ld == w.mem_dim
    spread = GpuWorkload(w, table=False, wkv_ld=w.mem_dim + 72)
    desc = E.forward_desc(w.batch, w.seq, w.hc, w.dim, dense.rows, dense.row_format, w.row_dim,
                          w.eps, w.gate_clamp, wkv_ld=spread.wkv_ld)
    ws, n = dense.workspace()
    outs = {False: [], True: []}
    for d, wkv in ((dense.desc, dense.wkv), (desc, spread.wkv)):
        for static in (False, True):
            h = dense.h.clone()
            g = torch.empty((w.tokens, w.hc), dtype=torch.float32, device=DEV)
            if static:
                E.engram_forward_static(dense.params, d, dense.ids, None, None, dense.table,
                                        wkv, dense.q_w, dense.k_w, h, g)
            else:
                E.engram_forward(dense.params, d, dense.ids, None, None, dense.table, wkv,
                                 dense.q_w, dense.k_w, h, g, ws, n)
            torch.cuda.synchronize()
            outs[static].append((h, g))
    for (h0, g0), (h1, g1) in outs.values():
        assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
        assert torch.equal(g0, g1)
    dense.free()
    spread.free()


def test_transpose_into_strided_rows():
    """engram_transpose with dst_ld writes rows dst_ld apart and leaves the gaps."""
    rng = np.random.default_rng(9)
    rows, cols, ld = 200, 70, 264
    a = rng.integers(0, 2 ** 16, (rows, cols)).astype(np.uint16)
    src = to_device(a)
    dst = torch.full((cols, ld), 0.5, dtype=torch.bfloat16, device=DEV)
    E.engram_transpose(src, dst, rows, cols, ld, 2)
    torch.cuda.synchronize()
    got = bf16_bits(dst)
    assert np.array_equal(got[:, :rows], np.ascontiguousarray(a.T))
    assert (got[:, rows:] == 0x3F00).all()

