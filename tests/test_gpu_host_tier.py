"""The table in pinned host memory: the gather kernels read it over the host
link, a prefetch on a second stream overlaps the projection, and every result
equals the HBM-resident path bit for bit (same kernels, same inputs) and the
oracle's rows. Pageable host memory is rejected before any launch.
"""
import numpy as np
import pytest

import oracle as O
from tests.gpu_util import say
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hashed_gram_conditional_amd as E  # noqa: E402
from workloads.device import bf16_bits, fill_table, to_device  # noqa: E402
from workloads.harness import GpuWorkload  # noqa: E402
from tests.test_gpu_parity import S_A  # noqa: E402

DEV = "cuda"


def _pinned_copy(dev_table):
    host = torch.empty(dev_table.shape, dtype=dev_table.dtype, pin_memory=True)
    host.copy_(dev_table)
    torch.cuda.synchronize()
    return host


def test_host_table_gathers_equal_oracle_and_device_table():
    R, seed = 30011, 41
    dev = torch.empty((R, 264), dtype=torch.uint8, device=DEV)
    fill_table(dev, seed)
    host = _pinned_copy(dev)
    assert host.is_pinned()
    rng = np.random.default_rng(9)
    ids = rng.integers(-5, R + 5, 4099).astype(np.int64)
    ids[:3] = [0, R - 1, R]
    ids_d = to_device(ids)
    fetch = lambda r: gen.table_rows(seed, r)
    # raw rows
    out_h = torch.full((len(ids), 264), 7, dtype=torch.uint8, device=DEV)
    out_d = torch.full_like(out_h, 9)
    E.engram_gather_rows(host, R, ids_d, len(ids), out_h)
    E.engram_gather_rows(dev, R, ids_d, len(ids), out_d)
    torch.cuda.synchronize()
    exp = O.gather_rows(fetch, ids.reshape(-1, 1), R).reshape(-1, 264)
    assert np.array_equal(out_h.cpu().numpy(), exp)
    assert torch.equal(out_h, out_d)
    # dequantised rows
    e_h = torch.empty((len(ids), 256), dtype=torch.bfloat16, device=DEV)
    e_d = torch.empty_like(e_h)
    E.engram_gather(host, R, E.ROW_E4M3_E8M0_264, 256, ids_d, len(ids), e_h)
    E.engram_gather(dev, R, E.ROW_E4M3_E8M0_264, 256, ids_d, len(ids), e_d)
    torch.cuda.synchronize()
    exp_e = O.gather_e4m3(fetch, ids.reshape(-1, 1), R).reshape(-1, 256)
    assert np.array_equal(bf16_bits(e_h).reshape(-1, 256), exp_e)
    assert torch.equal(e_h.view(torch.int16), e_d.view(torch.int16))


def test_pageable_table_is_rejected_before_any_launch():
    R = 64
    pageable = torch.zeros((R, 264), dtype=torch.uint8)          # not pinned
    assert not pageable.is_pinned()
    ids = to_device(np.arange(8, dtype=np.int64))
    out = torch.full((8, 264), 5, dtype=torch.uint8, device=DEV)
    with pytest.raises(E.EngramError) as ex:
        E.engram_gather_rows(pageable, R, ids, 8, out)
    assert ex.value.status == E.EINVAL
    e = torch.empty((8, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(E.EngramError) as ex:
        E.engram_gather(pageable, R, E.ROW_E4M3_E8M0_264, 256, ids, 8, e)
    assert ex.value.status == E.EINVAL
    torch.cuda.synchronize()
    assert bool((out == 5).all())                                   # nothing ran


def _project_ws(T, K, N):
    n = E.engram_project_workspace_size(T, K, N, 0)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=DEV), n


def test_prefetch_on_a_second_stream_equals_the_resident_forward():
    """hash + gather from the host table on a side stream, an event, then the
    projection and gate on the compute stream: the bits of engram_forward on
    the HBM table. engram_forward and engram_forward_mx also take the host
    table directly."""
    w = S_A
    gw = GpuWorkload(w, wkv_mx=True)
    host = _pinned_copy(gw.table)
    T, S = w.tokens, w.segments
    K, N = S * 256, (w.hc + 1) * w.dim
    # reference: engram_forward with the HBM table
    ws, nws = gw.workspace()
    h_ref = gw.h.clone()
    g_ref = torch.empty((T, w.hc), dtype=torch.float32, device=DEV)
    E.engram_forward(gw.params, gw.desc, gw.ids, None, None, gw.table, gw.wkv, gw.q_w, gw.k_w,
                     h_ref, g_ref, ws, nws)
    torch.cuda.synchronize()
    # the pipeline
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    rows = torch.empty((T, S), dtype=torch.int64, device=DEV)
    e = torch.empty((T, K), dtype=torch.bfloat16, device=DEV)
    kv = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    pws, npws = _project_ws(T, K, N)
    h = gw.h.clone()
    g = torch.empty_like(g_ref)
    ready = torch.cuda.Event()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        E.engram_hash(gw.params, gw.ids, w.batch, w.seq, None, None, rows, stream=side)
        E.engram_gather(host, gw.rows, gw.row_format, 256, rows, T * S, e, stream=side)
        ready.record(side)
    main.wait_event(ready)
    E.engram_project(e, gw.wkv, kv, T, K, N, gw.wkv_ld, 0, pws, npws, stream=main)
    E.engram_gate(gw.desc, gw.ids, w.raw_vocab, kv, gw.q_w, gw.k_w, h, g, stream=main)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h_ref.view(torch.int16))
    assert torch.equal(g, g_ref)
    # the fused entry points on the host table
    h2 = gw.h.clone()
    g2 = torch.empty_like(g_ref)
    E.engram_forward(gw.params, gw.desc, gw.ids, None, None, host, gw.wkv, gw.q_w, gw.k_w, h2,
                     g2, ws, nws)
    wsm, nm = gw.workspace_mx()
    h3, h4 = gw.h.clone(), gw.h.clone()
    g3, g4 = torch.empty_like(g_ref), torch.empty_like(g_ref)
    E.engram_forward_mx(gw.params, gw.desc, gw.ids, None, None, host, gw.w_codes, gw.w_scales,
                        gw.q_w, gw.k_w, h3, g3, wsm, nm)
    E.engram_forward_mx(gw.params, gw.desc, gw.ids, None, None, gw.table, gw.w_codes,
                        gw.w_scales, gw.q_w, gw.k_w, h4, g4, wsm, nm)
    torch.cuda.synchronize()
    assert torch.equal(h2.view(torch.int16), h_ref.view(torch.int16)) and torch.equal(g2, g_ref)
    assert torch.equal(h3.view(torch.int16), h4.view(torch.int16)) and torch.equal(g3, g4)
    say(f"host tier: {T} tokens, {gw.rows} rows pinned on the host")
    gw.free()
