"""Decode-sized calls of engram_forward (the skinny projection schedule, at most
256 tokens) give the bits of the stage entry points called one by one, for
several token counts and for a table in pinned host memory."""
from dataclasses import replace

import numpy as np
import pytest

from tests.gpu_util import say
from workloads import C4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hashed_gram_conditional_amd as E  # noqa: E402
from workloads.harness import GpuWorkload  # noqa: E402

DEV = "cuda"
# the decode workload's shapes (hc 4 x 5120, 24 segments) over a small table
DEC = replace(C4, name="DEC", prime_base=5000, table_seed=3400)


def _stages(gw, start, batch, table, hist, h, gates):
    w = gw.w
    T, S = batch, w.segments
    ids = gw.ids[start:start + batch].contiguous()
    rows = torch.empty((T, S), dtype=torch.int64, device=DEV)
    E.engram_hash(gw.params, ids, batch, 1, hist, None, rows)
    e = torch.empty((T, S * 256), dtype=torch.bfloat16, device=DEV)
    E.engram_gather(table, gw.rows, gw.row_format, 256, rows, T * S, e)
    kv = torch.empty((T, (w.hc + 1) * w.dim), dtype=torch.bfloat16, device=DEV)
    n = E.engram_project_workspace_size(T, S * 256, (w.hc + 1) * w.dim, 0)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=DEV)
    E.engram_project(e, gw.wkv, kv, T, S * 256, (w.hc + 1) * w.dim, gw.wkv_ld, 0, ws, n)
    desc = E.forward_desc(batch, 1, w.hc, w.dim, gw.rows, gw.row_format, w.row_dim, w.eps,
                          w.gate_clamp, wkv_ld=gw.wkv_ld)
    E.engram_gate(desc, ids, w.raw_vocab, kv, gw.q_w, gw.k_w, h, gates)


def _forward(gw, start, batch, table, hist, h, gates):
    w = gw.w
    desc = E.forward_desc(batch, 1, w.hc, w.dim, gw.rows, gw.row_format, w.row_dim, w.eps,
                          w.gate_clamp, wkv_ld=gw.wkv_ld)
    n = E.engram_forward_workspace_size(gw.params, desc)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    E.engram_forward(gw.params, desc, gw.ids[start:start + batch].contiguous(), hist, None, table,
                     gw.wkv, gw.q_w, gw.k_w, h, gates, ws, n)


# (first sequence, token count); sequence 0 sits in a DEAD span
@pytest.mark.parametrize("start,batch", [(0, 256), (0, 100), (7, 33), (5, 1)])
def test_decode_forward_bits_of_the_stages(start, batch):
    say(f"decode forward vs stages: {batch} tokens from sequence {start}")
    gw = GpuWorkload(DEC)
    hist = gw.hist_in[start:start + batch].contiguous()
    outs = []
    for run in (_stages, _forward):
        h = gw.h[start:start + batch].clone()
        g = torch.empty((batch, DEC.hc), dtype=torch.float32, device=DEV)
        run(gw, start, batch, gw.table, hist, h, g)
        torch.cuda.synchronize()
        outs.append((h, g))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    assert bool((outs[1][1] != 0).any())
    gw.free()


def test_decode_forward_host_table():
    """The same with the table in pinned host memory (the gather's host mode)."""
    say("decode forward vs stages: 64 tokens, pinned host table")
    gw = GpuWorkload(DEC)
    host = torch.empty(gw.table.shape, dtype=torch.uint8, pin_memory=True)
    host.copy_(gw.table)
    batch = 64
    hist = gw.hist_in[:batch].contiguous()
    outs = []
    for run, table in ((_stages, gw.table), (_forward, host)):
        h = gw.h[:batch].clone()
        g = torch.empty((batch, DEC.hc), dtype=torch.float32, device=DEV)
        run(gw, 0, batch, table, hist, h, g)
        torch.cuda.synchronize()
        outs.append((h, g))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    gw.free()
