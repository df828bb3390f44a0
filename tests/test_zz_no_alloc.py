"""engram_forward_static (no workspace argument; its scratch is a static device
array) against engram_forward on the same inputs: two decode calls in a row,
the second smaller, bit for bit; a prefill call whose projection engram_forward
splits over the CUs, against the oracle; a call beyond the array refused before
any launch."""
import dataclasses

import numpy as np
import pytest

from tests.gpu_util import ATOL, RTOL, say
from workloads import C3, C4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hashed_gram_conditional_amd as E  # noqa: E402
from workloads.harness import GpuWorkload  # noqa: E402
from tests.test_gpu_parity import _check_forward  # noqa: E402

DEV = "cuda"

# decode steps at the full width against a small table (24 segments from 5000)
DECODE = dataclasses.replace(C4, name="static_decode", prime_base=5000, table_seed=3300)
# a prefill chunk of 600 tokens: fewer 256 x 256 tiles than CUs
PREFILL = dataclasses.replace(C3, name="static_prefill", seed=1310, batch=3, seq=200,
                              prime_base=5000, hc=2, dim=1024, dead_random=(1, 9),
                              table_seed=3301)


def _both(gw, batch, hist=True):
    """engram_forward and engram_forward_static on the first ``batch`` sequences."""
    w = gw.w
    desc = E.forward_desc(batch, w.seq, w.hc, w.dim, gw.rows, gw.row_format, w.row_dim, w.eps,
                          w.gate_clamp, wkv_ld=gw.wkv_ld)
    ids = gw.ids[:batch].contiguous()
    hin = gw.hist_in[:batch].contiguous() if (hist and gw.hist_in is not None) else None
    out = []
    for static in (False, True):
        h = gw.h[:batch].clone()
        g = torch.full((batch * w.seq, w.hc), -1.0, dtype=torch.float32, device=DEV)
        hout = torch.full((batch, 3), -9, dtype=torch.int32, device=DEV)
        if static:
            E.engram_forward_static(gw.params, desc, ids, hin, hout, gw.table, gw.wkv, gw.q_w,
                                    gw.k_w, h, g)
        else:
            n = E.engram_forward_workspace_size(gw.params, desc)
            ws = torch.empty(max(n, 256), dtype=torch.uint8, device=DEV)
            E.engram_forward(gw.params, desc, ids, hin, hout, gw.table, gw.wkv, gw.q_w, gw.k_w,
                             h, g, ws, n)
        torch.cuda.synchronize()
        out.append((h, g, hout))
    return out


def test_static_decode_two_calls_bit_exact():
    say(f"engram_forward_static: decode 256 then 100 tokens, hc 4 x 5120, "
        f"scratch {E.engram_forward_static_max_bytes() >> 20} MiB")
    gw = GpuWorkload(DECODE)
    for batch in (DECODE.batch, 100):
        (h0, g0, s0), (h1, g1, s1) = _both(gw, batch)
        assert torch.equal(h0.view(torch.int16), h1.view(torch.int16)), batch
        assert torch.equal(g0, g1), batch
        assert torch.equal(s0, s1), batch
        assert not torch.equal(h0.view(torch.int16), gw.h[:batch].view(torch.int16))
    gw.free()


def test_static_prefill_chunk_against_the_oracle():
    """engram_forward splits this call's projection over the CUs; the static
    variant's partial tiles would not fit, so it runs 128-wide tiles over the
    whole K. Its kv can then differ from engram_forward's in the last bit, so
    its gates and streams are checked against the oracle, every token."""
    say("engram_forward_static: 600-token prefill chunk (engram_forward splits K)")
    gw = GpuWorkload(PREFILL)
    (h0, g0, _), (h1, g1, _) = _both(gw, PREFILL.batch, hist=False)
    a0, a1 = g0.cpu().numpy().astype(np.float64), g1.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(a1 - a0) <= ATOL + RTOL * np.abs(a0))
    _check_forward(gw, h1, g1, np.arange(PREFILL.tokens))
    # then a smaller decode call on the same scratch gives engram_forward's bits
    gwd = GpuWorkload(DECODE)
    (h0, g0, s0), (h1, g1, s1) = _both(gwd, 37)
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(g0, g1) and torch.equal(s0, s1)
    gw.free()
    gwd.free()


def test_static_refuses_calls_beyond_the_array():
    gw = GpuWorkload(DECODE)
    big = E.forward_desc(2048, 1, 4, 5120, gw.rows, gw.row_format, 256, 1e-6, 0.0,
                         wkv_ld=gw.wkv_ld)
    ids = torch.zeros((2048, 1), dtype=torch.int32, device=DEV)
    h = torch.zeros((2048, 1, 4, 5120), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(E.EngramError) as ex:
        E.engram_forward_static(gw.params, big, ids, None, None, gw.table, gw.wkv, gw.q_w,
                                gw.k_w, h, None)
    assert ex.value.status == E.ESCRATCH
    torch.cuda.synchronize()
    assert not h.any()
    gw.free()


def test_static_captured_in_a_graph_replays_equal_eager():
    """The use the entry point is for: captured once in a HIP graph (after one
    eager call on the device, which looks the array up) and replayed with new
    ids in the same buffer, every replay giving the eager call's bits."""
    say("engram_forward_static captured in a HIP graph, 4 replays, 2 id batches")
    gw = GpuWorkload(DECODE)
    w = DECODE
    ids_buf, h, h0 = gw.ids, gw.h, gw.h.clone()
    ids_a = ids_buf.clone()
    ids_b = torch.roll(ids_a, shifts=1, dims=0).contiguous()
    gates = torch.empty((w.tokens, w.hc), dtype=torch.float32, device=DEV)
    hout = torch.empty((w.batch, 3), dtype=torch.int32, device=DEV)

    def step():
        E.engram_forward_static(gw.params, gw.desc, ids_buf, gw.hist_in, hout, gw.table, gw.wkv,
                                gw.q_w, gw.k_w, h, gates)

    def reset(ids):
        ids_buf.copy_(ids)
        h.copy_(h0)
        gates.fill_(-1.0)
        hout.fill_(-7)
        torch.cuda.synchronize()

    ref = {}
    for name, ids in (("a", ids_a), ("b", ids_b)):
        reset(ids)
        step()
        torch.cuda.synchronize()
        ref[name] = (h.clone(), gates.clone(), hout.clone())
    reset(ids_a)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for name in ("a", "b", "a", "b"):
        reset(ids_a if name == "a" else ids_b)
        graph.replay()
        torch.cuda.synchronize()
        rh, rg, rs = ref[name]
        assert torch.equal(h.view(torch.int16), rh.view(torch.int16)), name
        assert torch.equal(gates, rg) and torch.equal(hout, rs), name
    del graph
    gw.free()


def test_static_on_the_gate_sums_path():
    """A 2,700-token call whose projection fills the CUs with whole tiles takes
    the gate sums path in both entry points (46 MB of the array): the static
    variant gives engram_forward's bits, then a smaller decode call on the same
    array does too."""
    from tests.test_gpu_gate_sums import S_C
    say("engram_forward_static: 2,700-token call on the gate sums path, then decode")
    gw = GpuWorkload(S_C)
    (h0, g0, _), (h1, g1, _) = _both(gw, S_C.batch, hist=False)
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(g0, g1)
    assert not torch.equal(h0.view(torch.int16), gw.h.view(torch.int16))
    gw.free()
    gwd = GpuWorkload(DECODE)
    (h0, g0, s0), (h1, g1, s1) = _both(gwd, 64)
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(g0, g1) and torch.equal(s0, s1)
    gwd.free()
