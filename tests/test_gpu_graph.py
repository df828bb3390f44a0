"""engram_forward captured in a HIP graph and replayed (the skinny decode, split-K
and gate sums paths), and called from two host threads on two streams at once.

The library allocates nothing, never synchronises and records no memset, so a
step can be captured once and replayed with new ids written into the same input
buffer (the usual decode loop). Each replay must give the bits of the same call
made eagerly. The replays alternate two id batches and run eager work (input
copies, fills, synchronisations) between them.
"""
import dataclasses
import gc

import pytest

from tests.gpu_util import say
from workloads import C3, C4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hashed_gram_conditional_amd as E  # noqa: E402
from workloads.harness import GpuWorkload  # noqa: E402

DEV = "cuda"

# decode shape (256 sequences x 1 token with a 3-token history, hc 4, width
# 5120, 24 segments: the skinny projection) on the 24,003,916-row prefill table
D_S = dataclasses.replace(C4, name="D_S", prime_base=1_000_000, table_seed=2002)
# 300 tokens over few tiles: the split-K projection with its workspace and fixup
S_A = dataclasses.replace(C3, name="S_A", seed=1100, batch=2, seq=150, prime_base=5000, hc=2,
                          dim=136, dead_random=(1, 16), table_seed=3001)
# 2,700 tokens over 275 whole tiles: the projection with the gate's key sums,
# the fold and the gate from the sums
S_G = dataclasses.replace(C3, name="S_G", seed=1102, batch=3, seq=900, max_ngram=3, heads=4,
                          prime_base=5000, hc=4, dim=1280, dead_random=(2, 20),
                          table_seed=3003, hash_setup_seed=None)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("w", [D_S, S_A, S_G], ids=lambda w: w.name)
def test_forward_graph_replays_equal_eager(w):
    say(f"graph {w.name}: {w.batch}x{w.seq} tokens, hc={w.hc}, d={w.dim}")
    gw = GpuWorkload(w)
    try:
        ws, n = gw.workspace()
        h0 = gw.h.clone()
        ids_a = gw.ids.clone()
        ids_b = torch.roll(ids_a, shifts=1, dims=0).contiguous()   # other tokens per sequence
        ids_buf = gw.ids
        h = gw.h
        gates = torch.empty((w.tokens, w.hc), dtype=torch.float32, device=DEV)
        hout = torch.empty((w.batch, 3), dtype=torch.int32, device=DEV)

        def step():
            E.engram_forward(gw.params, gw.desc, ids_buf, gw.hist_in, hout, gw.table, gw.wkv,
                             gw.q_w, gw.k_w, h, gates, ws, n)

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
        assert not torch.equal(_bits(ref["a"][0]), _bits(ref["b"][0]))

        reset(ids_a)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        # capture records the launches without running them
        assert torch.equal(_bits(h), _bits(h0))

        for i in range(6):
            name = "ab"[i % 2]
            reset(ids_a if name == "a" else ids_b)
            graph.replay()
            torch.cuda.synchronize()
            h_ref, g_ref, hout_ref = ref[name]
            assert torch.equal(_bits(h), _bits(h_ref)), f"replay {i}: h"
            assert torch.equal(_bits(gates), _bits(g_ref)), f"replay {i}: gates"
            assert torch.equal(hout, hout_ref), f"replay {i}: history"
        del graph
    finally:
        gw.free()
        gc.collect()
        torch.cuda.empty_cache()


def test_forward_on_two_streams_from_two_threads():
    """Two host threads call engram_forward at once, each on its own stream with
    its own buffers (the library keeps no shared state); every result equals the
    same call made alone."""
    import threading
    w = S_A
    say(f"two streams: {w.name} x 2 threads x 4 calls")
    gw = GpuWorkload(w)
    try:
        h0 = gw.h.clone()
        n = E.engram_forward_workspace_size(gw.params, gw.desc)
        ids = [gw.ids.clone(), torch.roll(gw.ids, shifts=1, dims=0).contiguous()]
        ref = []
        for x in ids:
            ws = torch.empty(max(n, 256), dtype=torch.uint8, device=DEV)
            h = h0.clone()
            g = torch.empty((w.tokens, w.hc), dtype=torch.float32, device=DEV)
            E.engram_forward(gw.params, gw.desc, x, None, None, gw.table, gw.wkv, gw.q_w,
                             gw.k_w, h, g, ws, n)
            torch.cuda.synchronize()
            ref.append((h, g))
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        bufs = [(torch.empty(max(n, 256), dtype=torch.uint8, device=DEV), h0.clone(),
                 torch.empty((w.tokens, w.hc), dtype=torch.float32, device=DEV)) for _ in ids]
        torch.cuda.synchronize()
        errors = []
        results = [[], []]

        def worker(k):
            try:
                ws, h, g = bufs[k]
                for _ in range(4):
                    with torch.cuda.stream(streams[k]):
                        h.copy_(h0)
                        E.engram_forward(gw.params, gw.desc, ids[k], None, None, gw.table,
                                         gw.wkv, gw.q_w, gw.k_w, h, g, ws, n,
                                         stream=streams[k])
                        results[k].append((h.clone(), g.clone()))
            except Exception as ex:          # reported by the main thread
                errors.append(ex)

        threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        assert not errors, errors
        for k in range(2):
            assert len(results[k]) == 4
            for h, g in results[k]:
                assert torch.equal(_bits(h), _bits(ref[k][0]))
                assert torch.equal(_bits(g), _bits(ref[k][1]))
    finally:
        gw.free()
        gc.collect()
        torch.cuda.empty_cache()
