"""The whole-workload parity checker used by the GPU tests, run on the CPU with
the oracle's own results standing in for a device: it must accept them and
reject planted errors in kv, a gate, a stream element and a DEAD row."""
import dataclasses

import numpy as np
import pytest

import oracle as O
from tests.gpu_util import check_forward_chunks
from workloads import C3, gen

SMALL = dataclasses.replace(C3, name="checker", seed=1200, batch=2, seq=40, prime_base=5000,
                            hc=2, dim=64, dead_random=(1, 6), table_seed=3100)


def _oracle_device():
    w = SMALL
    tm, mult = gen.hash_setup(w)
    pad = int(tm[0])
    primes = O.primes_from(w.prime_base, w.segments)
    offs, R = O.segment_offsets(primes)
    ids, _ = gen.token_ids(w)
    rid, _ = O.hash_rows(ids, tm, w.compressed_vocab, pad, mult, primes, offs, w.max_ngram,
                         w.heads)
    dead = (ids.reshape(-1) < 0)
    d = gen.dense_inputs(w)
    wkv = O.bf16_bits_to_f64(d["wkv"])
    h_in = d["h"].reshape(w.tokens, w.hc, w.dim)
    fetch = lambda r: gen.table_rows(w.table_seed, r)
    res = O.forward_tokens(np.arange(w.tokens), rid, dead, fetch_rows=fetch, table_rows=R,
                           wkv=wkv, q_w=d["q_w"], k_w=d["k_w"], h=O.bf16_bits_to_f64(h_in),
                           hc=w.hc, dim=w.dim, eps=w.eps, clamp=w.gate_clamp, bf16=True)
    args = dict(tokens=np.arange(w.tokens), rid=rid, dead=dead, fetch_rows=fetch,
                table_f32=None, table_rows=R, wkv=wkv, q_w=d["q_w"], k_w=d["k_w"], h_in=h_in,
                hc=w.hc, dim=w.dim, eps=w.eps, clamp=w.gate_clamp, bf16=True, chunk=16)
    dev = dict(h_out=res["h_out_bits"].reshape(h_in.shape),
               gates=res["alpha"].astype(np.float32),
               kv=O.round_to_bf16_bits(res["kv_exact"]))
    return args, dev, dead


def test_checker_accepts_the_oracles_own_results():
    args, dev, dead = _oracle_device()
    assert dead.any() and not dead.all()
    st = check_forward_chunks(**args, **dev)
    assert st["tokens"] == SMALL.tokens and st["allowed"] == 0
    st = check_forward_chunks(**args, **dev, mx=True)
    assert st["allowed"] == 0


@pytest.mark.parametrize("what", ["kv", "gate", "h", "dead_h", "dead_gate"])
def test_checker_rejects_planted_errors(what):
    args, dev, dead = _oracle_device()
    live = int(np.flatnonzero(~dead)[7])
    dtok = int(np.flatnonzero(dead)[0])
    if what == "kv":
        kv = dev["kv"].copy()
        kv[live, 3] ^= np.uint16(0x0040)              # a few ulps off
        dev["kv"] = kv
    elif what == "gate":
        g = dev["gates"].copy()
        g[live, 1] += 0.05
        dev["gates"] = g
    elif what == "h":
        h = O.bf16_bits_to_f64(dev["h_out"]).copy()
        h[live, 0, 5] += 0.25 + 0.1 * abs(h[live, 0, 5])
        dev["h_out"] = O.round_to_bf16_bits(h)
    elif what == "dead_h":
        h = dev["h_out"].copy()
        h[dtok, 1, 0] ^= np.uint16(1)
        dev["h_out"] = h
    else:
        g = dev["gates"].copy()
        g[dtok, 0] = 1e-30
        dev["gates"] = g
    with pytest.raises(AssertionError):
        check_forward_chunks(**args, **dev)
