"""Parity of the papers' gate variants on the HIP path (through the C ABI) with
the CPU oracle: the plain sigmoid gate and the short convolution branch.

Inputs are seeded and synthetic (torch's generator, bf16 or fp32); the oracle
decodes the same bits. Gates and updated streams must agree within
|gpu - oracle| <= 1e-3 + 2e-2 |oracle|; the convolution's history buffers hold
copies of value rows (bit-exact) and per-position gates and mean squares.
"""
import dataclasses
import gc

import numpy as np
import pytest

import oracle as O
from tests.gpu_util import assert_close, say
from workloads import C3

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hashed_gram_conditional_amd as E  # noqa: E402
from workloads.harness import GpuWorkload  # noqa: E402

DEV = "cuda"
RAW_VOCAB = 1000


def _cleanup():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _vals(t):
    """float64 numpy values of a bf16 or fp32 tensor (any device)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


class Case:
    """Random gate + convolution inputs of one shape, on the device."""

    def __init__(self, B, T, hc, d, taps=4, dil=3, f32=False, seed=0, dead_frac=0.1,
                 norm=True, device=DEV, conv_scale=0.5):
        g = torch.Generator(device="cpu").manual_seed(seed)
        dt = torch.float32 if f32 else torch.bfloat16
        self.B, self.T, self.hc, self.d, self.taps, self.dil, self.f32 = B, T, hc, d, taps, dil, f32
        self.L = (taps - 1) * dil
        self.h = torch.randn((B, T, hc, d), generator=g).to(dt).to(device)
        self.kv = (0.7 * torch.randn((B * T, (hc + 1) * d), generator=g)).to(dt).to(device)
        self.q_w = (1 + 0.1 * torch.randn((hc, d), generator=g)).to(device)
        self.k_w = (1 + 0.1 * torch.randn((hc, d), generator=g)).to(device)
        self.cw = (conv_scale * torch.randn((hc, d, taps), generator=g)).to(device)
        self.nw = (1 + 0.2 * torch.randn((hc, d), generator=g)).to(device) if norm else None
        ids = torch.randint(0, RAW_VOCAB, (B, T), generator=g, dtype=torch.int32)
        dead = torch.rand((B, T), generator=g) < dead_frac
        ids[dead] = -1
        if T > 3:
            ids[0, 3] = RAW_VOCAB + 5          # out of range counts as DEAD too
        self.ids = ids.to(device)
        self.dead = ((ids < 0) | (ids >= RAW_VOCAB)).numpy()

    def desc(self, T=None, mode=E.GATE_SIGNED_SQRT, eps=1e-6, clamp=0.0):
        fmt = E.ROW_F32 if self.f32 else E.ROW_E4M3_E8M0_264
        return E.forward_desc(self.B, self.T if T is None else T, self.hc, self.d, 1, fmt,
                              4 if self.f32 else 256, eps, clamp, mode)

    def state(self):
        dt = torch.float32 if self.f32 else torch.bfloat16
        return (torch.zeros((self.B, self.L, self.d), dtype=dt, device=DEV),
                torch.zeros((self.B, self.L, self.hc + 1), dtype=torch.float32, device=DEV))

    def run(self, h, mode=E.GATE_SIGNED_SQRT, t0=0, t1=None, state_in=None, state_out=None,
            cw=None, clamp=0.0):
        """engram_gate_conv on positions [t0, t1) of every sequence; h is the
        full [B, T, hc, d] tensor, updated in place on that slice."""
        t1 = self.T if t1 is None else t1
        n = t1 - t0
        d = self.desc(n, mode, clamp=clamp)
        ids = self.ids[:, t0:t1].contiguous()
        kv = self.kv.view(self.B, self.T, -1)[:, t0:t1].contiguous()
        kv = kv.view(self.B * n, -1) if n > 0 else kv.reshape(0)
        hs = h[:, t0:t1].contiguous()
        gates = torch.full((max(self.B * n, 1), self.hc), -1.0, dtype=torch.float32, device=DEV)
        nb = E.engram_gate_conv_workspace_size(d)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
        sv_in, ss_in = state_in if state_in is not None else (None, None)
        sv_out, ss_out = state_out if state_out is not None else (None, None)
        conv = E.short_conv(self.cw if cw is None else cw, self.taps, self.dil, 1e-6, self.nw,
                            sv_in, ss_in, sv_out, ss_out)
        E.engram_gate_conv(d, conv, ids, RAW_VOCAB, kv, self.q_w, self.k_w, hs, gates, ws, nb)
        torch.cuda.synchronize()
        h[:, t0:t1] = hs
        return gates[:self.B * n].view(self.B, n, self.hc)

    def oracle(self, mode="signed_sqrt", cw=None, clamp=0.0):
        kv = _vals(self.kv).reshape(self.B, self.T, self.hc + 1, self.d)
        cw = self.cw if cw is None else cw
        return O.gate_conv(_vals(self.h), kv[:, :, :self.hc], kv[:, :, self.hc], _vals(self.q_w),
                           _vals(self.k_w), self.dead, 1e-6, clamp, _vals(cw),
                           None if self.nw is None else _vals(self.nw), self.dil, 1e-6,
                           mode=mode)


def _check(case, h_dev, gates, alpha, h_out, what):
    assert_close(_vals(gates), alpha, f"{what} gates")
    assert np.all(_vals(gates)[case.dead] == 0)
    hv = _vals(h_dev)
    h_exp = h_out if case.f32 else O.bf16_bits_to_f64(O.round_to_bf16_bits(h_out))
    assert_close(hv, h_exp, f"{what} h")
    # DEAD positions keep their streams bit for bit
    assert torch.equal(h_dev[torch.from_numpy(case.dead).to(DEV)].cpu(),
                       case.h[torch.from_numpy(case.dead).to(DEV)].cpu())


CASES = [
    # B, T, hc, d, taps, dil, f32, mode, norm
    (2, 37, 4, 136, 4, 3, False, "signed_sqrt", True),
    (3, 20, 2, 64, 1, 1, False, "plain", False),
    (1, 50, 3, 200, 3, 5, True, "signed_sqrt", True),
    (2, 12, 1, 5120, 4, 3, False, "plain", True),
    (1, 70, 4, 64, 8, 9, False, "signed_sqrt", False),
    (4, 2048, 2, 64, 4, 3, False, "signed_sqrt", True),      # runs of several tokens per thread
    (2, 5, 2, 16, 4, 3, True, "plain", True),                 # chunk shorter than the reach
]


@pytest.mark.parametrize("B,T,hc,d,taps,dil,f32,mode,norm", CASES,
                         ids=[f"B{c[0]}T{c[1]}hc{c[2]}d{c[3]}w{c[4]}x{c[5]}{'f32' if c[6] else 'bf16'}"
                              f"-{c[7]}" for c in CASES])
def test_gate_conv_matches_oracle(B, T, hc, d, taps, dil, f32, mode, norm):
    say(f"gate_conv B={B} T={T} hc={hc} d={d} taps={taps} dil={dil} f32={f32} {mode}")
    c = Case(B, T, hc, d, taps, dil, f32, seed=B * 1000 + T, norm=norm)
    h = c.h.clone()
    gm = E.GATE_PLAIN if mode == "plain" else E.GATE_SIGNED_SQRT
    gates = c.run(h, gm, clamp=0.5 if mode == "signed_sqrt" else 0.0)
    alpha, h_out, _ = c.oracle(mode, clamp=0.5 if mode == "signed_sqrt" else 0.0)
    _check(c, h, gates, alpha, h_out, f"gate_conv {mode}")


@pytest.mark.parametrize("B,T,hc,d,f32", [(2, 40, 4, 136, False), (256, 1, 4, 5120, False),
                                           (64, 1, 8, 5120, False), (32, 2, 4, 5120, True)],
                         ids=["80x4x136", "decode256x4x5120", "64x8x5120", "f32_64x4x5120"])
def test_gate_conv_zero_filters_equal_gate(B, T, hc, d, f32):
    """Filters at zero (the papers' init): the branch adds exactly the gated
    value, so engram_gate_conv agrees with engram_gate, and the gates are the
    same bits (the statistics pass reduces each stream as the update does; with
    few tokens both run one block per (token, stream))."""
    c = Case(B, T, hc, d, f32=f32, seed=7)
    zero = torch.zeros_like(c.cw)
    h1 = c.h.clone()
    g1 = c.run(h1, cw=zero)
    h2 = c.h.clone()
    g2 = torch.empty((c.B * c.T, c.hc), dtype=torch.float32, device=DEV)
    E.engram_gate(c.desc(), c.ids, RAW_VOCAB, c.kv, c.q_w, c.k_w, h2, g2)
    torch.cuda.synchronize()
    assert torch.equal(g1.reshape(-1, c.hc), g2)
    # The gate forms h + alpha v in one fma, the convolution pass in separate fp32
    # steps: where the sum cancels, the two differ by fp32 roundings at the scale
    # of the operands before the bf16 rounding of the result.
    v = _vals(c.kv).reshape(c.B, c.T, c.hc + 1, c.d)[:, :, c.hc:]
    ops = 2.0 ** -23 * (np.abs(_vals(c.h)) + np.abs(v))
    assert_close(_vals(h1), _vals(h2), "zero filters vs plain gate", atol=0.0, rtol=2.0 ** -7,
                 extra=ops)


@pytest.mark.parametrize("f32", [False, True], ids=["bf16", "f32"])
def test_plain_gate_mode(f32):
    """engram_gate with the papers' sigmoid(s) against the oracle."""
    c = Case(3, 29, 3, 72, f32=f32, seed=11)
    h = c.h.clone()
    g = torch.empty((c.B * c.T, c.hc), dtype=torch.float32, device=DEV)
    E.engram_gate(c.desc(mode=E.GATE_PLAIN, clamp=2.0), c.ids, RAW_VOCAB, c.kv, c.q_w, c.k_w, h, g)
    torch.cuda.synchronize()
    kv = _vals(c.kv).reshape(-1, c.hc + 1, c.d)
    a, ho = O.gate(_vals(c.h).reshape(-1, c.hc, c.d), kv[:, :c.hc], kv[:, c.hc], _vals(c.q_w),
                   _vals(c.k_w), c.dead.reshape(-1), 1e-6, 2.0, mode="plain")
    assert_close(_vals(g), a, "plain gates")
    h_exp = ho if f32 else O.bf16_bits_to_f64(O.round_to_bf16_bits(ho))
    assert_close(_vals(h).reshape(ho.shape), h_exp, "plain h")
    # the clamp belongs to the signed root only: a different clamp changes nothing
    h2 = c.h.clone()
    g2 = torch.empty_like(g)
    E.engram_gate(c.desc(mode=E.GATE_PLAIN, clamp=0.0), c.ids, RAW_VOCAB, c.kv, c.q_w, c.k_w, h2,
                  g2)
    torch.cuda.synchronize()
    assert torch.equal(g, g2)


@pytest.mark.parametrize("splits", [(5, 1, 1, 9), (1, 1, 1, 1, 1), (20,), (0, 3, 0)],
                         ids=["5-1-1-9", "decode5", "20", "empty-3-empty"])
def test_gate_conv_chunks_carry_history(splits):
    """Chunks (decode steps included) that pass the history on, in place,
    reproduce the one-shot call; the history holds the last 9 value rows bit
    for bit and their gates and mean squares."""
    c = Case(2, 40, 2, 64, seed=21, dead_frac=0.15)
    h_ref = c.h.clone()
    g_ref = c.run(h_ref)
    alpha, h_out, _ = c.oracle()
    _check(c, h_ref, g_ref, alpha, h_out, "one shot")

    h = c.h.clone()
    sv, ss = c.state()
    sv.fill_(1.0)                       # stale contents: a start without history ignores them
    ss.fill_(1.0)
    t0, first, gates = 0, True, []
    for n in list(splits) + [c.T - sum(splits)]:
        state_in = None if first else (sv, ss)
        gates.append(c.run(h, t0=t0, t1=t0 + n, state_in=state_in, state_out=(sv, ss)))
        t0 += n
        first = False
    assert_close(_vals(h), _vals(h_ref), "chunked vs one-shot h")
    assert_close(_vals(torch.cat(gates, 1)), _vals(g_ref), "chunked vs one-shot gates")
    _check(c, h, torch.cat(gates, 1), alpha, h_out, "chunked")
    # history = the last L positions: value rows copied, gates, mean(v^2)
    kv = c.kv.view(c.B, c.T, c.hc + 1, c.d)
    assert torch.equal(sv.cpu(), kv[:, -c.L:, c.hc].cpu())
    v = _vals(kv[:, -c.L:, c.hc])
    ms = np.where(c.dead[:, -c.L:], 0.0, np.mean(v * v, axis=-1))    # DEAD: gates and ms 0
    assert_close(_vals(ss[..., c.hc]), ms, "history mean squares", atol=0.0, rtol=1e-5)
    assert_close(_vals(ss[..., :c.hc]), alpha[:, -c.L:], "history gates")


def test_gate_conv_many_sequence_starts_with_history():
    """192 sequences of 37 tokens: every call (the chunks hold 3,840 and 3,264
    tokens) is large enough for the register-window kernel, whose blocks then
    hold several sequence starts; the second chunk reads its first 9
    positions' taps from the carried history."""
    c = Case(192, 37, 2, 64, seed=25, dead_frac=0.1)
    alpha, h_out, _ = c.oracle()
    h_ref = c.h.clone()
    g_ref = c.run(h_ref)
    _check(c, h_ref, g_ref, alpha, h_out, "one shot")
    h = c.h.clone()
    sv, ss = c.state()
    g1 = c.run(h, t0=0, t1=20, state_out=(sv, ss))
    g2 = c.run(h, t0=20, t1=37, state_in=(sv, ss), state_out=(sv, ss))
    _check(c, h, torch.cat([g1, g2], 1), alpha, h_out, "two chunks")
    assert_close(_vals(h), _vals(h_ref), "two chunks vs one shot")



def test_gate_conv_window_ragged_tail():
    """97 sequences of 37 tokens: 3,589 tokens, one past a multiple of the
    register-window kernel's 12-token blocks, so its last block holds a single
    token; every position is checked against the oracle."""
    c = Case(97, 37, 2, 64, seed=31, dead_frac=0.1)
    alpha, h_out, _ = c.oracle()
    h = c.h.clone()
    g = c.run(h)
    _check(c, h, g, alpha, h_out, "ragged tail")

def test_gate_conv_short_first_chunk_without_history():
    """A first chunk shorter than the reach: history rows before the sequence
    start are zero gates, i.e. zero input to the convolution."""
    c = Case(3, 4, 2, 32, seed=23, dead_frac=0.0)
    h = c.h.clone()
    sv, ss = c.state()
    sv.fill_(3.0)
    ss.fill_(3.0)
    g = c.run(h, state_out=(sv, ss))
    alpha, h_out, _ = c.oracle()
    _check(c, h, g, alpha, h_out, "short chunk")
    assert not ss[:, :c.L - c.T].cpu().any() and not sv[:, :c.L - c.T].cpu().any()
    kv = c.kv.view(c.B, c.T, c.hc + 1, c.d)
    assert torch.equal(sv[:, c.L - c.T:].cpu(), kv[:, :, c.hc].cpu())


def test_gate_conv_full_size_sampled():
    """The prefill shape (4 x 8192 tokens, 4 streams of 5120) in the launch
    configuration the benchmark uses, checked on sampled positions: the oracle
    takes each position's 10-token window, which holds everything it reads."""
    B, T, hc, d = C3.batch, C3.seq, C3.hc, C3.dim
    say(f"gate_conv full size B={B} T={T} hc={hc} d={d}")
    g = torch.Generator(device=DEV).manual_seed(41)
    h = torch.randn((B, T, hc, d), generator=g, device=DEV).to(torch.bfloat16)
    kv = (0.7 * torch.randn((B * T, (hc + 1) * d), generator=g, device=DEV)).to(torch.bfloat16)
    q_w = 1 + 0.1 * torch.randn((hc, d), generator=g, device=DEV)
    k_w = 1 + 0.1 * torch.randn((hc, d), generator=g, device=DEV)
    cw = 0.5 * torch.randn((hc, d, 4), generator=g, device=DEV)
    nw = 1 + 0.2 * torch.randn((hc, d), generator=g, device=DEV)
    ids = torch.randint(0, RAW_VOCAB, (B, T), generator=g, device=DEV, dtype=torch.int32)
    ids[:, 100:140] = -1
    h0 = h.clone()
    desc = E.forward_desc(B, T, hc, d, 1, E.ROW_E4M3_E8M0_264, 256, 1e-6, 0.0)
    nb = E.engram_gate_conv_workspace_size(desc)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    gates = torch.empty((B * T, hc), dtype=torch.float32, device=DEV)
    conv = E.short_conv(cw, 4, 3, 1e-6, nw)
    E.engram_gate_conv(desc, conv, ids, RAW_VOCAB, kv, q_w, k_w, h, gates, ws, nb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    picks = [(b, int(t)) for b in range(B) for t in rng.integers(0, T, 6)]
    picks += [(0, 0), (1, 1), (2, 8), (3, 9), (0, 99), (0, 100), (0, 140), (0, 142), (0, 149),
              (3, T - 1)]
    kv3 = kv.view(B, T, hc + 1, d)
    for b, t in picks:
        a = max(0, t - 9)
        sl = slice(a, t + 1)
        ids_w = ids[b, sl].cpu().numpy()
        dead = ((ids_w < 0) | (ids_w >= RAW_VOCAB))[None]
        kvw = _vals(kv3[b, sl])[None]
        al, ho, _ = O.gate_conv(_vals(h0[b, sl])[None], kvw[:, :, :hc], kvw[:, :, hc], _vals(q_w),
                                _vals(k_w), dead, 1e-6, 0.0, _vals(cw), _vals(nw), 3, 1e-6)
        assert_close(_vals(gates.view(B, T, hc)[b, t]), al[0, -1], f"gates ({b},{t})")
        assert_close(_vals(h[b, t]), O.bf16_bits_to_f64(O.round_to_bf16_bits(ho[0, -1])),
                     f"h ({b},{t})")
    del h, kv, h0, ws
    _cleanup()


# ---------------------------------------------------------------------------
# the whole layer with the branch
# ---------------------------------------------------------------------------

S_C = dataclasses.replace(C3, name="S_C", seed=1200, batch=2, seq=90, prime_base=7000, hc=3,
                          dim=96, dead_random=(1, 8), table_seed=3005)


@pytest.mark.parametrize("mode", [E.GATE_SIGNED_SQRT, E.GATE_PLAIN], ids=["signed", "plain"])
def test_forward_conv_equals_its_stages(mode):
    """engram_forward_conv computes the bits of engram_hash -> engram_gather ->
    engram_project -> engram_gate_conv; with zero filters it agrees with
    engram_forward."""
    w = S_C
    gw = GpuWorkload(w)
    desc = E.forward_desc(w.batch, w.seq, w.hc, w.dim, gw.rows, gw.row_format, w.row_dim, w.eps,
                          w.gate_clamp, mode, wkv_ld=gw.wkv_ld)
    g = torch.Generator(device="cpu").manual_seed(3)
    cw = (0.5 * torch.randn((w.hc, w.dim, 4), generator=g)).to(DEV)
    nw = (1 + 0.2 * torch.randn((w.hc, w.dim), generator=g)).to(DEV)
    T, S = w.tokens, w.segments
    # stages
    rows = torch.empty((T, S), dtype=torch.int64, device=DEV)
    E.engram_hash(gw.params, gw.ids, w.batch, w.seq, None, None, rows)
    e = torch.empty((T, S * 256), dtype=torch.bfloat16, device=DEV)
    E.engram_gather(gw.table, gw.rows, gw.row_format, 256, rows, T * S, e)
    kv = torch.empty((T, (w.hc + 1) * w.dim), dtype=torch.bfloat16, device=DEV)
    npw = E.engram_project_workspace_size(T, S * 256, (w.hc + 1) * w.dim, 0)
    pws = torch.empty(max(npw, 256), dtype=torch.uint8, device=DEV)
    E.engram_project(e, gw.wkv, kv, T, S * 256, (w.hc + 1) * w.dim, gw.wkv_ld, 0, pws, npw)
    h1 = gw.h.clone()
    g1 = torch.empty((T, w.hc), dtype=torch.float32, device=DEV)
    sv1 = torch.empty((w.batch, 9, w.dim), dtype=torch.bfloat16, device=DEV)
    ss1 = torch.empty((w.batch, 9, w.hc + 1), dtype=torch.float32, device=DEV)
    nb = E.engram_gate_conv_workspace_size(desc)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
    E.engram_gate_conv(desc, E.short_conv(cw, 4, 3, 1e-6, nw, None, None, sv1, ss1), gw.ids,
                       w.raw_vocab, kv, gw.q_w, gw.k_w, h1, g1, ws, nb)
    # fused
    h2 = gw.h.clone()
    g2 = torch.empty_like(g1)
    sv2, ss2 = torch.empty_like(sv1), torch.empty_like(ss1)
    nf = E.engram_forward_conv_workspace_size(gw.params, desc)
    wsf = torch.empty(nf, dtype=torch.uint8, device=DEV)
    E.engram_forward_conv(gw.params, desc, E.short_conv(cw, 4, 3, 1e-6, nw, None, None, sv2, ss2),
                          gw.ids, None, None, gw.table, gw.wkv, gw.q_w, gw.k_w, h2, g2, wsf, nf)
    torch.cuda.synchronize()
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(g1, g2)
    assert torch.equal(sv1.view(torch.int16), sv2.view(torch.int16)) and torch.equal(ss1, ss2)
    if mode == E.GATE_SIGNED_SQRT:
        h3 = gw.h.clone()
        g3 = torch.empty_like(g1)
        E.engram_forward_conv(gw.params, desc, E.short_conv(torch.zeros_like(cw), 4, 3, 1e-6, nw),
                              gw.ids, None, None, gw.table, gw.wkv, gw.q_w, gw.k_w, h3, g3, wsf,
                              nf)
        h4 = gw.h.clone()
        wsp, npf = gw.workspace()
        g4 = torch.empty_like(g1)
        E.engram_forward(gw.params, gw.desc, gw.ids, None, None, gw.table, gw.wkv, gw.q_w,
                         gw.k_w, h4, g4, wsp, npf)
        torch.cuda.synchronize()
        assert torch.equal(g3, g4)
        assert_close(_vals(h3), _vals(h4), "zero filters vs engram_forward", atol=0.0,
                     rtol=2.0 ** -7)
    gw.free()
    _cleanup()
