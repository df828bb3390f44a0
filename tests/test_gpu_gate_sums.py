"""The key side of the gate in the projection's epilogue
(engram_project_gate_sums + engram_gate_sums, and engram_forward where its
projection fills the CUs with whole tiles).

* engram_project_gate_sums: the value columns within the projection's bound of
  the exact fp64 product (and bit-equal to engram_project's, which sums each
  output's K in the same order); each (token, stream, 128-column block) pair
  within a bound derived from the keys' own bound and fp32 summation, against
  fp64 sums over the exact keys.
* engram_gate_sums fed sums formed on the host from bf16 keys: gates and
  streams against the oracle's gate on those keys, DEAD rows untouched.
* engram_forward on a workload that takes this path, every token against the
  oracle, and equal to its stage entry points bit for bit.
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
from tests.gpu_util import U32, assert_close, gemm_tolerance, say
from workloads import C3

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hashed_gram_conditional_amd as E  # noqa: E402
from workloads.device import bf16_bits, to_device  # noqa: E402
from workloads.harness import GpuWorkload  # noqa: E402
from tests.test_gpu_parity import (_check_forward, _forward, _run_stages,  # noqa: E402
                                   _run_sums_stages)

DEV = "cuda"

# 2,700 tokens (a ragged last tile of 140), hc 4 x 1280, K = 8 x 256: 11 x 25
# whole tiles, more than the CUs, so engram_forward takes the gate sums path.
S_C = dataclasses.replace(C3, name="S_C", seed=1102, batch=3, seq=900, max_ngram=3, heads=4,
                          prime_base=5000, hc=4, dim=1280, dead_random=(2, 20),
                          table_seed=3003, hash_setup_seed=None)


def _bf16(rng, shape, scale=1.0):
    return O.round_to_bf16_bits(scale * rng.standard_normal(shape))


def _desc(tokens, hc, dim, ld=0, mode=E.GATE_SIGNED_SQRT, clamp=1e-6):
    return E.forward_desc(1, tokens, hc, dim, 0, E.ROW_E4M3_E8M0_264, 256, 1e-6, clamp,
                          gate_mode=mode, wkv_ld=ld)


def _pairs(kv_bits, hc, dim):
    """The float pairs at the start of each kv row: [T, hc, dim / 128, 2]."""
    T = kv_bits.shape[0]
    raw = np.ascontiguousarray(kv_bits).view(np.uint8).reshape(T, -1)
    n = hc * (dim // 128) * 8
    return raw[:, :n].copy().view(np.float32).reshape(T, hc, dim // 128, 2)


@pytest.mark.parametrize("M,K,hc,dim,pad", [
    (300, 384, 1, 256, 0),        # fewer tiles than CUs, ragged tokens
    (1000, 768, 2, 512, 8),
    (2700, 2048, 4, 1280, 64),
    (513, 6144, 4, 5120, 64),     # the layer's width, 3 token tiles (one of a single token)
])
def test_project_gate_sums(M, K, hc, dim, pad):
    say(f"project_gate_sums M={M} K={K} hc={hc} dim={dim} ld={K + pad}")
    rng = np.random.default_rng(M + K + dim)
    N = (hc + 1) * dim
    e = _bf16(rng, (M, K))
    w = _bf16(rng, (N, K), 0.02)
    h = _bf16(rng, (M, hc * dim))
    qk = (rng.uniform(0.5, 1.5, (hc, dim)) * rng.uniform(0.5, 1.5, (hc, dim))).astype(np.float32)
    ld = K + pad
    w_dev = torch.full((N, ld), float("nan"), dtype=torch.bfloat16, device=DEV)
    w_dev[:, :K] = to_device(w).view(torch.bfloat16)
    e_dev, h_dev, qk_dev = to_device(e), to_device(h), to_device(qk)
    kv = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    E.engram_project_gate_sums(_desc(M, hc, dim, ld), e_dev, K, w_dev, h_dev, qk_dev, kv)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    E.engram_project(e_dev, w_dev, ref, M, K, N, ld, 0)
    torch.cuda.synchronize()
    got = bf16_bits(kv)
    assert np.array_equal(bf16_bits(h_dev), h)          # h is only read
    # the value columns: engram_project's bits (whole-K order, no split)
    assert np.array_equal(got[:, hc * dim:], bf16_bits(ref)[:, hc * dim:])
    # sampled tokens (first, last, the last tile's first) against fp64
    sel = np.unique(np.concatenate([rng.integers(0, M, 48), [0, M - 1, (M - 1) // 256 * 256]]))
    ef = O.bf16_bits_to_f64(e[sel])
    wf = O.bf16_bits_to_f64(w)
    exact = ef @ wf.T
    tol = gemm_tolerance(ef, wf, exact, bf16_out=True)
    gv = O.bf16_bits_to_f64(got[sel][:, hc * dim:])
    assert np.all(np.abs(gv - exact[:, hc * dim:]) <= tol[:, hc * dim:])
    # the pairs: k_dev differs from the exact key by at most tol, so over a
    # block sum k^2 moves by sum (2 |k| tol + tol^2) and sum h w k by
    # sum |h w| tol; fp32 summation of 128 terms adds 130 u sum |term|
    k = exact[:, :hc * dim].reshape(len(sel), hc, dim // 128, 128)
    t = tol[:, :hc * dim].reshape(k.shape)
    hh = O.bf16_bits_to_f64(h[sel]).reshape(k.shape)
    ww = qk.astype(np.float64).reshape(1, hc, dim // 128, 128)
    exp_kk = (k * k).sum(-1)
    exp_hk = (hh * ww * k).sum(-1)
    tol_kk = (2 * np.abs(k) * t + t * t).sum(-1) + 130 * U32 * ((np.abs(k) + t) ** 2).sum(-1)
    tol_hk = (np.abs(hh * ww) * t).sum(-1) + 131 * U32 * np.abs(hh * ww * (np.abs(k) + t)).sum(-1)
    p = _pairs(got[sel], hc, dim).astype(np.float64)
    bad_kk = ~(np.abs(p[..., 0] - exp_kk) <= tol_kk)
    bad_hk = ~(np.abs(p[..., 1] - exp_hk) <= tol_hk)
    assert not bad_kk.any(), f"sum k^2: {np.argwhere(bad_kk)[:3]}"
    assert not bad_hk.any(), f"sum h w k: {np.argwhere(bad_hk)[:3]}"
    _pairs_match_stored_keys(p, bf16_bits(ref)[sel], h[sel], qk, hc, dim)


def _pairs_match_stored_keys(p, kv_bits, h_bits, qk, hc, dim):
    """The pairs are the sums over the keys the plain projection stores (the
    same accumulators, rounded to bf16 the same way), up to fp32 summation."""
    n = kv_bits.shape[0]
    k = O.bf16_bits_to_f64(kv_bits[:, :hc * dim]).reshape(n, hc, dim // 128, 128)
    hh = O.bf16_bits_to_f64(h_bits).reshape(k.shape)
    ww = qk.astype(np.float64).reshape(1, hc, dim // 128, 128)
    kk, hk = (k * k).sum(-1), (hh * ww * k).sum(-1)
    assert np.all(np.abs(p[..., 0] - kk) <= 130 * U32 * (k * k).sum(-1))
    assert np.all(np.abs(p[..., 1] - hk) <= 131 * U32 * np.abs(hh * ww * k).sum(-1))


@pytest.mark.parametrize("T,hc,dim,mode", [
    (700, 4, 5120, E.GATE_SIGNED_SQRT),
    (40, 3, 256, E.GATE_SIGNED_SQRT),       # few tokens: 512-thread blocks
    (333, 8, 1024, E.GATE_PLAIN),
    (2500, 1, 8192, E.GATE_SIGNED_SQRT),    # 8 chunks per thread
])
def test_gate_sums_against_the_oracle(T, hc, dim, mode):
    """engram_gate_sums on sums formed on the host (fp64, stored as fp32) from
    bf16 keys: the oracle's gate on the same keys, values and streams."""
    say(f"gate_sums T={T} hc={hc} dim={dim} mode={mode}")
    rng = np.random.default_rng(T * 7 + dim)
    k = _bf16(rng, (T, hc, dim))
    v = _bf16(rng, (T, dim))
    h = _bf16(rng, (T, hc, dim))
    # keys partly aligned with the streams, so the gates spread over (0, 1)
    mix = rng.uniform(-1, 1, (T, hc, 1))
    k = O.round_to_bf16_bits(O.bf16_bits_to_f64(k) * 0.3 + mix * O.bf16_bits_to_f64(h))
    q_w = rng.uniform(0.5, 1.5, (hc, dim)).astype(np.float32)
    k_w = rng.uniform(0.5, 1.5, (hc, dim)).astype(np.float32)
    ids = rng.integers(0, 1000, T).astype(np.int32)
    ids[::13] = -1
    ids[5] = 1000                          # raw_vocab: DEAD as well
    dead = (ids < 0) | (ids >= 1000)
    kf, hf = O.bf16_bits_to_f64(k), O.bf16_bits_to_f64(h)
    wf = (q_w * k_w).astype(np.float64)    # the folded fp32 products
    blocks = dim // 128
    skk = (kf * kf).reshape(T, hc, blocks, 128).sum(-1)
    shk = (hf * wf[None] * kf).reshape(T, hc, blocks, 128).sum(-1)
    pairs = np.stack([skk, shk], -1).astype(np.float32)
    kv = np.zeros((T, (hc + 1) * dim), dtype=np.uint16)
    kv[:, hc * dim:] = v
    raw = kv.view(np.uint8).reshape(T, -1)
    raw[:, :pairs[0].nbytes] = pairs.reshape(T, -1).view(np.uint8)
    h_dev = to_device(h.reshape(T, -1))
    g_dev = torch.full((T, hc), -1.0, dtype=torch.float32, device=DEV)
    E.engram_gate_sums(_desc(T, hc, dim, mode=mode, clamp=1e-6), to_device(ids), 1000,
                       to_device(kv), h_dev, g_dev)
    torch.cuda.synchronize()
    alpha, h_out = O.gate(hf, kf, O.bf16_bits_to_f64(v), q_w, k_w, dead, 1e-6, 1e-6,
                          "plain" if mode == E.GATE_PLAIN else "signed_sqrt")
    g = g_dev.cpu().numpy()
    assert_close(g, alpha, "gates")
    assert np.all(g[dead] == 0.0)
    got_h = bf16_bits(h_dev).reshape(T, hc, dim)
    assert np.array_equal(got_h[dead], h[dead])
    assert_close(O.bf16_bits_to_f64(got_h), h_out, "h")
    if mode == E.GATE_SIGNED_SQRT:          # the signed root keeps the gates off 0 and 1
        assert 0.05 < np.median(g[~dead]) < 0.95


def test_gate_sums_equal_the_gate_on_stored_keys():
    """engram_project_gate_sums + engram_gate_sums against engram_project +
    engram_gate on the same inputs: the same value bits, gates equal up to the
    order of the fp32 sums (1e-4, a tenth of the parity bar's 1e-3; the signed
    root magnifies a change of s near 0), streams apart by no more than that
    gate difference and the two roundings explain."""
    rng = np.random.default_rng(21)
    T, K, hc, dim = 1536, 1024, 4, 2048
    N = (hc + 1) * dim
    e, w = to_device(_bf16(rng, (T, K))), to_device(_bf16(rng, (N, K), 0.03))
    h0 = to_device(_bf16(rng, (T, hc * dim)))
    q_w = to_device(rng.uniform(0.5, 1.5, (hc, dim)).astype(np.float32))
    k_w = to_device(rng.uniform(0.5, 1.5, (hc, dim)).astype(np.float32))
    ids = to_device(rng.integers(0, 50, T).astype(np.int32))
    d = _desc(T, hc, dim)
    qk = torch.empty((hc, dim), dtype=torch.float32, device=DEV)
    E.engram_fold_gate_weights(q_w, k_w, hc, dim, qk)
    kv_a, kv_b = (torch.empty((T, N), dtype=torch.bfloat16, device=DEV) for _ in range(2))
    h_a, h_b = h0.clone(), h0.clone()
    g_a, g_b = (torch.empty((T, hc), dtype=torch.float32, device=DEV) for _ in range(2))
    E.engram_project(e, w, kv_a, T, K, N, 0, 0)
    E.engram_gate(d, ids, 50, kv_a, q_w, k_w, h_a, g_a)
    E.engram_project_gate_sums(d, e, K, w, h_b, qk, kv_b)
    E.engram_gate_sums(d, ids, 50, kv_b, h_b, g_b)
    torch.cuda.synchronize()
    assert torch.equal(kv_a[:, hc * dim:].view(torch.int16), kv_b[:, hc * dim:].view(torch.int16))
    ga, gb = g_a.cpu().numpy().astype(np.float64), g_b.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(ga - gb) <= 1e-4)
    # h_out = bf16(h + alpha v): a gate that moves by d changes the sum by d |v|,
    # and each side's rounding adds up to half a bf16 step of its own result
    # (2^-8 of it at the bottom of a binade)
    ha = O.bf16_bits_to_f64(bf16_bits(h_a)).reshape(T, hc, dim)
    hb = O.bf16_bits_to_f64(bf16_bits(h_b)).reshape(T, hc, dim)
    v = O.bf16_bits_to_f64(bf16_bits(kv_a[:, hc * dim:]))[:, None, :]
    dg = np.abs(ga - gb)[:, :, None]
    bound = dg * np.abs(v) + 2.0 ** -8 * (np.abs(ha) + np.abs(hb))
    bad = ~(np.abs(ha - hb) <= bound)
    assert not bad.any(), [(tuple(i), ha[tuple(i)], hb[tuple(i)], bound[tuple(i)])
                           for i in np.argwhere(bad)[:4]]
    diff = ha != hb
    say(f"  max gate difference {float(dg.max()):.2e}; {int(diff.sum())} of {diff.size} "
        f"stream elements differ")


def test_forward_takes_the_gate_sums_path():
    """S_C: every token against the oracle, for engram_forward and for the
    separate stages; engram_forward equals the gate sums stage entry points
    bit for bit when its projection fills the CUs with whole tiles (as it
    does on a 256-CU MI355X), the separate stages otherwise."""
    w = S_C
    tiles = -(-w.tokens // 256) * ((w.hc + 1) * w.dim // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"S_C forward: {w.tokens} tokens, {tiles} whole tiles on {cus} CUs")
    gw = GpuWorkload(w)
    try:
        h_f, h_s = gw.h.clone(), gw.h.clone()
        g_f = _forward(gw, h_f)
        g_s = _run_sums_stages(gw, h_s)
        _, _, kv, g_p = _run_stages(gw)          # updates gw.h
        _check_forward(gw, gw.h, g_p, np.arange(w.tokens), kv_dev=kv,
                       also=(("S_C engram_forward", h_f, g_f),
                             ("S_C gate sums stages", h_s, g_s)))
        if tiles >= cus:
            assert torch.equal(h_f.view(torch.int16), h_s.view(torch.int16))
            assert torch.equal(g_f, g_s)
        else:
            assert torch.equal(h_f.view(torch.int16), gw.h.view(torch.int16))
            assert torch.equal(g_f, g_p)
    finally:
        gw.free()


@pytest.mark.parametrize("M,hc,dim,S", [(600, 2, 512, 3), (2700, 4, 1280, 8)])
def test_project_mx_gate_sums(M, hc, dim, S):
    """The FP8 weight: value columns with engram_project_mx's bits and within
    its bound of the exact product of the FP8 values; the pairs against fp64
    sums over the exact keys, within the bound that follows from the keys'
    bound, and equal to the sums over engram_project_mx's stored keys up to
    fp32 summation."""
    say(f"project_mx_gate_sums M={M} hc={hc} dim={dim} S={S}")
    from tests.gpu_util import kv_tolerance_mx
    from workloads import gen
    rng = np.random.default_rng(M + dim + S)
    N = (hc + 1) * dim
    rows = gen.table_rows(M + S, rng.integers(0, 10 ** 9, M * S)).reshape(M, S, 264)
    codes, scales = gen.quantize_mx_e4m3(rng.normal(0.0, 0.02, (N, S * 256)))
    e_codes = to_device(np.ascontiguousarray(rows[:, :, :256]).reshape(M, S * 256))
    e_scales = to_device(np.ascontiguousarray(rows[:, :, 256:]).reshape(M, S * 8))
    wc, wsc = to_device(codes), to_device(scales)
    h = _bf16(rng, (M, hc * dim))
    qk = (rng.uniform(0.5, 1.5, (hc, dim)) * rng.uniform(0.5, 1.5, (hc, dim))).astype(np.float32)
    kv = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    E.engram_project_mx_gate_sums(_desc(M, hc, dim), e_codes, e_scales, S, wc, wsc,
                                  to_device(h), to_device(qk), kv)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    E.engram_project_mx(e_codes, e_scales, S, wc, wsc, ref, M, N)
    torch.cuda.synchronize()
    got, refb = bf16_bits(kv), bf16_bits(ref)
    assert np.array_equal(got[:, hc * dim:], refb[:, hc * dim:])
    sel = np.unique(np.concatenate([rng.integers(0, M, 48), [0, M - 1, (M - 1) // 256 * 256]]))
    e = O.mx_values(rows[sel, :, :256].reshape(len(sel), S * 256),
                    rows[sel, :, 256:].reshape(len(sel), S * 8))
    exact = O.project(e, O.mx_values(codes, scales))
    tol = kv_tolerance_mx(exact)
    gv = O.bf16_bits_to_f64(got[sel][:, hc * dim:])
    assert np.all(np.abs(gv - exact[:, hc * dim:]) <= tol[:, hc * dim:])
    k = exact[:, :hc * dim].reshape(len(sel), hc, dim // 128, 128)
    t = tol[:, :hc * dim].reshape(k.shape)
    hh = O.bf16_bits_to_f64(h[sel]).reshape(k.shape)
    ww = qk.astype(np.float64).reshape(1, hc, dim // 128, 128)
    p = _pairs(got[sel], hc, dim).astype(np.float64)
    tol_kk = (2 * np.abs(k) * t + t * t).sum(-1) + 130 * U32 * ((np.abs(k) + t) ** 2).sum(-1)
    tol_hk = (np.abs(hh * ww) * t).sum(-1) + 131 * U32 * np.abs(hh * ww * (np.abs(k) + t)).sum(-1)
    assert np.all(np.abs(p[..., 0] - (k * k).sum(-1)) <= tol_kk)
    assert np.all(np.abs(p[..., 1] - (hh * ww * k).sum(-1)) <= tol_hk)
    _pairs_match_stored_keys(p, refb[sel], h[sel], qk, hc, dim)


def test_forward_mx_takes_the_gate_sums_path():
    """engram_forward_mx on S_C: every token against the oracle (the FP8 rules
    of the parity checks), and its stage entry points' bits (gather_mx, fold,
    engram_project_mx_gate_sums, engram_gate_sums) when its projection fills
    the CUs with whole tiles."""
    w = S_C
    tiles = -(-w.tokens // 256) * ((w.hc + 1) * w.dim // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    gw = GpuWorkload(w, wkv_mx=True)
    try:
        T, S = w.tokens, w.segments
        wsm, nm = gw.workspace_mx()
        h_f, h_s = gw.h.clone(), gw.h.clone()
        g_f = torch.empty((T, w.hc), dtype=torch.float32, device=DEV)
        E.engram_forward_mx(gw.params, gw.desc, gw.ids, None, None, gw.table, gw.w_codes,
                            gw.w_scales, gw.q_w, gw.k_w, h_f, g_f, wsm, nm)
        rows = torch.empty((T, S), dtype=torch.int64, device=DEV)
        E.engram_hash(gw.params, gw.ids, w.batch, w.seq, None, None, rows)
        codes = torch.empty((T, S * 256), dtype=torch.uint8, device=DEV)
        scales = torch.empty((T, S * 8), dtype=torch.uint8, device=DEV)
        E.engram_gather_mx(gw.table, gw.rows, rows, T * S, codes, scales)
        qk = torch.empty((w.hc, w.dim), dtype=torch.float32, device=DEV)
        E.engram_fold_gate_weights(gw.q_w, gw.k_w, w.hc, w.dim, qk)
        kv = torch.empty((T, (w.hc + 1) * w.dim), dtype=torch.bfloat16, device=DEV)
        E.engram_project_mx_gate_sums(gw.desc, codes, scales, S, gw.w_codes, gw.w_scales, h_s,
                                      qk, kv)
        g_s = torch.empty_like(g_f)
        E.engram_gate_sums(gw.desc, gw.ids, w.raw_vocab, kv, h_s, g_s)
        torch.cuda.synchronize()
        _check_forward(gw, h_f, g_f, np.arange(T), wkv=O.mx_values(*gw.wkv_mx_np), mx=True,
                       also=(("S_C FP8 gate sums stages", h_s, g_s),))
        if tiles >= cus:
            assert torch.equal(h_f.view(torch.int16), h_s.view(torch.int16))
            assert torch.equal(g_f, g_s)
    finally:
        gw.free()


def _sums_kv(rng, T, hc, dim, h_bits, k_bits, v_bits, q_w, k_w):
    """kv rows as engram_project_gate_sums leaves them, formed on the host from
    bf16 keys (fp64 sums stored as fp32) and bf16 values."""
    kf = O.bf16_bits_to_f64(k_bits).reshape(T, hc, dim)
    hf = O.bf16_bits_to_f64(h_bits).reshape(T, hc, dim)
    wf = (q_w * k_w).astype(np.float64)
    blocks = dim // 128
    pairs = np.stack([(kf * kf).reshape(T, hc, blocks, 128).sum(-1),
                      (hf * wf[None] * kf).reshape(T, hc, blocks, 128).sum(-1)], -1)
    pairs = pairs.astype(np.float32)
    kv = np.zeros((T, (hc + 1) * dim), dtype=np.uint16)
    kv[:, hc * dim:] = v_bits.reshape(T, dim)
    kv.view(np.uint8).reshape(T, -1)[:, :pairs[0].nbytes] = pairs.reshape(T, -1).view(np.uint8)
    return kv


@pytest.mark.parametrize("B,T,hc,dim,mode", [
    (2, 300, 4, 5120, E.GATE_SIGNED_SQRT),
    (3, 40, 2, 256, E.GATE_PLAIN),
    (1, 333, 1, 1024, E.GATE_SIGNED_SQRT),
])
def test_gate_conv_sums_against_the_oracle(B, T, hc, dim, mode):
    """engram_gate_conv_sums (the statistics from the sums, then the short
    convolution branch) on sums formed on the host from bf16 keys: the oracle's
    gate_conv on those keys, values and streams, DEAD positions untouched, and
    the history the branch leaves for the next chunk."""
    say(f"gate_conv_sums B={B} T={T} hc={hc} dim={dim} mode={mode}")
    rng = np.random.default_rng(B * T + dim)
    n = B * T
    h = _bf16(rng, (n, hc, dim))
    mix = rng.uniform(-1, 1, (n, hc, 1))
    k = O.round_to_bf16_bits(O.bf16_bits_to_f64(_bf16(rng, (n, hc, dim))) * 0.3 +
                             mix * O.bf16_bits_to_f64(h))
    v = _bf16(rng, (n, dim))
    q_w = rng.uniform(0.5, 1.5, (hc, dim)).astype(np.float32)
    k_w = rng.uniform(0.5, 1.5, (hc, dim)).astype(np.float32)
    cw = (0.5 * rng.standard_normal((hc, dim, 4))).astype(np.float32)
    nw = (1 + 0.2 * rng.standard_normal((hc, dim))).astype(np.float32)
    ids = rng.integers(0, 1000, n).astype(np.int32)
    ids[::11] = -1
    dead = ids < 0
    kv = _sums_kv(rng, n, hc, dim, h, k, v, q_w, k_w)
    desc = E.forward_desc(B, T, hc, dim, 0, E.ROW_E4M3_E8M0_264, 256, 1e-6, 1e-6,
                          gate_mode=mode)
    nb = E.engram_gate_conv_workspace_size(desc)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
    sv = torch.empty((B, 9, dim), dtype=torch.bfloat16, device=DEV)
    ss = torch.empty((B, 9, hc + 1), dtype=torch.float32, device=DEV)
    cw_d, nw_d = to_device(cw), to_device(nw)
    conv = E.short_conv(cw_d, 4, 3, 1e-6, nw_d, None, None, sv, ss)
    h_dev = to_device(h.reshape(n, -1))
    g_dev = torch.full((n, hc), -1.0, dtype=torch.float32, device=DEV)
    E.engram_gate_conv_sums(desc, conv, to_device(ids), 1000, to_device(kv), h_dev, g_dev, ws, nb)
    torch.cuda.synchronize()
    hf = O.bf16_bits_to_f64(h).reshape(B, T, hc, dim)
    al, ho, tail = O.gate_conv(hf, O.bf16_bits_to_f64(k).reshape(B, T, hc, dim),
                               O.bf16_bits_to_f64(v).reshape(B, T, dim), q_w, k_w,
                               dead.reshape(B, T), 1e-6, 1e-6, cw, nw, 3, 1e-6,
                               mode="plain" if mode == E.GATE_PLAIN else "signed_sqrt")
    g = g_dev.cpu().numpy().reshape(B, T, hc)
    assert_close(g, al, "gates")
    assert np.all(g.reshape(n, hc)[dead] == 0.0)
    got_h = bf16_bits(h_dev).reshape(n, hc, dim)
    assert np.array_equal(got_h[dead], h[dead])
    assert_close(O.bf16_bits_to_f64(got_h).reshape(B, T, hc, dim),
                 O.bf16_bits_to_f64(O.round_to_bf16_bits(ho)), "h")
    # the history: the last 9 value rows and their gates (the gated values factored)
    vt_tail = np.asarray(tail)                       # [B, 9, hc, dim] gated values
    ssn = ss.cpu().numpy()
    svn = O.bf16_bits_to_f64(bf16_bits(sv))
    assert_close(ssn[..., :hc, None] * svn[:, :, None, :], vt_tail, "history (gated values)")


def test_forward_conv_takes_the_gate_sums_path():
    """engram_forward_conv on S_C: the bits of its stage entry points on the
    sums path (fold, engram_project_gate_sums, engram_gate_conv_sums) when its
    projection fills the CUs with whole tiles, and close to the separate stages
    (engram_project + engram_gate_conv, checked against the oracle in
    test_gpu_conv.py): gates within 1e-4, streams within one bf16 step (where
    the two gates' last bits flip a rounding) or 1e-3."""
    w = S_C
    tiles = -(-w.tokens // 256) * ((w.hc + 1) * w.dim // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    gw = GpuWorkload(w)
    try:
        T, S = w.tokens, w.segments
        K, N = S * 256, (w.hc + 1) * w.dim
        g = torch.Generator(device="cpu").manual_seed(8)
        cw = (0.5 * torch.randn((w.hc, w.dim, 4), generator=g)).to(DEV)
        nw = (1 + 0.2 * torch.randn((w.hc, w.dim), generator=g)).to(DEV)
        nb = E.engram_gate_conv_workspace_size(gw.desc)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
        nf = E.engram_forward_conv_workspace_size(gw.params, gw.desc)
        wsf = torch.empty(nf, dtype=torch.uint8, device=DEV)
        outs = {}
        for path in ("forward", "sums", "separate"):
            h = gw.h.clone()
            gt = torch.empty((T, w.hc), dtype=torch.float32, device=DEV)
            sv = torch.empty((w.batch, 9, w.dim), dtype=torch.bfloat16, device=DEV)
            ss = torch.empty((w.batch, 9, w.hc + 1), dtype=torch.float32, device=DEV)
            conv = E.short_conv(cw, 4, 3, 1e-6, nw, None, None, sv, ss)
            if path == "forward":
                E.engram_forward_conv(gw.params, gw.desc, conv, gw.ids, None, None, gw.table,
                                      gw.wkv, gw.q_w, gw.k_w, h, gt, wsf, nf)
            else:
                rows = torch.empty((T, S), dtype=torch.int64, device=DEV)
                E.engram_hash(gw.params, gw.ids, w.batch, w.seq, None, None, rows)
                e = torch.empty((T, K), dtype=torch.bfloat16, device=DEV)
                E.engram_gather(gw.table, gw.rows, gw.row_format, 256, rows, T * S, e)
                kv = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
                if path == "sums":
                    qk = torch.empty((w.hc, w.dim), dtype=torch.float32, device=DEV)
                    E.engram_fold_gate_weights(gw.q_w, gw.k_w, w.hc, w.dim, qk)
                    E.engram_project_gate_sums(gw.desc, e, K, gw.wkv, h, qk, kv)
                    E.engram_gate_conv_sums(gw.desc, conv, gw.ids, w.raw_vocab, kv, h, gt, ws,
                                            nb)
                else:
                    E.engram_project(e, gw.wkv, kv, T, K, N, gw.wkv_ld, 0)
                    E.engram_gate_conv(gw.desc, conv, gw.ids, w.raw_vocab, kv, gw.q_w, gw.k_w,
                                       h, gt, ws, nb)
            torch.cuda.synchronize()
            outs[path] = (h, gt, sv, ss)
        hf, gf, svf, ssf = outs["forward"]
        if tiles >= cus:
            hs, gs, svs, sss = outs["sums"]
            assert torch.equal(hf.view(torch.int16), hs.view(torch.int16))
            assert torch.equal(gf, gs) and torch.equal(ssf, sss)
            assert torch.equal(svf.view(torch.int16), svs.view(torch.int16))
        hp, gp, _, _ = outs["separate"]
        ga, gb = gp.cpu().numpy().astype(np.float64), gf.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(ga - gb) <= 1e-4)
        assert_close(O.bf16_bits_to_f64(bf16_bits(hf)), O.bf16_bits_to_f64(bf16_bits(hp)),
                     "h: forward_conv against the separate stages", atol=1e-3, rtol=2.0 ** -7)
    finally:
        gw.free()


def test_forward_on_a_host_table_takes_the_gate_sums_path():
    """engram_forward with S_C's table in pinned host memory (the gather reading
    rows over the host link) gives the bits of the HBM-resident table on the
    gate sums path, and so does the two-stream pipeline of the benchmark's host
    tier (hash + gather on a side stream, then fold, engram_project_gate_sums
    and engram_gate_sums on the compute stream)."""
    w = S_C
    gw = GpuWorkload(w)
    try:
        T, S = w.tokens, w.segments
        host = torch.empty(gw.table.shape, dtype=gw.table.dtype, pin_memory=True)
        host.copy_(gw.table)
        ws, n = gw.workspace()
        outs = []
        for table in (gw.table, host):
            h = gw.h.clone()
            g = torch.empty((T, w.hc), dtype=torch.float32, device=DEV)
            E.engram_forward(gw.params, gw.desc, gw.ids, None, None, table, gw.wkv, gw.q_w,
                             gw.k_w, h, g, ws, n)
            torch.cuda.synchronize()
            outs.append((h, g))
        assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
        assert torch.equal(outs[0][1], outs[1][1])
        side = torch.cuda.Stream()
        main = torch.cuda.current_stream()
        rows = torch.empty((T, S), dtype=torch.int64, device=DEV)
        e = torch.empty((T, S * 256), dtype=torch.bfloat16, device=DEV)
        kv = torch.empty((T, (w.hc + 1) * w.dim), dtype=torch.bfloat16, device=DEV)
        qk = torch.empty((w.hc, w.dim), dtype=torch.float32, device=DEV)
        h = gw.h.clone()
        g = torch.empty((T, w.hc), dtype=torch.float32, device=DEV)
        ready = torch.cuda.Event()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            E.engram_hash(gw.params, gw.ids, w.batch, w.seq, None, None, rows, stream=side)
            E.engram_gather(host, gw.rows, gw.row_format, 256, rows, T * S, e, stream=side)
            ready.record(side)
        E.engram_fold_gate_weights(gw.q_w, gw.k_w, w.hc, w.dim, qk, stream=main)
        main.wait_event(ready)
        E.engram_project_gate_sums(gw.desc, e, S * 256, gw.wkv, h, qk, kv, stream=main)
        E.engram_gate_sums(gw.desc, gw.ids, w.raw_vocab, kv, h, g, stream=main)
        torch.cuda.synchronize()
        tiles = -(-T // 256) * ((w.hc + 1) * w.dim // 256)
        if tiles >= torch.cuda.get_device_properties(0).multi_processor_count:
            assert torch.equal(h.view(torch.int16), outs[0][0].view(torch.int16))
            assert torch.equal(g, outs[0][1])
        del host
    finally:
        gw.free()
