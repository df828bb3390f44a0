"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types an oracle formula: each compares the oracle with a value
printed on a page (tests/golden/, with citations), a library routine that
computes the same thing independently (sympy's primes, torch's float8 and
bfloat16 conversions), a closed form, an invariant, or brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import sympy
import torch

import oracle as O
from workloads import C0, C1, C2, C4, gen


def _golden(name):
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# hash: worked example, prime table, segments
# ---------------------------------------------------------------------------

def test_worked_example_mix_and_indices():
    g = _golden("worked_example.json")
    toks = np.array([g["compressed_tokens"]], dtype=np.int64)
    mult = g["multipliers_newest_first"]
    cells, dead = O.ngram_cells(toks, pad=0, n_cells=3)
    assert not dead.any()
    t = toks.shape[1] - 1
    for n_str, exp in g["expected"].items():
        n = int(n_str)
        mix = O.mix_values(cells[:, t:t + 1], mult, n)
        assert int(mix[0, 0]) == exp["mix"]
        idx = O.head_rows(mix, g["primes_per_order"][n_str], [0, 0])[0, 0]
        assert idx.tolist() == exp["indices"]


def test_worked_example_through_single_table():
    """Same example through hash_rows: one physical table, offsets = cumsum."""
    g = _golden("worked_example.json")
    primes = g["primes_per_order"]["2"] + g["primes_per_order"]["3"]
    offs, R = O.segment_offsets(primes)
    assert offs == [0, 101, 204, 311] and R == 420
    ident = np.arange(256, dtype=np.int32)
    ids = np.array([g["compressed_tokens"]], dtype=np.int32)
    rows, _ = O.hash_rows(ids, ident, 256, 0, g["multipliers_newest_first"] + [0],
                          primes, offs, max_ngram=3, heads=2)
    e2, e3 = g["expected"]["2"]["indices"], g["expected"]["3"]["indices"]
    assert rows[3].tolist() == [e2[0], e2[1] + 101, e3[0] + 204, e3[1] + 311]
    # the leading token lies outside both windows of the last position
    ids2 = ids.copy()
    ids2[0, 0] = 7
    rows2, _ = O.hash_rows(ids2, ident, 256, 0, g["multipliers_newest_first"] + [0],
                           primes, offs, max_ngram=3, heads=2)
    assert rows2[3].tolist() == rows[3].tolist()


def test_prime_table_of_both_layers():
    g = _golden("prime_table.json")
    n = g["primes_per_layer"]
    p = O.primes_from(g["engram_vocab_size"], 2 * n)
    for li, layer in enumerate(g["layers"]):
        seg = p[li * n:(li + 1) * n]
        assert min(seg) == layer["min_prime"]
        assert max(seg) == layer["max_prime"]
        assert sum(seg) == layer["sum"]
        assert O.segment_offsets(seg)[1] == g["config"]["engram_num_embeddings"][li]


def test_layer_primes_match_both_layers_table():
    g = _golden("prime_table.json")
    n = g["primes_per_layer"]
    primes, offs, rows = O.layer_primes(g["engram_vocab_size"], 2, n)
    for li, layer in enumerate(g["layers"]):
        assert len(primes[li]) == n
        assert min(primes[li]) == layer["min_prime"]
        assert max(primes[li]) == layer["max_prime"]
        assert sum(primes[li]) == layer["sum"]
        assert rows[li] == g["config"]["engram_num_embeddings"][li]
        assert offs[li][0] == 0 and offs[li][-1] + primes[li][-1] == rows[li]
    assert max(primes[0]) < min(primes[1])


def _two_layer_case(tokens=512):
    tm, _ = gen.hash_setup(C1)
    mults = gen.layer_multipliers(C1, 2)
    primes, offs, rows = O.layer_primes(C1.prime_base, 2, C1.segments)
    ids = gen.token_ids(C1)[0][:, :tokens]
    return tm, mults, primes, offs, rows, ids


def _layers(ids, tm, mults, primes, offs, hist=None):
    return O.hash_rows_layers(ids, tm, C1.compressed_vocab, int(tm[0]), mults, primes, offs,
                              C1.max_ngram, C1.heads, hist)


def test_two_layer_rows_stay_in_each_layers_segments():
    tm, mults, primes, offs, rows_per_layer, ids = _two_layer_case()
    rows, hist = _layers(ids, tm, mults, primes, offs)
    assert rows.shape == (2, ids.size, C1.segments)
    for li in range(2):
        lo = np.array(offs[li])
        hi = lo + np.array(primes[li])
        assert np.all(rows[li] >= lo) and np.all(rows[li] < hi)
        assert hi[-1] == rows_per_layer[li]
    # the history depends on the tokens only, not on the layer
    _, h1 = O.hash_rows(ids, tm, C1.compressed_vocab, int(tm[0]), mults[0], primes[0], offs[0],
                        C1.max_ngram, C1.heads)
    assert np.array_equal(hist, h1)
    # exchanging the layers' parameters exchanges their row ids
    swapped, _ = _layers(ids, tm, mults[::-1], primes[::-1], offs[::-1])
    assert np.array_equal(swapped[0], rows[1]) and np.array_equal(swapped[1], rows[0])


def test_layers_with_own_multipliers_hit_unrelated_rows():
    # P1: each layer draws its own multipliers, so even over the same primes the
    # same n-gram lands on unrelated rows; the same multipliers land on the same rows.
    tm, mults, primes, offs, _, ids = _two_layer_case()
    assert mults[0] != mults[1]
    own, _ = _layers(ids, tm, mults, [primes[0]] * 2, [offs[0]] * 2)
    assert np.mean(own[0] == own[1]) < 0.01
    same, _ = _layers(ids, tm, [mults[0]] * 2, [primes[0]] * 2, [offs[0]] * 2)
    assert np.array_equal(same[0], same[1])


def test_mx_values_one_scale_per_32_inputs():
    # code 0x38 is 1.0; block b carries scale 127 + b - 4, so element k is 2^(k//32 - 4)
    K = 256
    codes = np.full((3, K), 0x38, np.uint8)
    codes[1] = 0xB8                                   # -1.0
    codes[2, ::2] = 0x00                              # +0
    scales = np.tile(np.arange(123, 131, dtype=np.uint8), (3, 1))
    v = O.mx_values(codes, scales)
    expect = np.exp2(np.arange(K) // 32 - 4.0)
    assert np.array_equal(v[0], expect)
    assert np.array_equal(v[1], -expect)
    assert np.array_equal(v[2, 1::2], expect[1::2]) and not v[2, ::2].any()


def test_mx_values_equal_the_table_rows_dequant():
    # a table row is one MX block row of 256: its bytes give the same values
    rng = np.random.default_rng(21)
    rows = gen.table_rows(77, rng.integers(0, 10 ** 8, 64))
    v = O.mx_values(rows[:, :256], rows[:, 256:])
    assert np.array_equal(v, O.bf16_bits_to_f64(O.dequant_rows_bf16(rows)))


def test_gather_rows_are_the_table_bytes():
    rng = np.random.default_rng(22)
    R = 1000
    ids = rng.integers(-3, R + 3, (5, 6))
    fetch = lambda r: gen.table_rows(9, r)
    raw = O.gather_rows(fetch, ids, R)
    ok = (ids >= 0) & (ids < R)
    assert np.array_equal(raw[ok], gen.table_rows(9, ids[ok]))
    assert not raw[~ok].any()
    deq = O.bf16_bits_to_f64(O.dequant_rows_bf16(raw.reshape(-1, 264))).reshape(5, -1)
    assert np.array_equal(deq, O.bf16_bits_to_f64(O.gather_e4m3(fetch, ids, R)))


def test_primes_against_sympy():
    for base, count in ((1009, 6), (1_000_000, 24), (16_000_000, 30), (2, 10), (90, 5)):
        got = O.primes_from(base, count)
        exp = []
        q = sympy.nextprime(base - 1)
        while len(exp) < count:
            exp.append(int(q))
            q = sympy.nextprime(q)
        assert got == exp


def test_config_table_values():
    g = _golden("prime_table.json")["config"]
    assert C1.compressed_vocab == g["engram_compressed_vocab_size"]
    assert C1.raw_vocab == g["raw_vocab_size"]
    assert C1.max_ngram == g["engram_max_ngram_size"]
    assert C1.heads == g["engram_n_heads"]
    assert C1.row_dim == g["engram_head_dim"]
    assert C1.segments * C1.row_dim == 6144


def test_layer_facts():
    f = _golden("layer_facts.json")
    assert f["rows_per_token_per_layer"] == C1.segments
    assert f["row_bytes"] == gen.ROW_BYTES
    assert abs(C1.segments * gen.ROW_BYTES / 1000 - f["bytes_per_token_per_layer_approx_kb"]) < 0.05
    assert abs(2 * C1.segments * gen.ROW_BYTES / 1024 - f["two_layer_kib_approx"]) < 0.35
    g = _golden("prime_table.json")["config"]
    params = sum(g["engram_num_embeddings"]) * g["engram_head_dim"] / 1e9
    assert abs(params - f["two_table_params_billion_approx"]) < 0.05


def _c1_setup(w=C1, tokens=None):
    tm, mult = gen.hash_setup(w)
    primes = O.primes_from(w.prime_base, w.segments)
    offs, R = O.segment_offsets(primes)
    ids, spans = gen.token_ids(w)
    if tokens is not None:
        ids = ids[:, :tokens]
    return tm, mult, primes, offs, R, ids, spans


def test_segments_disjoint_and_cover_table():
    tm, mult, primes, offs, R, ids, _ = _c1_setup()
    rows, _ = O.hash_rows(ids, tm, C1.compressed_vocab, int(tm[0]), mult, primes, offs,
                          C1.max_ngram, C1.heads)
    assert rows.shape == (C1.tokens, 24)
    lo = np.array(offs)
    hi = lo + np.array(primes)
    assert np.all(rows >= lo) and np.all(rows < hi)
    assert hi[-1] == R and np.all(lo[1:] == hi[:-1])
    assert R == _golden("prime_table.json")["config"]["engram_num_embeddings"][0]


# ---------------------------------------------------------------------------
# hash: order sensitivity, incremental mixing, overflow, CRT bound
# ---------------------------------------------------------------------------

def test_order_sensitivity_all_pairs_c0():
    _, mult = gen.hash_setup(C0)
    V = C0.compressed_vocab
    a, b = np.meshgrid(np.arange(V), np.arange(V), indexing="ij")
    sel = a != b
    ab = np.stack([a[sel], b[sel]], -1)       # cells: c0 = A (newest), c1 = B
    ba = ab[:, ::-1]
    assert not np.any(O.mix_values(ab, mult, 2) == O.mix_values(ba, mult, 2))


def test_order_sensitivity_sampled_full_vocab():
    _, mult = gen.hash_setup(C1)
    rng = np.random.default_rng(5)
    a = rng.integers(0, C1.compressed_vocab, 200_000)
    b = rng.integers(0, C1.compressed_vocab, 200_000)
    keep = a != b
    ab = np.stack([a[keep], b[keep]], -1)
    assert not np.any(O.mix_values(ab, mult, 2) == O.mix_values(ab[:, ::-1], mult, 2))


def test_incremental_mixing():
    tm, mult, *_ , ids, _ = _c1_setup(tokens=512)
    xc = O.compress(ids, tm, C1.compressed_vocab)
    cells, _ = O.ngram_cells(xc, int(tm[0]), 4)
    m2, m3, m4 = (O.mix_values(cells, mult, n) for n in (2, 3, 4))
    c = cells.astype(np.uint64)
    assert np.array_equal(m3, m2 ^ (c[..., 2] * np.uint64(mult[2])))
    assert np.array_equal(m4, m3 ^ (c[..., 3] * np.uint64(mult[3])))


def test_heads_share_one_mix():
    """The 8 heads of an order are one 64-bit mix taken mod 8 primes: the head
    rows are congruent to a single value modulo each prime (CRT reconstruction
    recovers the same mix from any 3 heads at base 16,000,000)."""
    tm, mult, primes, offs, R, ids, _ = _c1_setup(tokens=64)
    rows, _ = O.hash_rows(ids, tm, C1.compressed_vocab, int(tm[0]), mult, primes, offs, 4, 8)
    xc = O.compress(ids, tm, C1.compressed_vocab)
    cells, _ = O.ngram_cells(xc, int(tm[0]), 4)
    for n in (2, 3, 4):
        mix = O.mix_values(cells, mult, n).reshape(-1)
        z = rows[:, (n - 2) * 8:(n - 1) * 8] - np.array(offs[(n - 2) * 8:(n - 1) * 8])
        for t in range(0, 64, 7):
            for trio in ((0, 1, 2), (3, 5, 7)):
                ps = [primes[(n - 2) * 8 + k] for k in trio]
                rs = [int(z[t, k]) for k in trio]
                rec, mod = sympy.ntheory.modular.crt(ps, rs)
                assert int(rec) == int(mix[t]) and mod > 2 ** 63


def test_no_overflow():
    for w in (C0, C1):
        _, mult = gen.hash_setup(w)
        lim = O.multiplier_limit(w.compressed_vocab)
        assert lim == ((1 << 63) - 1) // w.compressed_vocab
        for m in mult:
            assert m % 2 == 1 and 0 < m <= lim
            assert (w.compressed_vocab - 1) * m <= (1 << 63) - 1
    tm, mult, primes, offs, R, ids, _ = _c1_setup()
    xc = O.compress(ids, tm, C1.compressed_vocab)
    cells, _ = O.ngram_cells(xc, int(tm[0]), 4)
    for n in (2, 3, 4):
        assert int(O.mix_values(cells, mult, n).max()) < (1 << 63)


def test_crt_bound_closed_form():
    two63 = 2 ** 63
    for base, bound in ((16_000_000, 2), (1_000_000, 3)):
        p = sorted(O.primes_from(base, 24))
        # fewest-digit products decide: any bound+1 primes multiply past 2^63
        assert math.prod(p[:bound + 1]) > two63
        assert math.prod(p[:bound]) < two63 or bound == 2
    p16 = sorted(O.primes_from(16_000_000, 24))
    assert math.prod(p16[:3]) > 4.0e21            # page: about 4 x 10^21


def test_crt_bound_brute_force_tiny():
    primes = [11, 13, 17, 19, 23, 29, 31, 37]
    offs = [0] * 8
    lim = 11 * 13 * 17
    a = np.arange(lim, dtype=np.uint64)
    z = O.head_rows(a, primes, offs)                 # [lim, 8]
    worst = 0
    for i in range(lim - 1):
        shared = (z[i + 1:] == z[i]).sum(axis=1)
        worst = max(worst, int(shared.max()))
    assert worst == 2
    # tight: b = a + 11*13 shares exactly heads {11, 13}
    for a0 in (0, 5, 100, 2000):
        b0 = a0 + 11 * 13
        same = np.nonzero(O.head_rows(np.array([a0], np.uint64), primes, offs)[0]
                          == O.head_rows(np.array([b0], np.uint64), primes, offs)[0])[0]
        assert same.tolist() == [0, 1]


def test_crt_bound_full_shape():
    tm, mult, primes, offs, R, ids, _ = _c1_setup()
    P = primes[8:16]                               # order 3 heads
    rng = np.random.default_rng(9)
    xc = O.compress(ids, tm, C1.compressed_vocab)
    cells, _ = O.ngram_cells(xc, int(tm[0]), 4)
    mix = np.unique(O.mix_values(cells, mult, 3).reshape(-1))
    z = O.head_rows(mix, P, [0] * 8)
    i = rng.integers(0, len(mix), 200_000)
    j = rng.integers(0, len(mix), 200_000)
    keep = i != j
    assert (z[i[keep]] == z[j[keep]]).sum(axis=1).max() <= 2
    for (hi, hj) in ((0, 1), (2, 7), (4, 5)):
        a0 = int(mix[3])
        b0 = a0 + P[hi] * P[hj]
        same = np.nonzero(O.head_rows(np.array([a0], np.uint64), P, [0] * 8)[0]
                          == O.head_rows(np.array([b0], np.uint64), P, [0] * 8)[0])[0]
        assert same.tolist() == sorted([hi, hj])


# ---------------------------------------------------------------------------
# hash: pad and DEAD semantics, history
# ---------------------------------------------------------------------------

def test_pad_and_dead_cells_c0():
    tm, mult = gen.hash_setup(C0)
    pad = int(tm[0])
    ids, spans = gen.token_ids(C0)
    assert spans[0] == [(20, 28)]
    xc = O.compress(ids, tm, C0.compressed_vocab)
    cells, dead = O.ngram_cells(xc, pad, 4)
    c = cells[0]
    x = xc[0]
    assert c[0].tolist() == [x[0], pad, pad, pad]
    assert c[1].tolist() == [x[1], x[0], pad, pad]
    assert c[2].tolist() == [x[2], x[1], x[0], pad]
    assert dead[0, 20:28].all() and not dead[0, :20].any() and not dead[0, 28:].any()
    for t in range(20, 28):
        assert c[t].tolist() == [pad] * 4
    assert c[28].tolist() == [x[28], pad, pad, pad]
    assert c[29].tolist() == [x[29], x[28], pad, pad]
    assert c[30].tolist() == [x[30], x[29], x[28], pad]
    for t in list(range(3, 20)) + list(range(31, 64)):
        assert c[t].tolist() == [x[t], x[t - 1], x[t - 2], x[t - 3]]


def test_dead_rows_are_the_all_pad_ngram():
    tm, mult = gen.hash_setup(C0)
    pad = int(tm[0])
    primes = O.primes_from(C0.prime_base, C0.segments)
    offs, R = O.segment_offsets(primes)
    ids, _ = gen.token_ids(C0)
    rows, _ = O.hash_rows(ids, tm, C0.compressed_vocab, pad, mult, primes, offs, 4, 2)
    all_pad = np.array([[0, pad, pad, pad, pad]])[:, 1:]
    # an all-pad sequence of length 4 gives the all-pad n-gram at t = 3
    pad_raw = np.zeros((1, 4), np.int32)
    rows_pad, _ = O.hash_rows(pad_raw, tm, C0.compressed_vocab, pad, mult, primes, offs, 4, 2)
    for t in range(20, 28):
        assert rows[t].tolist() == rows_pad[3].tolist()
    assert all_pad.shape == (1, 4)


def test_invalid_ids_count_as_dead():
    tm, mult, primes, offs, R, ids, _ = _c1_setup(tokens=64)
    pad = int(tm[0])
    bad = ids[:1].copy()
    bad[0, 10] = C1.raw_vocab + 5
    bad[0, 20] = -7
    dead = ids[:1].copy()
    dead[0, 10] = -1
    dead[0, 20] = -1
    r1, h1 = O.hash_rows(bad, tm, C1.compressed_vocab, pad, mult, primes, offs, 4, 8)
    r2, h2 = O.hash_rows(dead, tm, C1.compressed_vocab, pad, mult, primes, offs, 4, 8)
    assert np.array_equal(r1, r2) and np.array_equal(h1, h2)


@pytest.mark.parametrize("splits", [(1,), (2,), (3,), (5, 17), (255, 256, 257), (1, 2, 3, 4)])
def test_chunked_prefill_equals_one_shot(splits):
    tm, mult, primes, offs, R, ids, _ = _c1_setup()
    pad = int(tm[0])
    seq = ids[:2, 600:1200].copy()          # crosses a DEAD span boundary in some rows
    seq[1, 255:259] = -1
    full, hfull = O.hash_rows(seq, tm, C1.compressed_vocab, pad, mult, primes, offs, 4, 8)
    full = full.reshape(2, -1, 24)
    bounds = [0] + list(splits) + [seq.shape[1]]
    hist = None
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        r, hist = O.hash_rows(seq[:, a:b], tm, C1.compressed_vocab, pad, mult, primes, offs,
                              4, 8, hist=hist)
        parts.append(r.reshape(2, b - a, 24))
    assert np.array_equal(np.concatenate(parts, axis=1), full)
    assert np.array_equal(hist, hfull)


def test_decode_with_history_equals_prefill_tail():
    tm, mult, primes, offs, R, ids, _ = _c1_setup()
    pad = int(tm[0])
    seq = ids[:4, 1000:1040].copy()
    seq[2, 37] = -1
    seq[3, 39] = -1
    full, _ = O.hash_rows(seq, tm, C1.compressed_vocab, pad, mult, primes, offs, 4, 8)
    full = full.reshape(4, -1, 24)
    _, hist = O.hash_rows(seq[:, :-1], tm, C1.compressed_vocab, pad, mult, primes, offs, 4, 8)
    step, hist2 = O.hash_rows(seq[:, -1:], tm, C1.compressed_vocab, pad, mult, primes, offs,
                              4, 8, hist=hist)
    assert np.array_equal(step.reshape(4, 24), full[:, -1])
    xc = O.compress(seq, tm, C1.compressed_vocab)
    assert np.array_equal(hist2, xc[:, -3:].astype(np.int32))


def test_history_of_short_chunks():
    tm, mult, primes, offs, R, ids, _ = _c1_setup(tokens=8)
    pad = int(tm[0])
    xc = O.compress(ids[:1], tm, C1.compressed_vocab)
    _, h = O.hash_rows(ids[:1, :1], tm, C1.compressed_vocab, pad, mult, primes, offs, 4, 8)
    assert h[0].tolist() == [pad, pad, int(xc[0, 0])]
    _, h0 = O.hash_rows(ids[:1, :0], tm, C1.compressed_vocab, pad, mult, primes, offs, 4, 8,
                        hist=np.array([[5, -1, 7]], np.int32))
    assert h0[0].tolist() == [5, -1, 7]


def test_decode_dead_sequence_reads_all_pad_rows():
    """C4's sequence 0: new id DEAD, history all DEAD -> the all-pad n-gram."""
    tm, mult = gen.hash_setup(C4)
    pad = int(tm[0])
    primes = O.primes_from(C4.prime_base, 24)
    offs, _ = O.segment_offsets(primes)
    ids, _ = gen.token_ids(C4)
    hist = gen.history(C4, tm)
    assert ids[0, 0] == -1 and hist[0].tolist() == [-1, -1, -1]
    rows, hout = O.hash_rows(ids, tm, C4.compressed_vocab, pad, mult, primes, offs, 4, 8,
                             hist=hist)
    pad4, _ = O.hash_rows(np.zeros((1, 4), np.int32), tm, C4.compressed_vocab, pad, mult,
                          primes, offs, 4, 8)
    assert rows[0].tolist() == pad4[3].tolist()
    assert hout[0].tolist() == [-1, -1, -1]


# ---------------------------------------------------------------------------
# dequantisation and bf16 rounding against torch's float8 / bfloat16
# ---------------------------------------------------------------------------

def test_dequant_exhaustive_against_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    q = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float()
    s = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).float()
    prod = (q[None, :] * s[:, None])                 # [scale, code], exact in fp32
    ref = prod.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    rows = np.zeros((256, 8, 264), dtype=np.uint8)   # 8 rows per scale cover 256 codes
    for S in range(256):
        for r in range(8):
            rows[S, r, :256] = codes[(r * 32 + np.arange(256)) % 256]
            rows[S, r, 256:] = S
    got = O.dequant_rows_bf16(rows.reshape(-1, 264)).reshape(256, 8, 256)
    for S in range(256):
        for r in range(8):
            cs = (r * 32 + np.arange(256)) % 256
            exp = ref[S, cs]
            g = got[S, r]
            nan_e = np.isnan(prod[S, cs].numpy())
            nan_g = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
            assert np.array_equal(nan_e, nan_g)
            assert np.array_equal(g[~nan_e], exp[~nan_e])
    # the workloads' scale range 120..134 never leaves the bf16 normal range
    for S in range(120, 135):
        fin = ~np.isnan(prod[S].numpy())
        v = np.abs(prod[S].numpy()[fin]).astype(np.float64)
        v = v[v > 0]
        assert v.min() >= 2.0 ** -126 and v.max() < 2.0 ** 128


def test_round_to_bf16_against_torch():
    rng = np.random.default_rng(3)
    parts = [
        rng.standard_normal(200_000).astype(np.float32) * np.float32(1e3),
        (rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895314e38, -3.3895314e38,
                  1e-40, -1e-42, 1.17549435e-38, 9.18e-41, np.inf, -np.inf], dtype=np.float32),
    ]
    x = np.concatenate(parts)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = O.round_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)
    # halfway cases built to exercise ties-to-even on both sides
    base = rng.integers(0, 2 ** 15, 10_000).astype(np.uint32) << np.uint32(16)
    half = (base | np.uint32(0x8000)).view(np.float32)
    half = half[np.isfinite(half)]
    ref = torch.from_numpy(half.copy()).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(O.round_to_bf16_bits(half.astype(np.float64)), ref)


def test_gather_zero_rows_and_copy():
    table = np.arange(40 * 8, dtype=np.float32).reshape(40, 8)
    rid = np.array([[0, 39, 40, -1], [7, 1_000_000, 3, 3]], dtype=np.int64)
    e = O.gather_f32(table, rid).reshape(2, 4, 8)
    assert np.array_equal(e[0, 0], table[0]) and np.array_equal(e[0, 1], table[39])
    assert not e[0, 2].any() and not e[0, 3].any() and not e[1, 1].any()
    assert np.array_equal(e[1, 2], table[3]) and np.array_equal(e[1, 0], table[7])
    rows = gen.table_rows(11, np.arange(16))
    got = O.gather_e4m3(lambda r: gen.table_rows(11, r), np.array([[3, 16, -2, 15]]), 16)
    got = got.reshape(4, 256)
    assert not got[1].any() and not got[2].any()
    assert np.array_equal(got[0], O.dequant_rows_bf16(rows[3])[0])
    assert np.array_equal(got[3], O.dequant_rows_bf16(rows[15])[0])


def test_table_rows_format():
    rows = gen.table_rows(2002, np.array([0, 1, 24_003_915, 384_006_167]))
    pay, sc = rows[:, :256], rows[:, 256:]
    assert not np.any(pay == 0x7F) and not np.any(pay == 0xFF)
    assert sc.min() >= 120 and sc.max() <= 134


# ---------------------------------------------------------------------------
# projection and gate: special cases and closed forms
# ---------------------------------------------------------------------------

def test_projection_one_hot_picks_weight_columns():
    rng = np.random.default_rng(1)
    W = rng.standard_normal((40, 24))              # [(hc+1)*d, K]
    e = np.zeros((24, 24))
    e[np.arange(24), np.arange(24)] = 1.0
    kv = O.project(e, W)
    assert np.array_equal(kv, W.T)
    e2 = np.zeros((3, 24))
    e2[0, 5] = 2.0
    e2[1, 0] = -0.5
    e2[1, 23] = 4.0
    kv2 = O.project(e2, W)
    assert np.array_equal(kv2[0], 2.0 * W[:, 5])
    assert np.array_equal(kv2[1], -0.5 * W[:, 0] + 4.0 * W[:, 23])
    assert not kv2[2].any()


def _unit_gate(h, k, d, dead=False, clamp=0.0, eps=1e-6):
    ones = np.ones((1, d))
    v = np.ones((1, d))
    return O.gate(h.reshape(1, 1, d), k.reshape(1, 1, d), v, ones, ones,
                  np.array([dead]), eps=eps, clamp=clamp)


def test_gate_closed_forms():
    f = _golden("layer_facts.json")
    d = f["d"]
    rng = np.random.default_rng(2)
    h = rng.standard_normal(d)
    # h parallel to k: s = sqrt(d) (up to eps), alpha = sigmoid(d^(1/4))
    a, _ = _unit_gate(h, 3.0 * h, d)
    s = math.sqrt(d)
    assert abs(s - f["s_max_abs"]) < 0.05
    assert abs(math.sqrt(s) - f["signed_sqrt_max_abs"]) < 0.05
    assert abs(a[0, 0] - 1 / (1 + math.exp(-math.sqrt(s)))) < 1e-9
    assert abs(a[0, 0] - 0.99979) < 1e-5
    a, _ = _unit_gate(h, -h, d)
    assert abs(a[0, 0] - 1 / (1 + math.exp(math.sqrt(s)))) < 1e-9
    assert abs(a[0, 0] - 2.1e-4) < 1e-5
    # h orthogonal to k: s = 0, alpha = 1/2
    k = rng.standard_normal(d)
    k -= h * (k @ h) / (h @ h)
    a, _ = _unit_gate(h, k, d)
    assert abs(a[0, 0] - 0.5) < 1e-6       # |s| ~ 1e-16 residue, amplified by the root
    # cosine: s = sqrt(d) cos(theta) for unit weights, |s| <= sqrt(d)
    for _ in range(5):
        k = rng.standard_normal(d)
        cos = (h @ k) / np.linalg.norm(h) / np.linalg.norm(k)
        a, _ = _unit_gate(h, k, d)
        sg = math.copysign(math.sqrt(abs(s * cos)), cos)
        assert abs(a[0, 0] - 1 / (1 + math.exp(-sg))) < 1e-6


def test_gate_is_scale_invariant_and_clamped():
    d = 256
    rng = np.random.default_rng(4)
    h, k = rng.standard_normal(d), rng.standard_normal(d)
    a1, _ = _unit_gate(h, k, d, eps=0.0)
    a2, _ = _unit_gate(7.0 * h, 0.25 * k, d, eps=0.0)
    assert abs(a1[0, 0] - a2[0, 0]) < 1e-9
    # eps sits inside the root: a tiny k is damped towards s = 0
    a3, _ = _unit_gate(h, 1e-6 * k, d, eps=1e-6)
    assert abs(a3[0, 0] - 0.5) < abs(a1[0, 0] - 0.5) / 10
    k0 = k - h * (k @ h) / (h @ h)           # s = 0
    a, _ = _unit_gate(h, k0, d, clamp=4.0)
    assert abs(abs(a[0, 0] - 0.5) - abs(1 / (1 + math.exp(-2.0)) - 0.5)) < 1e-9


def test_gate_dead_and_zero_value_leave_h():
    d, hc, T = 64, 2, 3
    rng = np.random.default_rng(6)
    h = rng.standard_normal((T, hc, d))
    k = rng.standard_normal((T, hc, d))
    v = rng.standard_normal((T, d))
    qw = 1 + 0.1 * rng.standard_normal((hc, d))
    kw = 1 + 0.1 * rng.standard_normal((hc, d))
    dead = np.array([False, True, False])
    a, h2 = O.gate(h, k, v, qw, kw, dead, 1e-6)
    assert np.all(a[1] == 0) and np.array_equal(h2[1], h[1])
    assert np.all((a[[0, 2]] > 0) & (a[[0, 2]] < 1))
    np.testing.assert_allclose(h2[0], h[0] + a[0][:, None] * v[0][None], rtol=0, atol=1e-12)
    a0, h3 = O.gate(h, k, np.zeros_like(v), qw, kw, np.zeros(T, bool), 1e-6)
    assert np.array_equal(h3, h)


def test_gate_weights_multiply_the_dot():
    """With q_w * k_w = c on one stream the score scales by c (before the root)."""
    d = 128
    rng = np.random.default_rng(8)
    h = rng.standard_normal((1, 1, d))
    k = h + 0.3 * rng.standard_normal((1, 1, d))
    v = np.zeros((1, d))
    one = np.ones((1, d))
    a1, _ = O.gate(h, k, v, one, one, np.array([False]), 0.0)
    a2, _ = O.gate(h, k, v, 2.0 * one, 0.5 * one, np.array([False]), 0.0)
    a3, _ = O.gate(h, k, v, 0.5 * one, 0.5 * one, np.array([False]), 0.0)
    logit = lambda a: math.log(a / (1 - a))
    assert abs(a1[0, 0] - a2[0, 0]) < 1e-12
    assert abs(logit(a3[0, 0]) ** 2 - 0.25 * logit(a1[0, 0]) ** 2) < 1e-9


# ----------------------------------------------------------------------------
# The papers' variants: plain sigmoid gate, short convolution branch
# ----------------------------------------------------------------------------

def test_plain_gate_closed_forms():
    """[P5] §4.1: alpha = sigmoid(s); [P1] "门控": s = sqrt(d) cos(theta)."""
    f = _golden("layer_facts.json")
    d = f["d"]
    rng = np.random.default_rng(12)
    h = rng.standard_normal(d)
    ones = np.ones((1, d))

    def plain(h, k, dd=d, eps=0.0, clamp=0.0):
        a, _ = O.gate(h.reshape(1, 1, dd), k.reshape(1, 1, dd), np.ones((1, dd)),
                      np.ones((1, dd)), np.ones((1, dd)), np.array([False]), eps=eps,
                      clamp=clamp, mode="plain")
        return a[0, 0]

    # parallel at d = 5120: s = sqrt(d) = 71.55, the gate saturates
    assert abs(plain(h, 2.0 * h) - 1 / (1 + math.exp(-math.sqrt(d)))) < 1e-12
    assert plain(-h, h) < 1e-30
    # d = 4, h = k: s = 2 exactly, plain sigmoid(2) against the signed root's sigmoid(sqrt 2)
    x = np.array([1.0, -2.0, 0.5, 3.0])
    assert abs(plain(x, x, dd=4) - 1 / (1 + math.exp(-2.0))) < 1e-12
    a_sq, _ = O.gate(x.reshape(1, 1, 4), x.reshape(1, 1, 4), np.ones((1, 4)), np.ones((1, 4)),
                     np.ones((1, 4)), np.array([False]), eps=0.0)
    assert abs(a_sq[0, 0] - 1 / (1 + math.exp(-math.sqrt(2.0)))) < 1e-12
    # orthogonal: 1/2; the clamp only enters the signed root
    k = rng.standard_normal(d)
    k -= h * (k @ h) / (h @ h)
    assert abs(plain(h, k) - 0.5) < 1e-9
    assert abs(plain(h, k, clamp=4.0) - 0.5) < 1e-9
    for _ in range(4):
        k = rng.standard_normal(d)
        cos = (h @ k) / np.linalg.norm(h) / np.linalg.norm(k)
        assert abs(plain(h, k) - 1 / (1 + math.exp(-math.sqrt(d) * cos))) < 1e-9
    with pytest.raises(ValueError):
        O.gate(h.reshape(1, 1, d), h.reshape(1, 1, d), ones, ones, ones, np.array([False]),
               eps=0.0, mode="softmax")


def _conv_case(B=2, T=14, hc=2, d=16, taps=4, seed=20):
    rng = np.random.default_rng(seed)
    vt = rng.standard_normal((B, T, hc, d))
    w = rng.standard_normal((hc, d, taps))
    g = 1 + 0.2 * rng.standard_normal((hc, d))
    return vt, w, g


def test_short_conv_zero_filters_leave_the_gated_value():
    """[P5] §4.2: filters start at zero, so the branch starts as V~ itself."""
    vt, w, g = _conv_case()
    y = O.short_conv(vt, np.zeros_like(w), g, 3, 1e-6)
    assert np.array_equal(y, vt)
    rng = np.random.default_rng(21)
    B, T, hc, d = 2, 7, 3, 32
    h, k = rng.standard_normal((2, B, T, hc, d))
    v = rng.standard_normal((B, T, d))
    qw, kw = 1 + 0.1 * rng.standard_normal((2, hc, d))
    dead = rng.random((B, T)) < 0.2
    a0, h0 = O.gate(h.reshape(-1, hc, d), k.reshape(-1, hc, d), v.reshape(-1, d), qw, kw,
                    dead.reshape(-1), 1e-6)
    a1, h1, _ = O.gate_conv(h, k, v, qw, kw, dead, 1e-6, 0.0, np.zeros((hc, d, 4)), None, 3,
                            1e-6)
    assert np.array_equal(a1.reshape(-1, hc), a0)
    np.testing.assert_allclose(h1.reshape(-1, hc, d), h0, rtol=0, atol=1e-13)


def test_short_conv_equals_torch_rmsnorm_conv1d_silu():
    """The whole branch as library routines: rms_norm, a grouped (depthwise)
    conv1d padded by (taps-1)*dilation and cut to T outputs, silu."""
    import torch.nn.functional as F
    for taps, dil in ((4, 3), (1, 1), (2, 1), (3, 5)):
        vt, w, g = _conv_case(taps=taps, seed=22 + taps)
        B, T, hc, d = vt.shape
        y = O.short_conv(vt, w, g, dil, 1e-5)
        x = torch.from_numpy(vt)
        xn = F.rms_norm(x, (d,), None, 1e-5) * torch.from_numpy(g)   # [B, T, hc, d]
        xc = xn.reshape(B, T, hc * d).transpose(1, 2)                   # [B, C, T]
        wt = torch.from_numpy(w).reshape(hc * d, 1, taps)
        u = F.conv1d(xc, wt, padding=(taps - 1) * dil, dilation=dil, groups=hc * d)[..., :T]
        ref = (F.silu(u).transpose(1, 2).reshape(B, T, hc, d) + x).numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_short_conv_reaches_t_minus_3_6_9():
    """[P5] §4.2: with 4 taps at dilation 3 position t uses t, t-3, t-6, t-9;
    each stream is normalised and filtered on its own, each sequence too."""
    vt, w, g = _conv_case(B=2, T=20, hc=2)
    y0 = O.short_conv(vt, w, g, 3, 1e-6)
    t0 = 4
    vt2 = vt.copy()
    vt2[1, t0, 0, 5] += 0.75
    changed = np.any(O.short_conv(vt2, w, g, 3, 1e-6) != y0, axis=-1)   # [B, T, hc]
    expect = np.zeros_like(changed)
    expect[1, [t0, t0 + 3, t0 + 6, t0 + 9], 0] = True
    assert np.array_equal(changed, expect)
    assert O.conv_history_len(4, 3) == 9
    # depthwise: one channel's filter moves only that channel
    w2 = w.copy()
    w2[1, 7, 2] += 1.0
    diff = O.short_conv(vt, w2, g, 3, 1e-6) != y0
    assert diff[:, :, 1, 7].any() and not np.delete(diff.reshape(2, 20, -1), 16 + 7, axis=2).any()


def test_short_conv_tiny_by_hand():
    """d = 2, one stream, V~ = (a, -a): RMSNorm gives (1, -1) times the norm
    weight (eps 0), so Y = SiLU(u) + V~ with u a weighted sum of those."""
    sig = lambda x: 1 / (1 + math.exp(-x))
    a = 0.3
    vt = np.array([a, -a]).reshape(1, 1, 1, 2)
    w = np.array([2.0, 3.0]).reshape(1, 2, 1)
    y = O.short_conv(vt, w, None, 1, 0.0).reshape(2)
    assert abs(y[0] - (2 * sig(2) + a)) < 1e-14
    assert abs(y[1] - (-3 * sig(-3) - a)) < 1e-14
    # two taps, dilation 2, three positions; values (a,-a), (b,-b), (c,-c)
    vals = [0.3, -1.5, 2.0]
    vt = np.array([[v, -v] for v in vals]).reshape(1, 3, 1, 2)
    w = np.array([[0.5, 4.0], [-1.0, 2.0]]).reshape(1, 2, 2)            # [hc, d, taps]
    g = np.array([[1.0, 0.5]])
    y = O.short_conv(vt, w, g, 2, 0.0).reshape(3, 2)
    sgn = lambda x: math.copysign(1.0, x)
    for t in range(3):
        n_now = [sgn(vals[t]) * 1.0, -sgn(vals[t]) * 0.5]
        n_back = [0.0, 0.0] if t < 2 else [sgn(vals[t - 2]), -sgn(vals[t - 2]) * 0.5]
        for c in range(2):
            u = w[0, c, 1] * n_now[c] + w[0, c, 0] * n_back[c]
            assert abs(y[t, c] - (u * sig(u) + (vals[t] if c == 0 else -vals[t]))) < 1e-14


@pytest.mark.parametrize("splits", [(1,), (2, 3), (4, 5), (9,), (10, 1, 1, 1), (13,)])
def test_gate_conv_chunked_equals_one_shot(splits):
    """Chunks that carry the last 9 gated values on equal the whole sequence
    ([P5] §9.5: chunked prefill and decode keep the convolution's history)."""
    rng = np.random.default_rng(30)
    B, T, hc, d = 2, 16, 2, 24
    h, k = rng.standard_normal((2, B, T, hc, d))
    v = rng.standard_normal((B, T, d))
    qw, kw = 1 + 0.1 * rng.standard_normal((2, hc, d))
    cw = 0.5 * rng.standard_normal((hc, d, 4))
    nw = 1 + 0.1 * rng.standard_normal((hc, d))
    dead = rng.random((B, T)) < 0.15
    a, ho, tail = O.gate_conv(h, k, v, qw, kw, dead, 1e-6, 0.0, cw, nw, 3, 1e-6)
    hist, t0, pa, ph = None, 0, [], []
    for n in list(splits) + [T - sum(splits)]:
        sl = slice(t0, t0 + n)
        a_, h_, hist = O.gate_conv(h[:, sl], k[:, sl], v[:, sl], qw, kw, dead[:, sl], 1e-6, 0.0,
                                   cw, nw, 3, 1e-6, hist)
        pa.append(a_)
        ph.append(h_)
        t0 += n
    np.testing.assert_allclose(np.concatenate(pa, 1), a, rtol=0, atol=1e-14)
    np.testing.assert_allclose(np.concatenate(ph, 1), ho, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hist, tail, rtol=0, atol=1e-14)
    assert hist.shape == (B, 9, hc, d)
    vt = a[..., None] * v[:, :, None, :]
    np.testing.assert_allclose(tail, vt[:, -9:], rtol=0, atol=1e-14)


def test_gate_conv_dead_positions():
    """A DEAD position keeps its streams and feeds V~ = 0 to its neighbours."""
    rng = np.random.default_rng(31)
    B, T, hc, d = 1, 12, 2, 16
    h, k = rng.standard_normal((2, B, T, hc, d))
    v = rng.standard_normal((B, T, d))
    qw = kw = np.ones((hc, d))
    cw = rng.standard_normal((hc, d, 4))
    dead = np.zeros((B, T), bool)
    dead[0, 6] = True            # its own branch input is 0, but it reaches t = 3 and t = 0
    a, ho, _ = O.gate_conv(h, k, v, qw, kw, dead, 1e-6, 0.0, cw, None, 3, 1e-6)
    assert np.array_equal(ho[0, 6], h[0, 6]) and np.all(a[0, 6] == 0)
    vt = a[..., None] * v[:, :, None, :]
    assert not vt[0, 6].any()
    y = O.short_conv(vt, cw, None, 3, 1e-6)
    assert np.abs(y[0, 6]).min() > 0            # the branch is not zero there, yet h stays
    live = ~dead[0]
    np.testing.assert_allclose(ho[0, live], h[0, live] + y[0, live], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# compression map, and the whole layer on hand-built inputs
# ---------------------------------------------------------------------------

def test_compress_hand_built_map():
    """x' = P[x] on a six-entry map whose values include two outside [0, V'):
    P1 "tokenizer 压缩" (the map), and the reading that a raw id outside [0, V),
    the DEAD marker and a map value outside [0, V') all come out DEAD."""
    tm = np.array([3, 0, 7, 9, -2, 5], dtype=np.int32)          # V = 6, V' = 8
    ids = np.array([[0, 1, 2, 3, 4, 5, 6, -1, -5, 2, 1]], dtype=np.int32)
    got = O.compress(ids, tm, 8)
    assert got.tolist() == [[3, 0, 7, -1, -1, 5, -1, -1, -1, 7, 0]]
    # with V' = 10 the value 9 is a valid compressed id
    assert O.compress(np.array([[3]], np.int32), tm, 10).tolist() == [[9]]
    # an invalid map value blocks its cell and every older one, like DEAD
    # (pad' = P[0] = 3): at t = 2 the window is (7, [9 -> DEAD], 0, pad)
    xc = O.compress(np.array([[1, 3, 2]], np.int32), tm, 8)
    cells, dead = O.ngram_cells(xc, 3, 4)
    assert cells[0, 2].tolist() == [7, 3, 3, 3]
    assert cells[0, 0].tolist() == [0, 3, 3, 3]
    assert dead[0].tolist() == [False, True, False]


# One-hot rows make every kv row a column of W (times a power of two), so the
# gate and the update of each stream have closed forms. Stream m of a token
# whose row is r sees h = a_t * (1, ..., 1) and k = c_m * sigma, where sigma has
# P[r][m] entries +1 followed by d - P[r][m] entries -1. With unit weights the
# two mean squares are a_t^2 and c_m^2, so
#   s = a_t c_m (2P - d) / (sqrt(a_t^2 + eps) sqrt(c_m^2 + eps) sqrt(d)),
# i.e. sqrt(d) cos(theta) up to eps (P1 "门控").
_FT_D = 8
_FT_HC = 4
_FT_P = [[8, 6, 2, 4], [2, 4, 8, 6], [6, 8, 4, 2], [8, 8, 8, 8], [4, 2, 6, 8]]
_FT_C = [1.0, -2.0, 0.5, 4.0]                        # key scale of stream m (bf16 exact)
_FT_POS = [5, 200, 33, 64, 255]                      # one-hot input of row r (segment 0)
_FT_SH = [0, 1, -1, 2, 0]                            # the row's value is 2^SH
_FT_V = np.array([0.5, -1.25, 3.0, 7.5, -0.375, 10.0, -6.0, 2.25])   # bf16 exact
_FT_A = [1.5, -2.0, 0.75, 3.0, 1.0, -0.5]            # h scale of token t
# token t reads rows ROWS[t] = (segment 0, segment 1); ids 5..9 are all-zero
# rows, -1 and 10 (= R) lie outside the table
_FT_ROWS = np.array([[0, 5], [1, 6], [2, 7], [3, 8], [-1, 9], [4, 10]], dtype=np.int64)
_FT_DEAD = np.array([False, False, False, True, False, False])
_FT_TOK_ROW = [0, 1, 2, 3, None, 4]                  # the one-hot row of token t
_FT_EPS = 1e-6


def _ft_w(row_dim):
    """W [(hc+1) d, 2 row_dim]: column POS[r] holds the keys c_m sigma and the
    value V (1 + 2^-10), which bf16 rounds down to V (half an ulp is >= 2^-9)."""
    d, hc = _FT_D, _FT_HC
    w = np.zeros(((hc + 1) * d, 2 * row_dim))
    for r, pos in enumerate(_FT_POS):
        p = pos % row_dim
        for m in range(hc):
            sig = np.where(np.arange(d) < _FT_P[r][m], 1.0, -1.0)
            w[m * d:(m + 1) * d, p] = _FT_C[m] * sig
        w[hc * d:, p] = _FT_V * (1.0 + 2.0 ** -10)
    return w


def _ft_expected(tokens, v_rounded):
    d, hc = _FT_D, _FT_HC
    alpha = np.zeros((len(tokens), hc))
    h_out = np.zeros((len(tokens), hc, d))
    for i, t in enumerate(tokens):
        h = _FT_A[t] * np.ones((hc, d))
        r = _FT_TOK_ROW[t]
        if _FT_DEAD[t]:
            h_out[i] = h
            continue
        if r is None:                   # zero e: k = 0 gives s = 0, v = 0 leaves h
            alpha[i] = 0.5
            h_out[i] = h
            continue
        v = 2.0 ** _FT_SH[r] * _FT_V * (1.0 if v_rounded else 1.0 + 2.0 ** -10)
        for m in range(hc):
            a, c = _FT_A[t], _FT_C[m] * 2.0 ** _FT_SH[r]
            s = a * c * (2 * _FT_P[r][m] - d) / (
                math.sqrt(a * a + _FT_EPS) * math.sqrt(c * c + _FT_EPS) * math.sqrt(d))
            alpha[i, m] = 1.0 / (1.0 + math.exp(-math.copysign(math.sqrt(abs(s)), s)))
            h_out[i, m] = h[m] + alpha[i, m] * v
    return alpha, h_out


def _ft_inputs():
    d, hc = _FT_D, _FT_HC
    h = np.array(_FT_A)[:, None, None] * np.ones((len(_FT_A), hc, d))
    ones = np.ones((hc, d))
    return h, ones


def test_forward_tokens_closed_form_bf16():
    """Steps 3-5 composed, on E4M3 rows: kv columns are [k^0 .. k^3 | v] with
    key m going with stream m (P1 "门控": one key per stream, one shared value),
    kv is rounded to bf16 before the gate and the update (P4 "消费":
    h + gate * bf16(v)), DEAD tokens keep h, zero and out-of-range rows give
    e = 0. Tokens are taken out of order to check the per-token indexing."""
    R = 10

    def fetch(rows):
        out = np.zeros((len(rows), 264), dtype=np.uint8)
        out[:, 256:] = 127                                   # scale 2^0
        for i, r in enumerate(np.asarray(rows)):
            if r < len(_FT_POS):
                p = _FT_POS[r]
                out[i, p] = 0x38                             # E4M3 1.0
                out[i, 256 + p // 32] = 127 + _FT_SH[r]
        return out

    tokens = np.array([3, 0, 5, 1, 4, 2])
    h, ones = _ft_inputs()
    res = O.forward_tokens(tokens, _FT_ROWS, _FT_DEAD, fetch_rows=fetch, table_rows=R,
                           wkv=_ft_w(256), q_w=ones, k_w=ones, h=h, hc=_FT_HC, dim=_FT_D,
                           eps=_FT_EPS, clamp=0.0, bf16=True)
    e_exp = np.zeros((len(tokens), 512))
    for i, t in enumerate(tokens):
        r = _FT_TOK_ROW[t]
        if r is not None:
            e_exp[i, _FT_POS[r]] = 2.0 ** _FT_SH[r]
    assert np.array_equal(res["e"], e_exp)
    a_exp, h_exp = _ft_expected(tokens, v_rounded=True)
    np.testing.assert_allclose(res["alpha"], a_exp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["h_out"], h_exp, rtol=0, atol=1e-12)
    assert np.array_equal(res["h_out_bits"], O.round_to_bf16_bits(h_exp))
    # the values here are distinct per stream and per token
    assert len(np.unique(np.round(a_exp[[1, 2, 3, 5]], 9))) >= 6


def test_forward_tokens_closed_form_f32():
    """The fp32 instance keeps kv unrounded: the same construction through fp32
    rows of 256 (C0 keeps fp32 throughout)."""
    R = 10
    table = np.zeros((R, 256), dtype=np.float32)
    for r, p in enumerate(_FT_POS):
        table[r, p] = 2.0 ** _FT_SH[r]
    tokens = np.array([2, 4, 0, 3, 5, 1])
    h, ones = _ft_inputs()
    res = O.forward_tokens(tokens, _FT_ROWS, _FT_DEAD, table_f32=table, table_rows=R,
                           wkv=_ft_w(256), q_w=ones, k_w=ones, h=h, hc=_FT_HC, dim=_FT_D,
                           eps=_FT_EPS, clamp=0.0, bf16=False)
    a_exp, h_exp = _ft_expected(tokens, v_rounded=False)
    np.testing.assert_allclose(res["alpha"], a_exp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["h_out"], h_exp, rtol=0, atol=1e-12)
    assert "h_out_bits" not in res
