"""Seeded synthetic input generators for the Engram workloads.

Both the HIP path and the oracle take their inputs from here; this module holds
none of the layer's arithmetic (no hashing, no modulo, no dequantisation, no
projection, no gate). Random numbers that the method itself draws -- the token
compression map and the odd hash multipliers -- are drawn here and passed to
both sides as inputs.

Streams: every tensor has its own numpy ``SeedSequence(seed).spawn`` child, so
adding a tensor never changes the values of another. Large dense tensors are
filled chunk by chunk, each chunk from its own grandchild stream, so the result
does not depend on how many threads fill it.

The byte table is a pure counter-based function of (seed, row, byte), so any
row of a 101 GB table can be regenerated on the host without storing the table.
Each byte comes from SplitMix64 (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014): the state after ``c`` steps from
``seed`` is ``seed + c * 0x9E3779B97F4A7C15``, finalised by ``mix64``; the
counter of byte ``b`` of row ``r`` is ``c = r * 264 + b + 1``. The device twin
lives in ``workloads/csrc/table_gen.hip``.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .configs import EngramWorkload, ROW_F32

ROW_BYTES = 264           # 256 E4M3 payload bytes + 8 E8M0 scale bytes
PAYLOAD_BYTES = 256
SCALE_BYTES = 8
GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Payload codes exclude the two E4M3FN NaN encodings 0x7F and 0xFF: a uniform
# draw u in [0, 254) maps to u (0x00..0x7E) or u + 1 (0x80..0xFE).
PAYLOAD_CHOICES = 254
# E8M0 scale bytes are 120 + u, u uniform in [0, 15): exponents 120..134.
SCALE_BASE = 120
SCALE_CHOICES = 15

# child stream index of each tensor
S_TOKEN_MAP, S_MULT, S_ZIPF_PERM, S_IDS, S_DEAD, S_TABLE_F32, S_WKV, S_QW, S_KW, \
    S_H, S_HIST, S_MULT_LAYERS, S_WKV_MX = range(13)

_CHUNK = 1 << 22


def _streams(seed: int, n: int = 16):
    return np.random.SeedSequence(seed).spawn(n)


def _rng(seed: int, idx: int) -> np.random.Generator:
    return np.random.default_rng(_streams(seed)[idx])


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on uint64 arrays (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def table_rows(seed: int, rows) -> np.ndarray:
    """Bytes of the given rows of the counter-based E4M3+E8M0 table, uint8 [n, 264]."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    b = np.arange(ROW_BYTES, dtype=np.uint64)
    ctr = rows.astype(np.uint64)[:, None] * np.uint64(ROW_BYTES) + b[None, :] + np.uint64(1)
    with np.errstate(over="ignore"):
        z = mix64(np.uint64(seed) + ctr * GOLDEN_GAMMA)
    hi = z >> np.uint64(32)
    out = np.empty(z.shape, dtype=np.uint8)
    with np.errstate(over="ignore"):
        u = (hi[:, :PAYLOAD_BYTES] * np.uint64(PAYLOAD_CHOICES)) >> np.uint64(32)
        out[:, :PAYLOAD_BYTES] = (u + (u >= np.uint64(127)).astype(np.uint64)).astype(np.uint8)
        s = (hi[:, PAYLOAD_BYTES:] * np.uint64(SCALE_CHOICES)) >> np.uint64(32)
        out[:, PAYLOAD_BYTES:] = (s + np.uint64(SCALE_BASE)).astype(np.uint8)
    return out


def token_map(raw_vocab: int, compressed_vocab: int, rng: np.random.Generator) -> np.ndarray:
    """Seeded random surjection [0, V) -> [0, V').

    Stands in for the normalisation-based tokenizer compression, which needs the
    real vocabulary. The first V' entries of a seeded shuffle map one-to-one onto
    0..V'-1, the rest map to uniform draws, so every compressed id is hit.
    """
    assert 0 < compressed_vocab <= raw_vocab
    perm = rng.permutation(raw_vocab)
    m = np.empty(raw_vocab, dtype=np.int32)
    m[perm[:compressed_vocab]] = np.arange(compressed_vocab, dtype=np.int32)
    m[perm[compressed_vocab:]] = rng.integers(0, compressed_vocab,
                                              raw_vocab - compressed_vocab, dtype=np.int32)
    return m


def multiplier_bound(compressed_vocab: int) -> int:
    """Largest multiplier allowed for V' compressed ids: floor((2^63 - 1) / V')."""
    return ((1 << 63) - 1) // compressed_vocab


def multipliers(compressed_vocab: int, count: int, rng: np.random.Generator) -> list:
    """``count`` seeded odd values in [1, floor((2^63-1)/V')]."""
    bound = multiplier_bound(compressed_vocab)
    half = (bound + 1) // 2                 # odd values 2k+1 <= bound, k < half
    ks = [int(rng.integers(0, half)) for _ in range(count)]
    return [2 * k + 1 for k in ks]


def zipf_ranks(raw_vocab: int, s: float, n: int, rng: np.random.Generator) -> np.ndarray:
    """n draws of a finite Zipf(s) rank r in [1, V], P(r) proportional to r^-s."""
    w = np.arange(1, raw_vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), raw_vocab - 1) + 1


def dead_spans(seq: int, count: int, length: int, rng: np.random.Generator):
    """``count`` non-overlapping [start, start+length) spans, rejection-sampled."""
    if count == 0:
        return []
    assert count * length <= seq
    while True:
        starts = np.sort(rng.integers(0, seq - length + 1, count))
        if np.all(np.diff(starts) >= length):
            return [(int(a), int(a) + length) for a in starts]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 draws to bfloat16 bit patterns (nearest, ties to even)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill_normal(shape, mean: float, std: float, seed_seq, as_bf16: bool,
                 threads: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if as_bf16 else np.float32)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = seed_seq.spawn(nchunks)

    def work(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.default_rng(kids[i])
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        out[lo:hi] = f32_to_bf16_bits(v) if as_bf16 else v

    threads = threads or min(16, os.cpu_count() or 1)
    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def hash_setup(w: EngramWorkload):
    """Token map, compressed pad id and multipliers of a workload's hash setup."""
    tm = token_map(w.raw_vocab, w.compressed_vocab, _rng(w.setup_seed, S_TOKEN_MAP))
    mult = multipliers(w.compressed_vocab, w.max_ngram, _rng(w.setup_seed, S_MULT))
    return tm, mult


def layer_multipliers(w: EngramWorkload, layers: int) -> list:
    """Multipliers of ``layers`` Engram layers sharing this hash setup: layer 0
    keeps ``hash_setup``'s, later layers draw their own from a separate stream."""
    _, first = hash_setup(w)
    rng = _rng(w.setup_seed, S_MULT_LAYERS)
    return [first] + [multipliers(w.compressed_vocab, w.max_ngram, rng) for _ in range(layers - 1)]


_E4M3_POS = None


def _e4m3_positive_grid():
    """The 126 positive finite E4M3FN values (codes 0x01..0x7E), ascending."""
    global _E4M3_POS
    if _E4M3_POS is None:
        vals = []
        for c in range(1, 0x7F):
            e, m = (c >> 3) & 15, c & 7
            vals.append(2.0 ** -6 * m / 8 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8))
        _E4M3_POS = np.array(vals, dtype=np.float64)
    return _E4M3_POS


def quantize_mx_e4m3(x: np.ndarray):
    """OCP MX quantisation of float rows [..., K] (K % 32 == 0) to E4M3 codes and
    one E8M0 scale per 32 values: shared exponent floor(log2(amax)) - 8 (8 being
    E4M3's largest exponent), each value divided by it and rounded to the
    nearest E4M3 value, ties to the even code, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        se = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
    se = np.clip(se, -127, 127)
    q = np.abs(blocks) / np.exp2(se)[..., None]
    grid = _e4m3_positive_grid()
    hi = np.clip(np.searchsorted(grid, q), 0, grid.size - 1)
    lo = np.clip(hi - 1, 0, grid.size - 1)
    dlo, dhi = q - grid[lo], grid[hi] - q
    code_lo, code_hi = lo + 1, hi + 1
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (code_hi % 2 == 0))
    code = np.where(pick_hi, code_hi, code_lo)
    code = np.where(q < grid[0] / 2, 0, code)                    # rounds to zero
    code = np.where(q > grid[-1], grid.size, code)               # saturate at 448
    code = code | (np.signbit(blocks).astype(np.int64) << 7)
    codes = code.astype(np.uint8).reshape(x.shape)
    scales = (se + 127).astype(np.uint8)
    return codes, scales


def wkv_mx(w: EngramWorkload):
    """The projection weight in block-scaled FP8: N(0, 0.02) values of shape
    [(hc+1) d, S * row_dim] quantised by ``quantize_mx_e4m3`` (codes, scales)."""
    n, k = (w.hc + 1) * w.dim, w.segments * w.row_dim
    codes = np.empty((n, k), dtype=np.uint8)
    scales = np.empty((n, k // 32), dtype=np.uint8)
    kids = np.random.SeedSequence(w.seed).spawn(16)[S_WKV_MX].spawn((n + 1023) // 1024)

    def work(i):
        a, b = i * 1024, min(n, (i + 1) * 1024)
        x = np.random.default_rng(kids[i]).normal(0.0, 0.02, (b - a, k))
        codes[a:b], scales[a:b] = quantize_mx_e4m3(x)

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(work, range(len(kids))))
    return codes, scales


def token_ids(w: EngramWorkload):
    """Raw Zipf ids [B, T] (int32) with -1 at DEAD positions, and the spans."""
    perm = _rng(w.setup_seed, S_ZIPF_PERM).permutation(w.raw_vocab)
    ranks = zipf_ranks(w.raw_vocab, w.zipf_s, w.tokens, _rng(w.seed, S_IDS))
    ids = perm[ranks - 1].astype(np.int32).reshape(w.batch, w.seq)
    spans = []
    rng = _rng(w.seed, S_DEAD)
    for b in range(w.batch):
        sp = list(w.dead_fixed)
        if w.dead_random[0]:
            sp += dead_spans(w.seq, w.dead_random[0], w.dead_random[1], rng)
        for a, e in sp:
            ids[b, a:e] = -1
        spans.append(sp)
    if w.dead_sequence0:
        ids[0, :] = -1
    return ids, spans


def history(w: EngramWorkload, tmap: np.ndarray) -> np.ndarray:
    """Decode history [B, N-1] of compressed ids, oldest first; sequence 0 DEAD."""
    perm = _rng(w.setup_seed, S_ZIPF_PERM).permutation(w.raw_vocab)
    ranks = zipf_ranks(w.raw_vocab, w.zipf_s, w.batch * (w.max_ngram - 1),
                       _rng(w.seed, S_HIST))
    raw = perm[ranks - 1].reshape(w.batch, w.max_ngram - 1)
    hist = tmap[raw].astype(np.int32)
    if w.dead_sequence0:
        hist[0, :] = -1
    return hist


def dense_inputs(w: EngramWorkload, table_rows_f32: int = 0):
    """wkv [(hc+1)*d, S*row_dim], q_w / k_w [hc, d], h [B, T, hc, d].

    bf16 workloads return uint16 bf16 bit patterns; the fp32 workload (C0)
    returns float32 arrays, plus its fp32 table [rows, row_dim] ~ N(0, 1).
    """
    ss = _streams(w.seed)
    bf = w.row_format != ROW_F32
    out = {
        "wkv": _fill_normal((w.kv_cols, w.mem_dim), 0.0, 0.02, ss[S_WKV], bf),
        "q_w": _fill_normal((w.hc, w.dim), 1.0, 0.1, ss[S_QW], False),
        "k_w": _fill_normal((w.hc, w.dim), 1.0, 0.1, ss[S_KW], False),
        "h": _fill_normal((w.batch, w.seq, w.hc, w.dim), 0.0, 1.0, ss[S_H], bf),
    }
    if not bf:
        out["table"] = _fill_normal((table_rows_f32, w.row_dim), 0.0, 1.0,
                                    ss[S_TABLE_F32], False)
    return out
