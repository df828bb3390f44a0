"""Plain CPU oracle of the Engram layer forward.

TEST INFRASTRUCTURE. Only the tests, the smoke check of ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run this module. The
product path (the HIP library and its Python binding) never does, and this
module imports nothing from it.

It computes, slowly and step by step in the pages' order, what the layer is
defined to compute: floating point in fp64 (numpy), integer work in uint64.
A library primitive (a matmul, a cumulative sum) may serve as a step; nothing
is blocked, fused or reordered beyond the definition.

Pages cited (title, then section / equation / table):

* [P1] "DeepSeek-V4.1 模型结构（5）：记忆，Engram"
* [P2] "Engram条件记忆：DeepSeek-V4.1-Flash中196B稀疏参数N-gram哈希查表的实现原理"
* [P3] "条件记忆：DeepSeek V4.1 Engram 如何用 O(1) 查表换掉一层计算"
* [P4] "ds4.c 学习笔记 · Engram"
* [P5] "DeepSeek Engram 详解：把静态知识从计算里拆出来"

Readings of points the pages leave open (each listed in the design notes):

* primes are taken ascending from the base, the base itself included when
  prime, one per (order, head) segment in order-major, head-minor order, never
  reused (P1 "一层只有一张表" and its prime table; P3 §2.2);
* a DEAD (-1) cell met while looking back blocks that cell and every older one:
  they become the compressed pad id; cells newer than it keep their ids
  (P1 "V4.1 相对原版的两处改动" preamble on image tokens; P2 "多模态细节");
* at a DEAD position all cells are blocked (so the all-pad n-gram's rows are
  looked up) and the gate is forced to zero (P1, P4 "布局与哈希探测" item 4);
* raw ids outside [-1, V) and compressed ids outside [0, V') count as DEAD;
* rows outside [0, R) gather as zero rows (P3 §五, cost side);
* E4M3 is the OCP E4M3FN encoding, E8M0 has bias 127 and 0xFF = NaN;
* gate scale divides the weighted dot of the two RMS-normalised vectors by
  sqrt(d) (P1 "门控" eq. for s^(m)); the RMS has eps inside the root and no
  weight, and the weights q_w * k_w multiply the dot (P4 "消费：学习投影 + 余弦门控");
* kv and h are rounded to bf16 where the device path stores bf16 (P4: the
  residual update is bf16(h + gate * bf16(v)));
* the papers' plain gate sigmoid(s) ignores the clamp (P5 §4.1);
* the short convolution branch (P5 §4.2) gives every channel of every stream
  its own filter and no bias, tap j meets the value (taps - 1 - j) * dilation
  positions back, its RMSNorm runs per stream and position with eps inside the
  root, the convolution input is zero before the sequence start, and a DEAD
  position contributes V~ = 0 and keeps its streams.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence

import numpy as np

DEAD = -1
INT63_MAX = (1 << 63) - 1


# ----------------------------------------------------------------------------
# Setup: prime search, segment offsets, multiplier bound
# ----------------------------------------------------------------------------

def is_prime(n: int) -> bool:
    """Trial division up to floor(sqrt(n))."""
    if n < 2:
        return False
    if n % 2 == 0:
        return n == 2
    f = 3
    while f * f <= n:
        if n % f == 0:
            return False
        f += 2
    return True


def primes_from(base: int, count: int) -> list:
    """The first ``count`` primes >= base, ascending.

    [P1] "一层只有一张表": the code searches upward from engram_vocab_size
    (16,000,000), one prime per head, never reusing one; the page's table gives
    min / max / sum of the 24 primes of each of the two layers.
    """
    out = []
    n = base
    while len(out) < count:
        if is_prime(n):
            out.append(n)
        n += 1
    return out


def segment_offsets(primes: Sequence[int]):
    """Exclusive prefix sums of the segment sizes, and the total row count.

    [P1] "一层只有一张表": the 24 (order, head) tables are contiguous segments
    of one physical table; a head's row id is its local row plus the start of
    its segment, and the table's row count is the sum of the primes.
    """
    offs = [0] * len(primes)
    acc = 0
    for j, p in enumerate(primes):
        offs[j] = acc
        acc += int(p)
    return offs, acc


def layer_primes(base: int, layers: int, per_layer: int):
    """Primes, offsets and row counts of several Engram layers' tables.

    [P1] "一层只有一张表" and its table: the two layers' 24 primes each come
    from one upward search from the base with no prime used twice (layer 1:
    16000057..16000463, sum 384006168; layer 14: 16000477..16000889, sum
    384016682), and each layer has its own physical table whose row count is
    the sum of that layer's primes. [P3] §2.2: primes are drawn in (layer,
    order, head) order from one ascending sequence. Offsets therefore restart
    at 0 in every layer. Returns three lists indexed by layer.
    """
    p = primes_from(base, layers * per_layer)
    primes, offsets, rows = [], [], []
    for li in range(layers):
        seg = p[li * per_layer:(li + 1) * per_layer]
        offs, total = segment_offsets(seg)
        primes.append(seg)
        offsets.append(offs)
        rows.append(total)
    return primes, offsets, rows


def multiplier_limit(compressed_vocab: int) -> int:
    """[P1] §"哈希函数" item "乘子不会让乘积溢出": multipliers stay below
    (2^63 - 1) / V' so that no compressed id times a multiplier leaves int64."""
    return INT63_MAX // compressed_vocab


# ----------------------------------------------------------------------------
# Step 1: tokenizer compression x' = P(x)
# ----------------------------------------------------------------------------

def compress(ids: np.ndarray, token_map: np.ndarray, compressed_vocab: int) -> np.ndarray:
    """x'_t = P(x_t) ([P1] §"tokenizer 压缩", the displayed equation).

    Returns int64 compressed ids; DEAD (-1) positions, raw ids outside [0, V)
    and map values outside [0, V') are returned as -1.
    """
    ids = np.asarray(ids, dtype=np.int64)
    V = token_map.shape[0]
    ok = (ids >= 0) & (ids < V)
    out = np.full(ids.shape, DEAD, dtype=np.int64)
    mapped = token_map.astype(np.int64)[np.where(ok, ids, 0)]
    good = ok & (mapped >= 0) & (mapped < compressed_vocab)
    out[good] = mapped[good]
    return out


# ----------------------------------------------------------------------------
# Step 2: suffix n-gram cells, multiply-XOR mix, modulo per head, offsets
# ----------------------------------------------------------------------------

def ngram_cells(xc: np.ndarray, pad: int, n_cells: int, hist: Optional[np.ndarray] = None):
    """Look-back cells c_i = x'_{t-i}, i = 0..n_cells-1, for every position.

    [P1] §"哈希函数": cells before the start of the sequence hold the pad id
    and are looked up as usual; [P5] §3.2 the demo left-fills with the
    compressed pad id. [P1] image-token paragraph and [P2] "多模态细节": looking
    back stops at a DEAD cell; that cell and every older one count as pad.
    ``hist`` [B, n_cells-1] (oldest first; compressed ids or -1) supplies the
    cells before position 0 of this chunk ([P4] "布局与哈希探测": the hash state is the last 3 tokens).

    Returns cells int64 [B, T, n_cells] and dead [B, T] (position t itself DEAD).
    """
    xc = np.asarray(xc, dtype=np.int64)
    B, T = xc.shape
    H = n_cells - 1
    if hist is None:
        prev = np.full((B, H), pad, dtype=np.int64)
    else:
        prev = np.asarray(hist, dtype=np.int64).reshape(B, H)
    # sequence extended by the history on the left: ext[:, H + t] = xc[:, t]
    ext = np.concatenate([prev, xc], axis=1)
    cells = np.empty((B, T, n_cells), dtype=np.int64)
    blocked = np.zeros((B, T), dtype=bool)
    for i in range(n_cells):
        val = ext[:, H - i: H - i + T]          # x'_{t-i}
        blocked = blocked | (val == DEAD)
        cells[:, :, i] = np.where(blocked, pad, val)
    dead = xc == DEAD
    return cells, dead


def mix_values(cells: np.ndarray, multipliers: Sequence[int], n: int) -> np.ndarray:
    """mix_{t,n} = XOR over i < n of (x'_{t-i} * m_i)  ([P1] eq. (H)).

    Every product stays below 2^63 by the multiplier bound, so uint64 holds it
    exactly.
    """
    out = np.zeros(cells.shape[:-1], dtype=np.uint64)
    for i in range(n):
        prod = cells[..., i].astype(np.uint64) * np.uint64(multipliers[i])
        out ^= prod
    return out


def head_rows(mix: np.ndarray, primes: Sequence[int], offsets: Sequence[int]) -> np.ndarray:
    """z = mix mod p (eq. (H)), then the segment offset ([P1] "一层只有一张表").
    Returns int64 [..., len(primes)]."""
    mix = np.asarray(mix, dtype=np.uint64)
    out = np.empty(mix.shape + (len(primes),), dtype=np.int64)
    for j, (p, off) in enumerate(zip(primes, offsets)):
        out[..., j] = (mix % np.uint64(p)).astype(np.int64) + np.int64(off)
    return out


def hash_rows(ids: np.ndarray, token_map: np.ndarray, compressed_vocab: int, pad: int,
              multipliers: Sequence[int], primes: Sequence[int], offsets: Sequence[int],
              max_ngram: int, heads: int, hist: Optional[np.ndarray] = None):
    """Row ids of every (position, segment) and the history after the chunk.

    Segment j = (n - 2) * heads + k holds order n, head k ([P5] §3.3 concatenation
    order: orders outer, heads inner). Returns row ids int64 [B*T, S] and
    hist_out int32 [B, N-1]: the last N-1 positions' compressed ids (-1 if DEAD),
    oldest first, taking older slots from ``hist`` (or the pad id) when T < N-1.
    History entries outside [0, V') other than -1 count as DEAD.
    """
    ids = np.asarray(ids)
    B, T = ids.shape
    xc = compress(ids, token_map, compressed_vocab)
    H = max_ngram - 1
    if hist is None:
        prev = np.full((B, H), pad, dtype=np.int64)
    else:
        prev = np.asarray(hist, dtype=np.int64).reshape(B, H)
        prev = np.where((prev >= 0) & (prev < compressed_vocab), prev, DEAD)
    cells, _ = ngram_cells(xc, pad, max_ngram, prev)
    S = (max_ngram - 1) * heads
    assert len(primes) == S and len(offsets) == S
    rows = np.empty((B, T, S), dtype=np.int64)
    for n in range(2, max_ngram + 1):
        mix = mix_values(cells, multipliers, n)
        sl = slice((n - 2) * heads, (n - 1) * heads)
        rows[:, :, sl] = head_rows(mix, primes[sl], offsets[sl])
    ext = np.concatenate([prev, xc], axis=1)
    hist_out = ext[:, ext.shape[1] - H:].astype(np.int32)
    return rows.reshape(B * T, S), hist_out


def hash_rows_layers(ids: np.ndarray, token_map: np.ndarray, compressed_vocab: int, pad: int,
                     multipliers: Sequence[Sequence[int]], primes: Sequence[Sequence[int]],
                     offsets: Sequence[Sequence[int]], max_ngram: int, heads: int,
                     hist: Optional[np.ndarray] = None):
    """Row ids of several Engram layers over the same tokens: int64
    [L, B*T, S], layer l addressing its own table, and the shared history.

    [P1] "一层只有一张表": each layer draws its own multipliers and primes, so
    the same n-gram lands on unrelated rows in the two layers. [P3] §2.4: the
    row ids of every Engram layer depend on the token ids only and are all
    computed before the layer loop, then handed to each layer. The cells (and
    so the history) do not depend on the layer.
    """
    out, hist_out = [], None
    for li in range(len(multipliers)):
        rows, h = hash_rows(ids, token_map, compressed_vocab, pad, multipliers[li], primes[li],
                            offsets[li], max_ngram, heads, hist)
        out.append(rows)
        hist_out = h
    return np.stack(out), hist_out


# ----------------------------------------------------------------------------
# Step 3: gather + row-wise dequantisation (E4M3 payload, E8M0 block scales)
# ----------------------------------------------------------------------------

def e4m3fn_value(code: int) -> float:
    """OCP E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
    exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m / 8.0, -6)
    return s * math.ldexp(1.0 + m / 8.0, e - 7)


def e8m0_value(code: int) -> float:
    """E8M0 block scale: 2^(code - 127); 0xFF is NaN."""
    if code == 0xFF:
        return math.nan
    return math.ldexp(1.0, code - 127)


E4M3_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def round_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bfloat16 bit patterns, to nearest, ties to even,
    with subnormals (quantum 2^-133) and overflow to infinity. NaN -> 0x7FC0
    with the input's sign. -0 is kept."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint16) << np.uint16(15)
    a = np.abs(x)
    finite = np.isfinite(a)
    af = np.where(finite, a, 0.0)
    _, e = np.frexp(af)                       # af = m * 2^e, m in [0.5, 1)
    q = np.maximum(e - 1, -126) - 7            # exponent of one unit in the last place
    r = np.rint(np.ldexp(af, -q))             # ties to even
    val = np.ldexp(r, q)                       # exact; >= 2^128 overflows below
    with np.errstate(over="ignore"):
        bits = (val.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isinf(a), np.uint16(0x7F80), bits)
    bits = np.where(np.isnan(a), np.uint16(0x7FC0), bits)
    return (bits | sign).astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def dequant_rows_bf16(row_bytes: np.ndarray) -> np.ndarray:
    """264-byte rows -> 256 bf16 values each.

    [P4] "布局与哈希探测" / "永不常驻的 I/O 设计": 256 E4M3 bytes then 8 E8M0
    bytes, 32 elements share one scale; [P1] "196B 参数怎么存、怎么取": each row
    dequantises on its own; [P3] §2.3: the lookup emits bf16. The value
    E4M3(q) * 2^(s - 127) is exact in fp64, then rounded once to bf16.
    """
    row_bytes = np.asarray(row_bytes, dtype=np.uint8).reshape(-1, 264)
    q = E4M3_TABLE[row_bytes[:, :256]]
    s = E8M0_TABLE[row_bytes[:, 256:264]]
    val = q * np.repeat(s, 32, axis=1)
    return round_to_bf16_bits(val)


def mx_values(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Block-scaled FP8 values: element k of a row is E4M3(code[k]) times
    E8M0(scale[k // 32]), exact in float64.

    [P4] "永不常驻的 I/O 设计": the encoding e4m3_e8m0_32 (32 elements share
    one E8M0 scale); [P3] §2.3: the projection weight is block-FP8 beside the
    table's e4m3 + e8m0 rows. Reading: the weight uses the table's own block
    encoding, one scale per 32 consecutive inputs of an output row.
    codes uint8 [..., K], scales uint8 [..., K/32].
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    assert codes.shape[-1] == 32 * scales.shape[-1]
    return E4M3_TABLE[codes] * np.repeat(E8M0_TABLE[scales], 32, axis=-1)


def gather_rows(fetch_rows: Callable[[np.ndarray], np.ndarray], row_ids: np.ndarray,
                table_rows: int) -> np.ndarray:
    """The looked-up rows themselves, bytes unchanged: uint8 [T, S, 264], all
    zeros for ids outside [0, R) ([P3] §五: such rows output zero rows)."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    T, S = row_ids.shape
    flat = row_ids.reshape(-1)
    ok = (flat >= 0) & (flat < table_rows)
    out = np.zeros((flat.size, 264), dtype=np.uint8)
    if ok.any():
        out[ok] = fetch_rows(flat[ok])
    return out.reshape(T, S, 264)


def gather_e4m3(fetch_rows: Callable[[np.ndarray], np.ndarray], row_ids: np.ndarray,
                table_rows: int) -> np.ndarray:
    """e[t, j*256:(j+1)*256] = dequant(table[row_ids[t, j]]), zeros outside [0, R)
    ([P3] §五: out-of-range and non-local rows output zero rows).

    ``fetch_rows(r)`` returns the 264-byte rows r (uint8 [n, 264]).
    Returns bf16 bits uint16 [T, S*256].
    """
    row_ids = np.asarray(row_ids, dtype=np.int64)
    T, S = row_ids.shape
    flat = row_ids.reshape(-1)
    ok = (flat >= 0) & (flat < table_rows)
    out = np.zeros((flat.size, 256), dtype=np.uint16)
    if ok.any():
        out[ok] = dequant_rows_bf16(fetch_rows(flat[ok]))
    return out.reshape(T, S * 256)


def gather_f32(table: np.ndarray, row_ids: np.ndarray) -> np.ndarray:
    """fp32 rows copied verbatim; zeros outside [0, R)."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    T, S = row_ids.shape
    R, D = table.shape
    flat = row_ids.reshape(-1)
    ok = (flat >= 0) & (flat < R)
    out = np.zeros((flat.size, D), dtype=np.float32)
    out[ok] = table[flat[ok]]
    return out.reshape(T, S * D)


# ----------------------------------------------------------------------------
# Step 4: the fused key/value projection
# ----------------------------------------------------------------------------

def project(e: np.ndarray, wkv: np.ndarray) -> np.ndarray:
    """kv = e W, W = wkv^T: one matmul producing hc keys and one value.

    [P1] "每条流一个 key 的设计沿用自原版": the key and value projections are
    one matrix wkv of shape 6144 x 25600; [P4] "消费": the weight is stored
    [24*256, 5*5120] with the 6144 input dimension innermost, i.e. one row of
    6144 inputs per output column. ``wkv`` is that [(hc+1)*d, S*row_dim] array.
    Returns kv in float64, columns [k^(0) .. k^(hc-1) | v].
    """
    return np.asarray(e, dtype=np.float64) @ np.asarray(wkv, dtype=np.float64).T


# ----------------------------------------------------------------------------
# Step 5: context gate and residual update
# ----------------------------------------------------------------------------

def gate(h: np.ndarray, k: np.ndarray, v: np.ndarray, q_w: np.ndarray, k_w: np.ndarray,
         dead: np.ndarray, eps: float, clamp: float = 0.0, mode: str = "signed_sqrt"):
    """Gate alpha [T, hc] and updated streams h + alpha * v, in float64.

    [P1] "门控" and "sigmoid 之前多一步带符号的平方根":
      s = RMSNorm(h^(m)) . RMSNorm(k^(m)) / sqrt(d),
      alpha = sigmoid(sign(s) * sqrt(max(|s|, clamp))),  h^(m) += alpha * v;
    [P4] "消费": the learned element-wise scales q_w and k_w of stream m
    multiply the dot, and eps sits inside each reciprocal root of mean squares.
    [P1] image-token paragraph: the gate at a DEAD position is 0, and [P4]
    item 4: such rows are returned untouched.
    mode "plain" is the papers' own gate alpha = sigmoid(s) ([P5] §4.1, the
    equation for alpha_t; [P1] "sigmoid 之前多一步带符号的平方根" names it as the
    formula the signed root departs from); clamp does not enter it.

    h, k: [T, hc, d]; v: [T, d]; q_w, k_w: [hc, d]; dead: [T] bool.
    """
    if mode not in ("signed_sqrt", "plain"):
        raise ValueError(f"unknown gate mode {mode!r}")
    h = np.asarray(h, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = h.shape[-1]
    w = np.asarray(q_w, dtype=np.float64) * np.asarray(k_w, dtype=np.float64)
    rh = 1.0 / np.sqrt(np.mean(h * h, axis=-1) + eps)
    rk = 1.0 / np.sqrt(np.mean(k * k, axis=-1) + eps)
    dot = np.sum(h * w[None, :, :] * k, axis=-1)
    s = dot * rh * rk / math.sqrt(d)
    if mode == "plain":
        z = s
    else:
        z = np.copysign(np.sqrt(np.maximum(np.abs(s), clamp)), s)
    alpha = 1.0 / (1.0 + np.exp(-z))
    alpha = np.where(np.asarray(dead)[:, None], 0.0, alpha)
    h_out = h + alpha[:, :, None] * v[:, None, :]
    h_out = np.where(np.asarray(dead)[:, None, None], h, h_out)
    return alpha, h_out


# ----------------------------------------------------------------------------
# Short convolution branch after the gate (the papers' variant)
# ----------------------------------------------------------------------------

def conv_history_len(taps: int, dilation: int) -> int:
    """Positions before the current one that a causal convolution of ``taps``
    taps spaced ``dilation`` apart reaches: (taps - 1) * dilation, 9 for the
    papers' 4 taps at dilation 3 ([P5] §4.2: position t uses t, t-3, t-6, t-9;
    [P5] §9.5: a decode state covering the past 9 positions)."""
    if taps < 1 or dilation < 1:
        raise ValueError("taps and dilation must be >= 1")
    return (taps - 1) * dilation


def rms_norm(x: np.ndarray, weight: Optional[np.ndarray], eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis, times ``weight`` (ones if
    None). Reading: the branch's RMSNorm normalises each stream's d channels at
    one position, like the gate's, with eps inside the root."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    return y


def short_conv(vt: np.ndarray, conv_w: np.ndarray, norm_w: Optional[np.ndarray],
               dilation: int, eps: float, hist: Optional[np.ndarray] = None) -> np.ndarray:
    """Y = SiLU(Conv1D(RMSNorm(V~))) + V~ over each sequence, in float64.

    [P5] §4.2, the equation for Y: a short depthwise causal convolution of the
    RMS-normalised gated values, SiLU, plus the gated values themselves; kernel
    size 4 and dilation equal to the largest n-gram order (3) in the papers'
    setting, one filter per channel. [P3] §三 states the same branch as
    value + short_conv(value). Readings: every channel of every stream has its
    own filter and no bias; tap j of a filter multiplies the value
    (taps - 1 - j) * dilation positions back (the causal Conv1D whose last tap
    meets the current position); before the sequence start, or before
    ``hist``, the normalised input is zero.

    vt: [B, T, hc, d] gated values alpha v (zero at DEAD positions);
    conv_w: [hc, d, taps]; norm_w: [hc, d] or None;
    hist: [B, L, hc, d] gated values of the L = (taps - 1) * dilation positions
    before the chunk, or None for a sequence start.
    """
    vt = np.asarray(vt, dtype=np.float64)
    B, T, hc, d = vt.shape
    w = np.asarray(conv_w, dtype=np.float64)
    taps = w.shape[-1]
    L = conv_history_len(taps, dilation)
    # the causal convolution pads its (normalised) input with zeros
    n_prev = np.zeros((B, L, hc, d)) if hist is None else \
        rms_norm(np.asarray(hist, dtype=np.float64).reshape(B, L, hc, d), norm_w, eps)
    n = np.concatenate([n_prev, rms_norm(vt, norm_w, eps)], axis=1)
    u = np.zeros_like(vt)
    for j in range(taps):
        back = (taps - 1 - j) * dilation
        u += w[None, None, :, :, j] * n[:, L - back:L - back + T]
    silu = u / (1.0 + np.exp(-u))
    return silu + vt


def gate_conv(h: np.ndarray, k: np.ndarray, v: np.ndarray, q_w: np.ndarray, k_w: np.ndarray,
              dead: np.ndarray, eps: float, clamp: float, conv_w: np.ndarray,
              norm_w: Optional[np.ndarray], dilation: int, conv_eps: float,
              hist: Optional[np.ndarray] = None, mode: str = "signed_sqrt"):
    """The gate followed by the short convolution branch, in float64.

    [P5] §4.1-§4.2: V~ = alpha v per stream, Y = SiLU(Conv1D(RMSNorm(V~))) + V~,
    H += Y. At a DEAD position alpha = 0, so V~ = 0 there as the neighbours'
    convolution sees it, and that position's streams are left untouched, as
    without the branch (reading: [P1]'s forced-zero gate and [P4] item 4 carry
    over to the whole update).

    h, k: [B, T, hc, d]; v: [B, T, d]; dead: [B, T] bool; hist as short_conv.
    Returns alpha [B, T, hc], h_out [B, T, hc, d] and the gated values of the
    last L positions of hist followed by this chunk (the next chunk's hist).
    """
    h = np.asarray(h, dtype=np.float64)
    B, T, hc, d = h.shape
    alpha, _ = gate(h.reshape(B * T, hc, d), np.asarray(k).reshape(B * T, hc, d),
                    np.asarray(v).reshape(B * T, d), q_w, k_w,
                    np.asarray(dead).reshape(B * T), eps, clamp, mode=mode)
    alpha = alpha.reshape(B, T, hc)
    vt = alpha[..., None] * np.asarray(v, dtype=np.float64)[:, :, None, :]
    y = short_conv(vt, conv_w, norm_w, dilation, conv_eps, hist)
    dead = np.asarray(dead).reshape(B, T)
    h_out = np.where(dead[:, :, None, None], h, h + y)
    L = conv_history_len(np.asarray(conv_w).shape[-1], dilation)
    prev = np.zeros((B, L, hc, d)) if hist is None else np.asarray(hist, dtype=np.float64)
    tail = np.concatenate([prev, vt], axis=1)[:, T:]
    return alpha, h_out, tail


# ----------------------------------------------------------------------------
# The whole layer on a subset of positions
# ----------------------------------------------------------------------------

def forward_tokens(tokens: np.ndarray, row_ids: np.ndarray, dead: np.ndarray, *,
                   fetch_rows=None, table_f32=None, table_rows: int,
                   wkv: np.ndarray, q_w: np.ndarray, k_w: np.ndarray, h: np.ndarray,
                   hc: int, dim: int, eps: float, clamp: float, bf16: bool):
    """Steps 3-5 for the flat token indices ``tokens``.

    row_ids: [B*T, S] from ``hash_rows``; dead: [B*T] bool; h: [B*T, hc, d]
    (float64 values; bf16 workloads pass the decoded bf16 values).
    bf16 workloads round e (exact), kv and the output to bf16 as the device
    path stores them; the fp32 workload keeps float64 throughout.

    Returns dict with e, kv, alpha [n, hc], h_out [n, hc, d] (float64),
    kv_exact (the product before any rounding, [n, (hc+1)*d]) and, for bf16
    workloads, h_out_bits (uint16).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    rid = row_ids[tokens]
    if bf16:
        e = bf16_bits_to_f64(gather_e4m3(fetch_rows, rid, table_rows))
    else:
        e = gather_f32(table_f32, rid).astype(np.float64)
    kv_exact = project(e, wkv)
    kv = bf16_bits_to_f64(round_to_bf16_bits(kv_exact)) if bf16 else kv_exact
    kv = kv.reshape(len(tokens), hc + 1, dim)
    alpha, h_out = gate(h[tokens], kv[:, :hc, :], kv[:, hc, :], q_w, k_w, dead[tokens],
                        eps, clamp)
    out = {"e": e, "kv": kv, "kv_exact": kv_exact, "alpha": alpha, "h_out": h_out}
    if bf16:
        out["h_out_bits"] = round_to_bf16_bits(h_out)
    return out
