"""Plausible mistakes planted in the oracle (on the CPU, in this process only)
must each make at least one pin fail: evidence that the pins constrain every
step of the oracle, not just its happy path."""
import math

import numpy as np
import pytest

import oracle.engram_oracle as E
import tests.test_oracle_pins as P


def _mix_oldest_first(cells, multipliers, n):
    out = np.zeros(cells.shape[:-1], dtype=np.uint64)
    for i in range(n):
        out ^= cells[..., i].astype(np.uint64) * np.uint64(multipliers[n - 1 - i])
    return out


def _mix_add(cells, multipliers, n):
    out = np.zeros(cells.shape[:-1], dtype=np.uint64)
    for i in range(n):
        out += cells[..., i].astype(np.uint64) * np.uint64(multipliers[i])
    return out


def _offsets_inclusive(primes):
    offs, acc = [], 0
    for p in primes:
        acc += int(p)
        offs.append(acc)
    return offs, acc


def _primes_strictly_above(base, count):
    out, n = [], base + 1
    while len(out) < count:
        if E.is_prime(n):
            out.append(n)
        n += 1
    return out


def _cells_block_newer(xc, pad, n_cells, hist=None):
    """Wrong cascade: a DEAD cell in the window also blanks the newer cells."""
    cells, dead = _orig["ngram_cells"](xc, pad, n_cells, hist)
    xc = np.asarray(xc, dtype=np.int64)
    for t in range(1, xc.shape[1]):
        older_dead = (xc[:, max(0, t - n_cells + 1):t] == E.DEAD).any(axis=1)
        cells[older_dead, t, :] = pad
    return cells, dead


def _cells_no_pad_history(xc, pad, n_cells, hist=None):
    cells, dead = _orig["ngram_cells"](xc, pad, n_cells, hist)
    cells[:, 0, 1:] = 0
    return cells, dead


def _e8m0_bias128(code):
    return math.nan if code == 0xFF else math.ldexp(1.0, code - 128)


def _round_truncate(x):
    x = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _gate_over_d(h, k, v, q_w, k_w, dead, eps, clamp=0.0, mode="signed_sqrt"):
    d = h.shape[-1]
    return _orig["gate"](h, k, v, q_w, k_w, dead, eps, clamp, mode) if d == 1 else \
        _orig["gate"](np.asarray(h) / math.sqrt(d), k, v, q_w, k_w, dead, eps, clamp, mode)


def _gate_plain_sigmoid(h, k, v, q_w, k_w, dead, eps, clamp=0.0, mode="signed_sqrt"):
    h = np.asarray(h, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = h.shape[-1]
    w = np.asarray(q_w) * np.asarray(k_w)
    rh = 1 / np.sqrt(np.mean(h * h, -1) + eps)
    rk = 1 / np.sqrt(np.mean(k * k, -1) + eps)
    s = np.sum(h * w[None] * k, -1) * rh * rk / math.sqrt(d)
    a = 1 / (1 + np.exp(-s))
    a = np.where(np.asarray(dead)[:, None], 0.0, a)
    return a, h + a[:, :, None] * np.asarray(v)[:, None, :]


def _gate_no_weights(h, k, v, q_w, k_w, dead, eps, clamp=0.0, mode="signed_sqrt"):
    return _orig["gate"](h, k, v, np.ones_like(q_w), np.ones_like(k_w), dead, eps, clamp, mode)


def _gate_mode_ignored(h, k, v, q_w, k_w, dead, eps, clamp=0.0, mode="signed_sqrt"):
    return _orig["gate"](h, k, v, q_w, k_w, dead, eps, clamp)


def _short_conv_taps_reversed(vt, conv_w, norm_w, dilation, eps, hist=None):
    return _orig["short_conv"](vt, np.asarray(conv_w)[..., ::-1], norm_w, dilation, eps, hist)


def _short_conv_no_dilation(vt, conv_w, norm_w, dilation, eps, hist=None):
    return _orig["short_conv"](vt, conv_w, norm_w, 1, eps, None)


def _short_conv_no_residual(vt, conv_w, norm_w, dilation, eps, hist=None):
    return _orig["short_conv"](vt, conv_w, norm_w, dilation, eps, hist) - np.asarray(vt)


def _short_conv_sigmoid(vt, conv_w, norm_w, dilation, eps, hist=None):
    """Wrong: sigmoid(u) where SiLU(u) = u sigmoid(u) belongs."""
    y = _orig["short_conv"](vt, conv_w, norm_w, dilation, eps, hist) - np.asarray(vt)
    # invert SiLU numerically is awkward; rebuild u from the definition instead
    vt = np.asarray(vt, dtype=np.float64)
    w = np.asarray(conv_w, dtype=np.float64)
    taps, L = w.shape[-1], (w.shape[-1] - 1) * dilation
    B, T, hc, d = vt.shape
    n_prev = np.zeros((B, L, hc, d)) if hist is None else E.rms_norm(hist, norm_w, eps)
    n = np.concatenate([n_prev, E.rms_norm(vt, norm_w, eps)], axis=1)
    u = sum(w[None, None, :, :, j] * n[:, L - (taps - 1 - j) * dilation:][:, :T]
            for j in range(taps))
    return 1 / (1 + np.exp(-u)) + vt


def _rms_norm_eps_outside(x, weight, eps):
    x = np.asarray(x, dtype=np.float64)
    y = x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)
    return y if weight is None else y * weight


def _rms_norm_over_streams(x, weight, eps):
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=(-2, -1), keepdims=True) + eps)
    return y if weight is None else y * weight


def _gate_conv_updates_dead(h, k, v, q_w, k_w, dead, eps, clamp, conv_w, norm_w, dilation,
                            conv_eps, hist=None, mode="signed_sqrt"):
    a, _, tail = _orig["gate_conv"](h, k, v, q_w, k_w, dead, eps, clamp, conv_w, norm_w,
                                    dilation, conv_eps, hist, mode)
    vt = a[..., None] * np.asarray(v)[:, :, None, :]
    return a, np.asarray(h) + E.short_conv(vt, conv_w, norm_w, dilation, conv_eps, hist), tail


def _gate_conv_tail_ignores_hist(h, k, v, q_w, k_w, dead, eps, clamp, conv_w, norm_w, dilation,
                                 conv_eps, hist=None, mode="signed_sqrt"):
    a, ho, tail = _orig["gate_conv"](h, k, v, q_w, k_w, dead, eps, clamp, conv_w, norm_w,
                                     dilation, conv_eps, hist, mode)
    T = np.asarray(h).shape[1]
    if T < tail.shape[1]:
        tail = tail.copy()
        tail[:, :tail.shape[1] - T] = 0.0
    return a, ho, tail


def _project_transposed(e, wkv):
    w = np.asarray(wkv, dtype=np.float64)
    if w.shape[0] == w.shape[1]:
        return np.asarray(e, dtype=np.float64) @ w
    return np.asarray(e, dtype=np.float64) @ w.T[::-1]


def _mx_block16(codes, scales):
    """Wrong: one scale per 16 elements, the first half of the scales reused."""
    codes = np.asarray(codes, dtype=np.uint8)
    sc = np.asarray(scales, dtype=np.uint8)
    per16 = np.repeat(E.E8M0_TABLE[sc], 16, axis=-1)
    return E.E4M3_TABLE[codes] * np.concatenate([per16, per16], axis=-1)[..., :codes.shape[-1]]


def _layer_offsets_continue(base, layers, per_layer):
    """Wrong: one offset sequence over all layers instead of one table per layer."""
    p = E.primes_from(base, layers * per_layer)
    offs, _ = E.segment_offsets(p)
    primes = [p[i * per_layer:(i + 1) * per_layer] for i in range(layers)]
    offsets = [offs[i * per_layer:(i + 1) * per_layer] for i in range(layers)]
    return primes, offsets, [sum(x) for x in primes]


def _layer_primes_restart(base, layers, per_layer):
    """Wrong: every layer restarts the prime search at the base."""
    p = E.primes_from(base, per_layer)
    offs, total = E.segment_offsets(p)
    return [list(p)] * layers, [list(offs)] * layers, [total] * layers


def _layers_share_multipliers(ids, token_map, compressed_vocab, pad, multipliers, primes, offsets,
                              max_ngram, heads, hist=None):
    """Wrong: the first layer's multipliers serve every layer."""
    return _orig["hash_rows_layers"](ids, token_map, compressed_vocab, pad,
                                     [multipliers[0]] * len(multipliers), primes, offsets,
                                     max_ngram, heads, hist)


def _compress_skips_map(ids, token_map, compressed_vocab):
    """Wrong: the raw id is used as the compressed id."""
    ids = np.asarray(ids, dtype=np.int64)
    ok = (ids >= 0) & (ids < token_map.shape[0])
    return np.where(ok, ids, E.DEAD)


def _compress_no_value_check(ids, token_map, compressed_vocab):
    """Wrong: map values outside [0, V') pass through."""
    ids = np.asarray(ids, dtype=np.int64)
    ok = (ids >= 0) & (ids < token_map.shape[0])
    return np.where(ok, token_map.astype(np.int64)[np.where(ok, ids, 0)], E.DEAD)


def _forward_tokens_variant(v_col=None, round_kv=None, reverse_keys=False, dead_by_position=False):
    """forward_tokens with one planted mistake: v taken from block ``v_col``,
    kv rounding forced on/off (``round_kv``), keys in reverse stream order, or
    the DEAD flags taken by position instead of by token index."""
    def f(tokens, row_ids, dead, *, fetch_rows=None, table_f32=None, table_rows, wkv, q_w,
          k_w, h, hc, dim, eps, clamp, bf16):
        tokens = np.asarray(tokens, dtype=np.int64)
        rid = row_ids[tokens]
        if bf16:
            e = E.bf16_bits_to_f64(E.gather_e4m3(fetch_rows, rid, table_rows))
        else:
            e = E.gather_f32(table_f32, rid).astype(np.float64)
        kv = E.project(e, wkv)
        if (bf16 if round_kv is None else round_kv):
            kv = E.bf16_bits_to_f64(E.round_to_bf16_bits(kv))
        kv = kv.reshape(len(tokens), hc + 1, dim)
        keys = kv[:, :hc, :][:, ::-1] if reverse_keys else kv[:, :hc, :]
        v = kv[:, hc if v_col is None else v_col, :]
        dd = np.asarray(dead)[:len(tokens)] if dead_by_position else np.asarray(dead)[tokens]
        alpha, h_out = E.gate(h[tokens], keys, v, q_w, k_w, dd, eps, clamp)
        out = {"e": e, "kv": kv, "alpha": alpha, "h_out": h_out}
        if bf16:
            out["h_out_bits"] = E.round_to_bf16_bits(h_out)
        return out
    f.__name__ = "_forward_tokens_" + ("v_from_key0" if v_col is not None else
                                       "kv_unrounded" if round_kv is False else
                                       "kv_always_rounded" if round_kv else
                                       "keys_reversed" if reverse_keys else "dead_by_position")
    return f


_orig = {name: getattr(E, name) for name in
         ("mix_values", "segment_offsets", "primes_from", "ngram_cells", "gate", "project",
          "round_to_bf16_bits", "layer_primes", "hash_rows_layers", "mx_values", "short_conv",
          "rms_norm", "gate_conv", "compress", "forward_tokens")}

_FT_PINS = [P.test_forward_tokens_closed_form_bf16, P.test_forward_tokens_closed_form_f32]

MUTATIONS = [
    ("compress", _compress_skips_map, [P.test_compress_hand_built_map]),
    ("compress", _compress_no_value_check, [P.test_compress_hand_built_map]),
    ("forward_tokens", _forward_tokens_variant(v_col=0), _FT_PINS),
    ("forward_tokens", _forward_tokens_variant(round_kv=False), _FT_PINS),
    ("forward_tokens", _forward_tokens_variant(round_kv=True), _FT_PINS),
    ("forward_tokens", _forward_tokens_variant(reverse_keys=True), _FT_PINS),
    ("forward_tokens", _forward_tokens_variant(dead_by_position=True), _FT_PINS),
    ("mix_values", _mix_oldest_first, [P.test_worked_example_mix_and_indices]),
    ("mix_values", _mix_add, [P.test_worked_example_mix_and_indices]),
    ("segment_offsets", _offsets_inclusive, [P.test_worked_example_through_single_table]),
    ("primes_from", _primes_strictly_above, [P.test_primes_against_sympy]),
    ("ngram_cells", _cells_block_newer, [P.test_pad_and_dead_cells_c0]),
    ("ngram_cells", _cells_no_pad_history, [P.test_pad_and_dead_cells_c0]),
    ("round_to_bf16_bits", _round_truncate, [P.test_round_to_bf16_against_torch]),
    ("gate", _gate_over_d, [P.test_gate_closed_forms]),
    ("gate", _gate_plain_sigmoid, [P.test_gate_closed_forms]),
    ("gate", _gate_no_weights, [P.test_gate_weights_multiply_the_dot]),
    ("project", _project_transposed, [P.test_projection_one_hot_picks_weight_columns]),
    ("layer_primes", _layer_offsets_continue, [P.test_layer_primes_match_both_layers_table]),
    ("layer_primes", _layer_primes_restart, [P.test_layer_primes_match_both_layers_table]),
    ("hash_rows_layers", _layers_share_multipliers,
     [P.test_layers_with_own_multipliers_hit_unrelated_rows]),
    ("mx_values", _mx_block16, [P.test_mx_values_one_scale_per_32_inputs]),
    ("gate", _gate_mode_ignored, [P.test_plain_gate_closed_forms]),
    ("short_conv", _short_conv_taps_reversed, [P.test_short_conv_equals_torch_rmsnorm_conv1d_silu,
                                               P.test_short_conv_tiny_by_hand]),
    ("short_conv", _short_conv_no_dilation, [P.test_short_conv_reaches_t_minus_3_6_9]),
    ("short_conv", _short_conv_no_residual, [P.test_short_conv_zero_filters_leave_the_gated_value]),
    ("short_conv", _short_conv_sigmoid, [P.test_short_conv_tiny_by_hand]),
    ("rms_norm", _rms_norm_eps_outside, [P.test_short_conv_equals_torch_rmsnorm_conv1d_silu]),
    ("rms_norm", _rms_norm_over_streams, [P.test_short_conv_equals_torch_rmsnorm_conv1d_silu]),
    ("gate_conv", _gate_conv_updates_dead, [P.test_gate_conv_dead_positions]),
    ("gate_conv", _gate_conv_tail_ignores_hist,
     [lambda: P.test_gate_conv_chunked_equals_one_shot((4, 5)),
      lambda: P.test_gate_conv_chunked_equals_one_shot((10, 1, 1, 1))]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTATIONS,
                         ids=[m[1].__name__ for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(E, name, mutant)
    monkeypatch.setattr(P.O, name, mutant, raising=False)
    caught = False
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught = True
    assert caught, f"planted mistake in {name} ({mutant.__name__}) passed every pin"


def test_planted_scale_bias_is_caught(monkeypatch):
    table = np.array([_e8m0_bias128(c) for c in range(256)], dtype=np.float64)
    monkeypatch.setattr(E, "E8M0_TABLE", table)
    with pytest.raises(AssertionError):
        P.test_dequant_exhaustive_against_torch_float8()


def test_unmutated_pins_pass():
    for pins in {id(p): p for m in MUTATIONS for p in m[2]}.values():
        pins()
