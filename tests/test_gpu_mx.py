"""Parity of the block-scaled FP8 path (engram_gather_rows, engram_gather_mx,
engram_project_mx, engram_forward_mx) with the CPU oracle. The looked-up rows
and their split codes and scales match bit for bit; the projection is within
1e-3 + 2e-2 of its output row's RMS of the exact product of the FP8 values and
exact where every output has a single product; gates and streams follow the
bf16 path's element-wise tolerance, with the kv allowance taken from the
projection's bound."""
import numpy as np
import pytest

import oracle as O
from tests.gpu_util import assert_close, kv_tolerance_mx, oracle_rows, say
from workloads import C3, C4, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import hashed_gram_conditional_amd as E  # noqa: E402
from workloads.device import bf16_bits, to_device  # noqa: E402
from workloads.harness import GpuWorkload  # noqa: E402
from tests.test_gpu_parity import S_A, S_B, _check_forward, _cleanup, _sample_tokens  # noqa: E402

DEV = "cuda"


def _rows_of(seed, ids):
    return gen.table_rows(seed, np.asarray(ids, dtype=np.int64))


def test_gather_rows_bit_exact():
    say("gather_rows: 5000 ids incl. out-of-range")
    rng = np.random.default_rng(31)
    R = 100_000
    table = torch.from_numpy(gen.table_rows(5, np.arange(R))).to(DEV)
    ids = rng.integers(-5, R + 5, 5000).astype(np.int64)
    out = torch.full((ids.size, 264), 0xAB, dtype=torch.uint8, device=DEV)
    E.engram_gather_rows(table, R, to_device(ids), ids.size, out)
    torch.cuda.synchronize()
    exp = O.gather_rows(lambda r: gen.table_rows(5, r), ids.reshape(-1, 1), R).reshape(-1, 264)
    assert np.array_equal(out.cpu().numpy(), exp)


def test_gather_mx_splits_rows_bit_exact():
    """codes[i] = the row's 256 E4M3 bytes, scales[i] = its 8 E8M0 bytes, zeros
    for ids outside the table; the same bits from a pinned host copy; a pageable
    table is rejected before any launch."""
    say("gather_mx: 5003 ids incl. out-of-range, device and pinned host table")
    rng = np.random.default_rng(32)
    R = 70_001
    table = torch.from_numpy(gen.table_rows(6, np.arange(R))).to(DEV)
    host = torch.empty(table.shape, dtype=table.dtype, pin_memory=True)
    host.copy_(table)
    ids = rng.integers(-5, R + 5, 5003).astype(np.int64)
    ids[:3] = [0, R - 1, R]
    ids_d = to_device(ids)
    exp = O.gather_rows(lambda r: gen.table_rows(6, r), ids.reshape(-1, 1), R).reshape(-1, 264)
    for src in (table, host):
        codes = torch.full((ids.size, 256), 0xAB, dtype=torch.uint8, device=DEV)
        scales = torch.full((ids.size, 8), 0xCD, dtype=torch.uint8, device=DEV)
        E.engram_gather_mx(src, R, ids_d, ids.size, codes, scales)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), exp[:, :256])
        assert np.array_equal(scales.cpu().numpy(), exp[:, 256:])
    pageable = torch.zeros((64, 264), dtype=torch.uint8)
    codes = torch.full((8, 256), 5, dtype=torch.uint8, device=DEV)
    scales = torch.full((8, 8), 5, dtype=torch.uint8, device=DEV)
    with pytest.raises(E.EngramError) as ex:
        E.engram_gather_mx(pageable, 64, ids_d, 8, codes, scales)
    assert ex.value.status == E.EINVAL
    torch.cuda.synchronize()
    assert bool((codes == 5).all()) and bool((scales == 5).all())


def _mx_case(M, N, S, seed):
    rng = np.random.default_rng(seed)
    rows = _rows_of(seed, rng.integers(0, 10 ** 9, M * S)).reshape(M, S, 264)
    codes, scales = gen.quantize_mx_e4m3(rng.normal(0.0, 0.02, (N, S * 256)))
    e = O.mx_values(rows[:, :, :256].reshape(M, S * 256), rows[:, :, 256:].reshape(M, S * 8))
    w = O.mx_values(codes, scales)
    return rows, codes, scales, e, w


def _project_mx(rows, codes, scales, M, N, S, with_ws):
    return O.bf16_bits_to_f64(_project_mx_bits(rows, codes, scales, M, N, S, with_ws))


def _project_mx_bits(rows, codes, scales, M, N, S, with_ws):
    n = E.engram_project_mx_workspace_size(M, S, N) if with_ws else 0
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=DEV) if n else None
    kv = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    e_codes = to_device(np.ascontiguousarray(rows[:, :, :256]).reshape(M, S * 256))
    e_scales = to_device(np.ascontiguousarray(rows[:, :, 256:]).reshape(M, S * 8))
    E.engram_project_mx(e_codes, e_scales, S, to_device(codes), to_device(scales), kv, M, N,
                        ws, n)
    torch.cuda.synchronize()
    return bf16_bits(kv)


# shapes: tiny, ragged, a wide-tile grid (>= 256 tiles), the decode shape (the
# skinny schedule), a decode-sized call whose 8 K-steps do not fill the skinny
# schedule's 6-step ring (split over K instead), odd K-step counts (S = 1, 3: 2
# and 6 steps; S = 5: 10)
@pytest.mark.parametrize("M,N,S", [(1, 8, 1), (31, 264, 3), (300, 520, 24), (257, 1032, 5),
                                   (4100, 4104, 1), (256, 25600, 24), (200, 20480, 4)])
def test_project_mx_against_oracle(M, N, S):
    say(f"project_mx {M}x{N} S={S}")
    rows, codes, scales, e, w = _mx_case(M, N, S, M * 7 + N + S)
    exact = O.project(e, w)
    tol = kv_tolerance_mx(exact)
    for with_ws in (True, False):
        got = _project_mx(rows, codes, scales, M, N, S, with_ws)
        assert_close(got, exact, f"kv mx {M}x{N} S={S} ws={with_ws}", atol=0, rtol=0, extra=tol)


@pytest.mark.parametrize("N", [25600, 16384], ids=["rows_96_128_per_CU", "rows_64_per_CU"])
def test_project_mx_decode_bits_equal_wide_tiles(N):
    """Calls of at most 256 tokens take the skinny schedule (every token against
    one CU's weight rows, K not split); a 300-token call without a workspace
    takes one block per 256 x 256 tile over the whole K. Both sum each output's
    64-input chunks in order in one accumulator, so a decode call's kv is the
    bits of the same rows in the larger call."""
    S, big = 24, 300
    say(f"project_mx decode vs wide tiles, N={N}")
    rng = np.random.default_rng(N)
    rows = _rows_of(N, rng.integers(0, 10 ** 9, big * S)).reshape(big, S, 264)
    codes, scales = gen.quantize_mx_e4m3(rng.normal(0.0, 0.02, (N, S * 256)))
    ref = _project_mx_bits(rows, codes, scales, big, N, S, with_ws=False)
    for m in (256, 200, 1):
        got = _project_mx_bits(rows[:m], codes, scales, m, N, S, with_ws=True)
        assert np.array_equal(got, ref[:m]), f"{m} tokens"


def test_project_mx_single_products_exact():
    # each token's rows hold one nonzero code (1.0 = 0x38) under scale 127 + d,
    # so kv[t, c] = 2^d W[c, k_t], exact in bf16
    M, N, S = 600, 1032, 4
    rng = np.random.default_rng(5)
    rows = np.zeros((M, S, 264), np.uint8)
    rows[:, :, 256:] = 127
    ks = rng.integers(0, S * 256, M)
    d = rng.integers(-3, 4, M)
    for t in range(M):
        j, i = divmod(int(ks[t]), 256)
        rows[t, j, i] = 0x38
        rows[t, j, 256 + i // 32] = 127 + d[t]
    codes, scales = gen.quantize_mx_e4m3(rng.normal(0.0, 0.02, (N, S * 256)))
    w = O.mx_values(codes, scales)
    exp = O.round_to_bf16_bits(np.exp2(d)[:, None] * w.T[ks])
    for with_ws in (True, False):
        got = _project_mx(rows, codes, scales, M, N, S, with_ws)
        assert np.array_equal(O.round_to_bf16_bits(got), exp)


def _check_forward_mx(gw, h_dev, gates_dev, tokens):
    return _check_forward(gw, h_dev, gates_dev, tokens, wkv=O.mx_values(*gw.wkv_mx_np), mx=True)


@pytest.mark.parametrize("w", [S_A, S_B], ids=lambda w: w.name)
def test_forward_mx_small(w):
    say(f"forward_mx {w.name}: tokens={w.tokens}")
    gw = GpuWorkload(w, wkv_mx=True)
    ws, n = gw.workspace_mx()
    gates = torch.full((w.tokens, w.hc), -1.0, dtype=torch.float32, device=DEV)
    E.engram_forward_mx(gw.params, gw.desc, gw.ids, None, None, gw.table, gw.w_codes,
                        gw.w_scales, gw.q_w, gw.k_w, gw.h, gates, ws, n)
    torch.cuda.synchronize()
    _check_forward_mx(gw, gw.h, gates, np.arange(w.tokens))


def test_forward_mx_prefill_sampled():
    say("forward_mx C3 (4 x 8192 tokens), sampled tokens")
    gw = GpuWorkload(C3, wkv_mx=True)
    ws, n = gw.workspace_mx()
    gates = torch.empty((C3.tokens, C3.hc), dtype=torch.float32, device=DEV)
    E.engram_forward_mx(gw.params, gw.desc, gw.ids, None, None, gw.table, gw.w_codes,
                        gw.w_scales, gw.q_w, gw.k_w, gw.h, gates, ws, n)
    torch.cuda.synchronize()
    _check_forward_mx(gw, gw.h, gates, _sample_tokens(gw, 2048, 7))
    del ws
    gw.free()


def test_forward_mx_c4_decode_every_token():
    """The decode step with the block-scaled FP8 weight: 256 sequences x 1 token
    with their history on the 384,006,168-row (101.4 GB) table, the projection
    in the skinny schedule. Every token against the oracle at the gate
    tolerance, the history after the token, and the bits of the stage entry
    points."""
    say("forward_mx C4 decode: 256 x 1 token, 101.4 GB table, every token")
    gw = GpuWorkload(C4, wkv_mx=True)
    try:
        h0 = gw.h.clone()
        ws, n = gw.workspace_mx()
        gates = torch.full((C4.tokens, C4.hc), -1.0, dtype=torch.float32, device=DEV)
        hout = torch.empty((C4.batch, 3), dtype=torch.int32, device=DEV)
        E.engram_forward_mx(gw.params, gw.desc, gw.ids, gw.hist_in, hout, gw.table, gw.w_codes,
                            gw.w_scales, gw.q_w, gw.k_w, gw.h, gates, ws, n)
        torch.cuda.synchronize()
        _check_forward_mx(gw, gw.h, gates, np.arange(C4.tokens))
        _, exp_hist = oracle_rows(gw)
        assert np.array_equal(hout.cpu().numpy(), exp_hist)
        # the step forms and splits the rows in one launch; the stage entry points
        # (hash, then the row-splitting gather, the projection, the gate) give its bits
        T, S = C4.tokens, C4.segments
        rows = torch.empty((T, S), dtype=torch.int64, device=DEV)
        E.engram_hash(gw.params, gw.ids, C4.batch, C4.seq, gw.hist_in, None, rows)
        e_codes = torch.empty((T, S * 256), dtype=torch.uint8, device=DEV)
        e_scales = torch.empty((T, S * 8), dtype=torch.uint8, device=DEV)
        E.engram_gather_mx(gw.table, gw.rows, rows, T * S, e_codes, e_scales)
        N = (C4.hc + 1) * C4.dim
        kv = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
        E.engram_project_mx(e_codes, e_scales, S, gw.w_codes, gw.w_scales, kv, T, N)
        g2 = torch.empty_like(gates)
        E.engram_gate(gw.desc, gw.ids, C4.raw_vocab, kv, gw.q_w, gw.k_w, h0, g2)
        torch.cuda.synchronize()
        assert torch.equal(h0.view(torch.int16), gw.h.view(torch.int16))
        assert torch.equal(g2, gates)
    finally:
        gw.free()
        _cleanup()
