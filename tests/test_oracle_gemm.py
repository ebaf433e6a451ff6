"""Pins for oracle.gemm and oracle.swiglu.

* Integer-exact GEMM: small-integer codes with every scale byte 127, so every
  product and partial sum is an exact integer; the result must equal a
  Python-integer dot product rounded once to BF16 (exact for |sum| <= 256).
* Exact-rational brute force at 4 x 4 x 32 with random scales (Fractions +
  an integer BF16 rounding).
* gemm(A, B) == gemm(B, A)^T; batch / contiguous / masked equal a loop of
  dense GEMMs done by independent slicing; masked equals contiguous on the
  gathered valid rows.
* SwiGLU closed forms: silu(0) = 0, up = 0, large +-gate; torch's float64
  silu as an independent library routine.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from oracle import swiglu as S
from synth import to_bf16_bits
from tests import _exact as X

INT_E4M3 = {v: c for c, v in enumerate(F.E4M3_TABLE[:127]) if float(v).is_integer() and v <= 16}
INT_E2M1 = {0: 0, 1: 2, 2: 4, 3: 5, 4: 6, 6: 7}


def _int_codes(vals, fmt):
    if fmt == "mxfp8":
        table = INT_E4M3
        return np.vectorize(lambda v: table[abs(v)] | (0x80 if v < 0 else 0))(vals).astype(np.uint8)
    table = INT_E2M1
    c = np.vectorize(lambda v: table[abs(v)] | (0x8 if v < 0 else 0))(vals).astype(np.uint8)
    return F.pack_nibbles(c)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_integer_exact_gemm(fmt):
    rng = np.random.default_rng(11)
    M, N, K = 8, 12, 64
    choices = np.array([-2, -1, 0, 1, 2])
    av = rng.choice(choices, (M, K))
    bv = rng.choice(choices, (N, K))
    a = _int_codes(av, fmt)
    b = _int_codes(bv, fmt)
    sfa = np.full((M, K // 32), 127, np.uint8)
    sfb = np.full((N, K // 32), 127, np.uint8)
    out = G.dense_gemm(fmt, a, sfa, b, sfb)
    for m in range(M):
        for n in range(N):
            s = sum(int(av[m, k]) * int(bv[n, k]) for k in range(K))
            assert abs(s) <= 256
            want = torch.tensor(float(s)).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
            assert int(out[m, n]) == want, (m, n, s)


def test_integer_exact_gemm_nvfp4_unit_scales():
    rng = np.random.default_rng(12)
    M, N, K = 4, 8, 64
    av = rng.choice(np.array([-3, -1, 0, 1, 2, 4]), (M, K))
    bv = rng.choice(np.array([-2, -1, 0, 1, 6]), (N, K))
    a = _int_codes(av, "nvfp4")
    b = _int_codes(bv, "nvfp4")
    sfa = np.full((M, K // 16), 0x38, np.uint8)         # UE4M3 1.0
    sfb = np.full((N, K // 16), 0x38, np.uint8)
    out = G.dense_gemm("nvfp4", a, sfa, b, sfb, alpha=np.float32(1.0))
    want = F.bf16_round((av @ bv.T).astype(np.float64))
    assert np.array_equal(out, want)
    assert np.max(np.abs(av @ bv.T)) <= 256


def _rational_gemm(mode, a, sfa, b, sfb, bias=None, alpha=None):
    """Exact rationals from the bit fields, one BF16 rounding at the end."""
    if mode == "mxfp8":
        grid = dict(X.E4M3)

        def dec(c):
            v = grid[c & 0x7F]
            return -v if c & 0x80 else v
        A = [[dec(int(c)) for c in row] for row in a]
        Bm = [[dec(int(c)) for c in row] for row in b]
        gs = 32

        def sc(s):
            return X.Fr(2) ** (int(s) - 127)
    else:
        grid = dict(X.E2M1)

        def dec(c):
            v = grid[c & 0x7]
            return -v if c & 0x8 else v
        ua, ub = F.unpack_nibbles(a), F.unpack_nibbles(b)
        A = [[dec(int(c)) for c in row] for row in ua]
        Bm = [[dec(int(c)) for c in row] for row in ub]
        if mode == "mxfp4":
            gs = 32

            def sc(s):
                return X.Fr(2) ** (int(s) - 127)
        else:
            gs = 16
            e4 = dict(X.E4M3)

            def sc(s):
                return e4[int(s)]
    M, N, K = len(A), len(Bm), len(A[0])
    out = np.zeros((M, N), np.uint16)
    for m in range(M):
        for n in range(N):
            acc = X.Fr(0)
            for k in range(K):
                acc += A[m][k] * sc(sfa[m, k // gs]) * Bm[n][k] * sc(sfb[n, k // gs])
            if alpha is not None:
                acc *= X.Fr(float(np.float32(alpha)))
            if bias is not None:
                acc += X.bf16_value(int(bias[n]))[0]
            r = X.bf16_round_value(acc)
            out[m, n] = F.bf16_round(float(r))      # r is an exact BF16 value
            assert float(r) == F.bf16_decode(out[m, n])
    return out


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("seed", range(3))
def test_rational_brute_force_4x4x32(mode, seed):
    rng = np.random.default_rng(300 + seed)
    M = N = 4
    K = 32 if mode != "nvfp4" else 32
    xa = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32) * np.float32(2.0 ** rng.integers(-4, 4)))
    xb = to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    bias = to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.1)) if mode == "mxfp8" else None
    if mode == "nvfp4":
        a, sfa, ga = Q.nvfp4_quant_bf16(xa)
        b, sfb, gb = Q.nvfp4_quant_bf16(xb)
        alpha = np.float32(ga * gb)
    else:
        a, sfa = Q.mx_quant_bf16(xa, mode)
        b, sfb = Q.mx_quant_bf16(xb, mode)
        alpha = None
    got = G.dense_gemm(mode, a, sfa, b, sfb, bias=bias, alpha=alpha)
    want = _rational_gemm(mode, a, sfa, b, sfb, bias=bias, alpha=alpha)
    assert np.array_equal(got, want)


def _quantized(rng, rows, K, mode, sigma=1.0):
    x = to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32) * np.float32(sigma))
    if mode == "nvfp4":
        q, s, g = Q.nvfp4_quant_bf16(x)
        return q, s, g
    q, s = Q.mx_quant_bf16(x, mode)
    return q, s, None


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4"])
def test_transpose_symmetry(mode):
    rng = np.random.default_rng(5)
    a, sfa, _ = _quantized(rng, 24, 96, mode)
    b, sfb, _ = _quantized(rng, 40, 96, mode)
    assert np.array_equal(G.dense_gemm(mode, a, sfa, b, sfb), G.dense_gemm(mode, b, sfb, a, sfa).T)


def test_batch_is_loop_of_dense():
    rng = np.random.default_rng(6)
    Bn, M, N, K = 3, 16, 24, 64
    a, sfa, _ = _quantized(rng, Bn * M, K, "mxfp8")
    b, sfb, _ = _quantized(rng, Bn * N, K, "mxfp8")
    bias = to_bf16_bits(rng.standard_normal((Bn, N)).astype(np.float32))
    out = G.batch_gemm("mxfp8", a.reshape(Bn, M, K), sfa.reshape(Bn, M, -1),
                       b.reshape(Bn, N, K), sfb.reshape(Bn, N, -1), bias=bias)
    for i in range(Bn):
        full = G.dense_gemm("mxfp8", a, sfa, b[i * N:(i + 1) * N], sfb[i * N:(i + 1) * N], bias=bias[i])
        assert np.array_equal(out[i], full[i * M:(i + 1) * M])


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4"])
def test_contiguous_is_loop_of_dense_and_masked_matches(mode):
    rng = np.random.default_rng(8)
    E, K, N = 5, 64, 32
    counts = np.array([7, 0, 33, 1, 16])
    ends = np.cumsum(counts).astype(np.int32)
    R = int(ends[-1]) + 5                                  # 5 trailing rows in no group
    a, sfa, _ = _quantized(rng, R, K, mode)
    bq, bs, _ = _quantized(rng, E * N, K, mode)
    Kb = bq.shape[1]
    b, sfb = bq.reshape(E, N, Kb), bs.reshape(E, N, -1)
    sentinel = np.full((R, N), 0x7FC1, np.uint16)
    out, written = G.group_contiguous_gemm(mode, a, sfa, b, sfb, ends, out=sentinel)
    assert written.sum() == counts.sum()
    assert np.all(out[~written] == 0x7FC1)
    row_expert = np.repeat(np.arange(E), counts)
    for e in range(E):
        full = G.dense_gemm(mode, a, sfa, b[e], sfb[e])  # all rows against expert e
        rows = np.flatnonzero(row_expert == e)
        assert np.array_equal(out[rows], full[rows])
    # masked layout: each expert's rows copied into a 40-row slot
    Mmax = 40
    am = np.zeros((E * Mmax, a.shape[1]), np.uint8)
    sm = np.full((E * Mmax, sfa.shape[1]), 0xFF, np.uint8)   # garbage scales in padding
    starts = np.concatenate([[0], ends[:-1]])
    for e in range(E):
        am[e * Mmax:e * Mmax + counts[e]] = a[starts[e]:starts[e] + counts[e]]
        sm[e * Mmax:e * Mmax + counts[e]] = sfa[starts[e]:starts[e] + counts[e]]
    mout, mw = G.group_masked_gemm(mode, am, sm, b, sfb, counts.astype(np.int32), Mmax,
                                   out=np.full((E * Mmax, N), 0x7FC1, np.uint16))
    for e in range(E):
        assert np.array_equal(mout[e * Mmax:e * Mmax + counts[e]], out[starts[e]:starts[e] + counts[e]])
        assert np.all(mout[e * Mmax + counts[e]:(e + 1) * Mmax] == 0x7FC1)


def test_contiguous_clamps_bad_ends():
    rng = np.random.default_rng(9)
    a, sfa, _ = _quantized(rng, 20, 32, "mxfp8")
    bq, bs, _ = _quantized(rng, 3 * 8, 32, "mxfp8")
    b, sfb = bq.reshape(3, 8, 32), bs.reshape(3, 8, -1)
    out, written = G.group_contiguous_gemm("mxfp8", a, sfa, b, sfb, np.array([10, 4, 99], np.int32))
    assert written.sum() == 20          # [0,10), [10,10), [10,20)
    assert np.array_equal(out[10:], G.dense_gemm("mxfp8", a[10:], sfa[10:], b[2], sfb[2]))


def test_alpha_and_bias_applied_once():
    rng = np.random.default_rng(10)
    a, sfa, ga = _quantized(rng, 8, 64, "nvfp4")
    b, sfb, gb = _quantized(rng, 8, 64, "nvfp4")
    base = G.dense_f64(Q.dequant(a, sfa, "nvfp4"), Q.dequant(b, sfb, "nvfp4"))
    got = F.bf16_decode(G.dense_gemm("nvfp4", a, sfa, b, sfb, alpha=ga * gb))
    want = F.bf16_decode(F.bf16_round(base * float(np.float32(ga * gb))))
    assert np.array_equal(got, want)
    # the alpha-scaled result approximates the BF16 inputs' product
    xa = Q.dequant(a, sfa, "nvfp4", g=ga)
    assert np.allclose(got, F.bf16_decode(F.bf16_round(xa @ Q.dequant(b, sfb, "nvfp4", g=gb).T)), rtol=1e-2, atol=1e-3)


# ---------------------------------------------------------------- SwiGLU
def test_swiglu_closed_forms():
    h = 4
    gate = np.array([[0.0, 100.0, -100.0, 1.0]], np.float32)
    up = np.array([[5.0, 3.0, 7.0, 0.0]], np.float32)
    x = to_bf16_bits(np.concatenate([gate, up], axis=1))
    y = S.swiglu_f64(x, h)
    assert y[0, 0] == 0.0                  # silu(0) = 0
    assert y[0, 1] == 300.0                # exp(-100) vanishes next to 1
    assert abs(y[0, 2]) < 1e-40            # large negative gate -> 0
    assert y[0, 3] == 0.0                  # up = 0


def test_swiglu_matches_torch_silu():
    rng = np.random.default_rng(13)
    x = to_bf16_bits(rng.standard_normal((8, 64)).astype(np.float32) * 3)
    y = S.swiglu_f64(x, 32)
    xt = torch.from_numpy(F.bf16_decode(x))
    ref = (xt[:, 32:] * torch.nn.functional.silu(xt[:, :32])).numpy()
    assert np.allclose(y, ref, rtol=1e-14, atol=0)


def test_processed_rows_forms():
    m = S.processed_rows(10, group_end=np.array([3, 3, 8]), valid=np.array([2, 5, 4]))
    assert np.flatnonzero(m).tolist() == [0, 1, 3, 4, 5, 6]
    m = S.processed_rows(12, slot_rows=4, valid=np.array([4, 0, 9]), num_groups=3)
    assert np.flatnonzero(m).tolist() == [0, 1, 2, 3, 8, 9, 10, 11]
    m = S.processed_rows(6, group_end=np.array([4, 2, 9]))
    assert m.all()


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
def test_swiglu_quant_is_quant_of_y(mode):
    rng = np.random.default_rng(14)
    x = to_bf16_bits(rng.standard_normal((6, 128)).astype(np.float32))
    g = np.float32(0.01) if mode == "nvfp4" else None
    codes, sf, y = S.swiglu_quant(x, 64, mode, g=g)
    y32 = y.astype(np.float32).astype(np.float64)
    if mode == "nvfp4":
        c2, s2, _ = Q.nvfp4_quant_values(y32, g)
    else:
        c2, s2 = Q.mx_quant_values(y, mode)
    assert np.array_equal(codes, c2) and np.array_equal(sf, s2)
