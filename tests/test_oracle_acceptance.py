"""Pins for the oracle's spot-check and acceptance helpers (CPU only).

* ``oracle.gemm.dense_gemm_rows_cols`` -- the expected value of every
  full-size sampled GEMM test -- equals the full ``dense_gemm`` indexed at the
  same rows and columns, bit for bit, in all three modes, with bias (MXFP8)
  and alpha (NVFP4), for unsorted, non-contiguous and repeated indices.
* ``oracle.gemm.tolerance`` -- the absolute term of the acceptance bound --
  against a hand-worked golden (``tests/golden/tolerance_2x2.txt``): 2 x 2
  outputs with distinct per-group scales in each row, NVFP4 with a non-unit
  alpha and MXFP8 with UE8M0 scales on both sides of 2^0.  A transposed outer
  product, a missing alpha or norms of the codes instead of the dequantised
  values all fail it.
* ``tests._gpu.assert_gemm_close`` -- the acceptance check itself: an
  element inside the per-element bound passes, one just outside fails, the
  relative Frobenius criterion catches error spread inside the per-element
  bound, and non-finite outputs fail.
"""
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from synth import normal_bf16
from tests._gpu import assert_gemm_close

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tolerance_2x2.txt")


# ---------------------------------------------------------------- rows / cols
@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
def test_rows_cols_equals_indexed_full_gemm(mode):
    rng = np.random.default_rng(41)
    M, N, K = 40, 48, 128
    xa = normal_bf16(rng, (M, K))
    xb = normal_bf16(rng, (N, K), 0.3)
    bias = alpha = None
    if mode == "nvfp4":
        a, sfa, ga = Q.nvfp4_quant_bf16(xa)
        b, sfb, gb = Q.nvfp4_quant_bf16(xb)
        alpha = np.float32(np.float32(ga) * np.float32(gb))
        assert alpha != 1.0
    else:
        a, sfa = Q.mx_quant_bf16(xa, mode)
        b, sfb = Q.mx_quant_bf16(xb, mode)
        if mode == "mxfp8":
            bias = normal_bf16(rng, (N,), 0.5)
    full = G.dense_gemm(mode, a, sfa, b, sfb, bias=bias, alpha=alpha)
    for trial in range(4):
        rows = rng.choice(M, size=9, replace=trial == 3)        # unsorted; repeats in the last trial
        cols = rng.choice(N, size=11, replace=trial == 3)
        got = G.dense_gemm_rows_cols(mode, a, sfa, b, sfb, rows, cols, bias=bias, alpha=alpha)
        assert got.dtype == full.dtype and got.shape == (len(rows), len(cols))
        assert np.array_equal(got, full[rows][:, cols]), (mode, trial)
    # the bias must follow the selected columns, not the first ones
    if bias is not None:
        cols = np.array([N - 1, 0, N // 2])
        nb = G.dense_gemm_rows_cols(mode, a, sfa, b, sfb, np.arange(3), cols, bias=None)
        wb = G.dense_gemm_rows_cols(mode, a, sfa, b, sfb, np.arange(3), cols, bias=bias)
        assert not np.array_equal(nb, wb)
        assert np.array_equal(wb, full[:3][:, cols])


# ---------------------------------------------------------------- tolerance golden
def _read_golden():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "case":
            cur = {"mode": f[1], "M": int(f[2]), "N": int(f[3]), "K": int(f[4]),
                   "alpha": None if f[5] == "none" else float(f[5]),
                   "a": [], "b": [], "sfa": [], "sfb": [], "slack": []}
            cases.append(cur)
        elif f[0] in ("a", "b", "sfa", "sfb"):
            cur[f[0]].append((int(f[1]), int(f[2]), int(f[3], 16)))
        elif f[0] == "slack":
            cur["slack"].append((int(f[1]), int(f[2]), float(f[3])))
    return cases


def _operand(entries, sf_entries, rows, K, mode):
    gs = 16 if mode == "nvfp4" else 32
    codes = np.zeros((rows, K), np.uint8)
    for r, k, c in entries:
        codes[r, k] = c
    sf = np.zeros((rows, K // gs), np.uint8)
    seen = set()
    for r, g, byte in sf_entries:
        sf[r, g] = byte
        seen.add((r, g))
    assert len(seen) == rows * (K // gs), "every scale of the golden is given"
    return (codes if mode == "mxfp8" else F.pack_nibbles(codes)), sf


@pytest.mark.parametrize("idx", [0, 1])
def test_tolerance_matches_hand_worked_golden(idx):
    case = _read_golden()[idx]
    mode, M, N, K = case["mode"], case["M"], case["N"], case["K"]
    a, sfa = _operand(case["a"], case["sfa"], M, K, mode)
    b, sfb = _operand(case["b"], case["sfb"], N, K, mode)
    ad, bd = Q.dequant(a, sfa, mode), Q.dequant(b, sfb, mode)
    alpha = None if case["alpha"] is None else np.float32(case["alpha"])
    got = G.tolerance(ad, bd, alpha)
    want = np.zeros((M, N))
    for m, n, v in case["slack"]:
        want[m, n] = v
    assert len(case["slack"]) == M * N
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)
    # alpha enters as a magnitude
    if alpha is not None:
        np.testing.assert_allclose(G.tolerance(ad, bd, -alpha), want, rtol=1e-12, atol=0)


def test_golden_cases_cover_both_scale_encodings():
    modes = [c["mode"] for c in _read_golden()]
    assert modes == ["nvfp4", "mxfp8"]


# ---------------------------------------------------------------- the acceptance check
def _bf16(x):
    return F.bf16_round(np.asarray(x, np.float64))


def _setup(n=64):
    """ref = 1.0 everywhere; ||a_m|| = 1 and ||b_n|| = 3.90625, so the absolute
    slack is ~2^-8 and the bound at ref = 1 is 2^-7 + 2^-8 (BF16 ulp at 1 is
    2^-7 above and 2^-8 below)."""
    ref = _bf16(np.ones((n, n)))
    a = np.zeros((n, 8))
    a[:, 0] = 1.0
    b = np.zeros((n, 8))
    b[:, 3] = 3.90625
    return ref, a, b


def test_acceptance_inside_and_outside_one_element():
    ref, a, b = _setup()
    out = ref.copy()
    out[3, 5] = 0x3F81                         # 1 + 2^-7: error 2^-7 inside 1.5 * 2^-7
    assert_gemm_close(out, ref, a, b)
    out[3, 5] = 0x3F82                         # 1 + 2^-6: error 2^-6 outside
    with pytest.raises(AssertionError):
        assert_gemm_close(out, ref, a, b)
    out[3, 5] = 0x3F7F                         # 1 - 2^-8: inside
    assert_gemm_close(out, ref, a, b)
    out[3, 5] = 0x3F7C                         # 1 - 2^-6: outside
    with pytest.raises(AssertionError):
        assert_gemm_close(out, ref, a, b)


def test_acceptance_alpha_widens_the_absolute_term():
    ref, a, b = _setup()
    out = ref.copy()
    out[7, 1] = 0x3F82                         # error 2^-6
    with pytest.raises(AssertionError):
        assert_gemm_close(out, ref, a, b, alpha=np.float32(1.0))
    assert_gemm_close(out, ref, a, b, alpha=np.float32(4.0))    # slack ~2^-6, bound ~1.5 * 2^-6


def test_acceptance_frobenius_catches_spread_error():
    ref, a, b = _setup()
    out = np.full_like(ref, 0x3F81)            # every element off by 2^-7: each inside its bound
    with pytest.raises(AssertionError, match="Frobenius"):
        assert_gemm_close(out, ref, a, b)


def test_acceptance_rejects_non_finite():
    ref, a, b = _setup()
    out = ref.copy()
    out[0, 0] = 0x7FC0                         # NaN
    with pytest.raises(AssertionError):
        assert_gemm_close(out, ref, a, b)
