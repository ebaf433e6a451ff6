"""Pins for oracle.dglu (the backward grouped GEMM with the dSwiGLU epilogue;
cuDNN FE "Grouped GEMM + dGLU (SM100)": the R_g = alpha_g^2 A_g B_g^T
equation, Step 1 and Step 2 "For dSwiGLU").

* Autograd: with R integer-exact (small-integer codes, unit scales, alpha a
  power of two, checked against Python-integer sums), D and dprob equal
  torch's float64 autograd gradients of the forward loss
  L = sum_m prob_m sum_n R[m, n] * input[m, n] * silu(gate[m, n]) with
  respect to X = beta C and prob, where silu is torch.nn.functional.silu (an
  independent library routine) and the input / gate halves of X are picked
  out column by column from the interleave reading.
* Finite differences of the forward SwiGLU oracle (oracle.swiglu) at the
  same X values: D / (R prob) is its derivative in each half.
* Closed forms: gate = 0, prob = 0, input = 0, gate -> +inf / -inf.
* Identities: beta scales C exactly; alpha enters squared; each group uses
  its own weights; rows past the last end are not written; dprob
  accumulates onto what it held; the BF16 output is D rounded once.
* The tolerance helper against a hand-worked 1-row case.
"""
import math

import numpy as np
import pytest
import torch

from oracle import dglu as DG
from oracle import formats as F
from oracle import quant as Q
from oracle import swiglu as S
from synth import normal_bf16, to_bf16_bits
from tests.test_oracle_gemm import INT_E2M1, INT_E4M3


def _int_codes(vals, mode):
    table = INT_E4M3 if mode == "mxfp8" else INT_E2M1
    sign = 0x80 if mode == "mxfp8" else 0x8
    c = np.vectorize(lambda v: table[abs(int(v))] | (sign if v < 0 else 0))(vals).astype(np.uint8)
    return c if mode == "mxfp8" else F.pack_nibbles(c)


def _case(mode="mxfp8", seed=0, N=64, K=64, counts=(5, 0, 9, 3), extra=2):
    rng = np.random.default_rng(seed)
    G = len(counts)
    ends = np.cumsum(counts).astype(np.int32)
    M = int(ends[-1]) + extra                            # rows past the last end
    av = rng.choice(np.array([-2, -1, 0, 1, 2]), (M, K))
    bv = rng.choice(np.array([-1, 0, 1, 2]), (G, N, K))
    a = _int_codes(av, mode)
    b = _int_codes(bv.reshape(G * N, K), mode).reshape(G, N, -1)
    sfa = np.full((M, K // 32), 127, np.uint8)
    sfb = np.full((G, N, K // 32), 127, np.uint8)
    c = normal_bf16(rng, (M, 2 * N), 1.5)
    prob = rng.random(M).astype(np.float32)
    alpha = np.array([0.5, 2.0, 1.0, 0.25][:G], np.float32)
    beta = np.array([1.0, 0.5, 2.0, 0.75][:G], np.float32)
    return dict(mode=mode, a=a, sfa=sfa, b=b, sfb=sfb, ends=ends, c=c, prob=prob, alpha=alpha, beta=beta,
                av=av, bv=bv, M=M, N=N, G=G)


def _run(cs, **kw):
    args = dict(alpha=cs["alpha"], beta=cs["beta"])
    args.update(kw)
    return DG.grouped_gemm_dswiglu_f64(cs["mode"], cs["a"], cs["sfa"], cs["b"], cs["sfb"], cs["ends"], cs["c"],
                                       cs["prob"], **args)


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4"])
def test_R_is_integer_exact(mode):
    cs = _case(mode, seed=1)
    R, _, _, written = _run(cs)
    prev = 0
    for g, end in enumerate(cs["ends"]):
        for m in range(prev, end):
            for n in range(cs["N"]):
                s = sum(int(cs["av"][m, k]) * int(cs["bv"][g, n, k]) for k in range(cs["av"].shape[1]))
                assert R[m, n] == float(cs["alpha"][g]) ** 2 * s, (m, n)
        prev = end
    assert not written[prev:].any() and written[:prev].all()


def test_autograd_of_forward_loss():
    cs = _case("mxfp8", seed=2)
    R, D, dprob, written = _run(cs)
    N, M = cs["N"], cs["M"]
    # independent decode of C (torch's bfloat16) and of the interleave, column by column
    Ct = torch.from_numpy(cs["c"].view(np.int16)).view(torch.bfloat16).double()
    beta_row = torch.zeros(M, dtype=torch.float64)
    prev = 0
    for g, end in enumerate(cs["ends"]):
        beta_row[prev:end] = float(cs["beta"][g])
        prev = end
    X = (Ct * beta_row[:, None]).clone().requires_grad_(True)
    prob = torch.from_numpy(cs["prob"].astype(np.float64)).requires_grad_(True)
    inp_cols = [64 * (n // 32) + n % 32 for n in range(N)]
    gate_cols = [64 * (n // 32) + 32 + n % 32 for n in range(N)]
    inp, gate = X[:, inp_cols], X[:, gate_cols]
    Rt = torch.from_numpy(R)
    L = (prob[:, None] * Rt * inp * torch.nn.functional.silu(gate)).sum()
    L.backward()
    w = torch.from_numpy(written)
    np.testing.assert_allclose(D[written], X.grad[w].numpy(), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(dprob[written], prob.grad[w].numpy(), rtol=1e-12, atol=1e-300)


def test_finite_differences_of_forward_swiglu():
    cs = _case("mxfp8", seed=3, counts=(12,), extra=0)
    R, D, _, _ = _run(cs)
    ic, gc = DG.pair_columns(cs["N"])
    X = float(cs["beta"][0]) * F.bf16_decode(cs["c"])
    inp, gate = X[:, ic], X[:, gc]
    h = 1e-6
    d_gate = (S.swiglu_values_f64(gate + h, inp) - S.swiglu_values_f64(gate - h, inp)) / (2 * h)
    d_inp = (S.swiglu_values_f64(gate, inp + h) - S.swiglu_values_f64(gate, inp - h)) / (2 * h)
    scale = R * cs["prob"].astype(np.float64)[:, None]
    mask = np.abs(scale) > 0
    np.testing.assert_allclose(D[:, gc][mask] / scale[mask], d_gate[mask], rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(D[:, ic][mask] / scale[mask], d_inp[mask], rtol=1e-6, atol=1e-8)


def _one_row(c_in, c_gate, prob=1.0, N=32, K=32):
    """1 row, R[0, n] = 2 for every n (codes 1.0 and 2.0, unit scales)."""
    a = np.full((1, K), 0x38, np.uint8)                 # E4M3 1.0
    b = np.zeros((1, N, K), np.uint8)
    b[0, :, 0] = 0x40                                   # E4M3 2.0 at k = 0
    sfa = np.full((1, 1), 127, np.uint8)
    sfb = np.full((1, N, 1), 127, np.uint8)
    c = np.zeros((1, 2 * N), np.float32)
    c[0, :32], c[0, 32:] = c_in, c_gate
    return DG.grouped_gemm_dswiglu_f64("mxfp8", a, sfa, b, sfb, np.array([1], np.int32), to_bf16_bits(c),
                                       np.array([prob], np.float32))


def test_closed_forms():
    # gate = 0: swish = 0, sigmoid = 1/2 -> dinput = 0, dgate = R prob input / 2, dprob = 0
    R, D, dp, _ = _one_row(3.0, 0.0, prob=0.5)
    assert np.all(R == 2.0)
    assert np.all(D[0, :32] == 0.0) and np.all(D[0, 32:] == 2.0 * 0.5 * 3.0 * 0.5) and dp[0] == 0.0
    # prob = 0: D = 0, but dprob = sum R input swish (no factor of prob)
    R, D, dp, _ = _one_row(1.0, 2.0, prob=0.0)
    sw = 2.0 / (1.0 + math.exp(-2.0))
    assert np.all(D == 0.0) and dp[0] == pytest.approx(32 * 2.0 * 1.0 * sw, rel=1e-14)
    # input = 0: dgate = 0, dprob = 0, dinput = R prob swish
    R, D, dp, _ = _one_row(0.0, 2.0, prob=0.25)
    assert np.all(D[0, 32:] == 0.0) and dp[0] == 0.0
    np.testing.assert_allclose(D[0, :32], 2.0 * 0.25 * sw, rtol=1e-14)
    # gate -> +inf: sigmoid -> 1, dgate -> R prob input; gate -> -inf: everything -> 0
    R, D, dp, _ = _one_row(1.0, 60.0)
    np.testing.assert_allclose(D[0, 32:], 2.0, rtol=1e-14)
    np.testing.assert_allclose(D[0, :32], 2.0 * 60.0, rtol=1e-14)
    R, D, dp, _ = _one_row(1.0, -200.0)
    assert np.all(np.abs(D) < 1e-80) and abs(dp[0]) < 1e-80


def test_beta_scales_c_and_alpha_enters_squared():
    cs = _case("mxfp8", seed=4)
    _, D1, p1, _ = _run(cs, beta=np.full(cs["G"], 2.0, np.float32), alpha=None)
    c2 = to_bf16_bits(2.0 * F.bf16_decode(cs["c"]).astype(np.float32))   # exact doubling
    _, D2, p2, _ = DG.grouped_gemm_dswiglu_f64(cs["mode"], cs["a"], cs["sfa"], cs["b"], cs["sfb"], cs["ends"],
                                                c2, cs["prob"])
    assert np.array_equal(D1, D2) and np.array_equal(p1, p2)
    R1, Da, pa, _ = _run(cs, alpha=np.full(cs["G"], 1.0, np.float32))
    R3, Db, pb, _ = _run(cs, alpha=np.full(cs["G"], 3.0, np.float32))
    assert np.array_equal(R3, 9.0 * R1)
    np.testing.assert_allclose(Db, 9.0 * Da, rtol=1e-14)
    np.testing.assert_allclose(pb, 9.0 * pa, rtol=1e-14)


def test_groups_use_their_own_weights_and_rows_past_the_end_are_untouched():
    cs = _case("mxfp4", seed=5, counts=(4, 6, 0, 3))
    _, D, dp, written = _run(cs)
    # swapping experts 0 and 1 (weights, alpha, beta) moves the results of their rows only if the
    # rows are swapped too: compute expert 1's rows alone as a one-group problem
    lo, hi = int(cs["ends"][0]), int(cs["ends"][1])
    one = DG.grouped_gemm_dswiglu_f64(cs["mode"], cs["a"][lo:hi], cs["sfa"][lo:hi], cs["b"][1:2], cs["sfb"][1:2],
                                      np.array([hi - lo], np.int32), cs["c"][lo:hi], cs["prob"][lo:hi],
                                      cs["alpha"][1:2], cs["beta"][1:2])
    assert np.array_equal(one[1], D[lo:hi]) and np.array_equal(one[2], dp[lo:hi])
    end = int(cs["ends"][-1])
    assert not written[end:].any() and np.all(D[end:] == 0) and np.all(dp[end:] == 0)
    bits, dpf, wr = DG.grouped_gemm_dswiglu(cs["mode"], cs["a"], cs["sfa"], cs["b"], cs["sfb"], cs["ends"],
                                            cs["c"], cs["prob"], cs["alpha"], cs["beta"],
                                            out=np.full(D.shape, 0x7FC1, np.uint16))
    assert np.all(bits[~wr] == 0x7FC1)
    assert np.array_equal(bits[wr], F.bf16_round(D[wr]))
    # clamped ends: a decreasing end becomes an empty group
    ends2 = cs["ends"].copy()
    ends2[2] = 1
    _, D2, _, w2 = DG.grouped_gemm_dswiglu_f64(cs["mode"], cs["a"], cs["sfa"], cs["b"], cs["sfb"], ends2, cs["c"],
                                               cs["prob"], cs["alpha"], cs["beta"])
    assert np.array_equal(w2, written) and np.array_equal(D2, D)


def test_dprob_accumulates():
    cs = _case("mxfp8", seed=6)
    _, _, p0, written = _run(cs)
    prior = np.linspace(-1, 1, cs["M"]).astype(np.float32)
    _, _, p1, _ = _run(cs, dprob_in=prior)
    np.testing.assert_allclose(p1[written], p0[written] + prior[written].astype(np.float64), rtol=1e-14)
    assert np.array_equal(p1[~written], prior[~written].astype(np.float64))


def test_tolerance_hand_worked():
    """Two rows, K = 32: a = 2.0 at k = 0 (|a_m| = 2), b_n = 3.0 at k = 0 for
    every n (|b_n| = 3), alpha = 0.5: slack = 1e-3 * 2 * 3 * 0.25 = 1.5e-3;
    prob = 2; every input value 1.0.  Row 0, gate 0 (swish 0, sigmoid 1/2):
    input columns slack * 2 * |swish| = 0, gate columns
    slack * 2 * |1 * 0.5 * 1| = 1.5e-3, dprob term sum |swish * input| slack = 0.
    Row 1, gate 2.0: s = 1 / (1 + e^-2), swish = 2 s."""
    N, K = 32, 32
    a = np.zeros((2, K), np.uint8)
    a[:, 0] = 0x40                                      # 2.0
    b = np.zeros((1, N, K), np.uint8)
    b[0, :, 0] = 0x44                                   # 3.0
    sfa = np.full((2, 1), 127, np.uint8)
    sfb = np.full((1, N, 1), 127, np.uint8)
    c = np.zeros((2, 2 * N), np.float32)
    c[:, :32] = 1.0
    c[1, 32:] = 2.0
    tD, tP = DG.d_tolerance("mxfp8", a, sfa, b, sfb, np.array([2], np.int32), to_bf16_bits(c),
                            np.array([2.0, 2.0], np.float32), alpha=np.array([0.5], np.float32))
    assert np.all(tD[0, :32] == 0.0)
    np.testing.assert_allclose(tD[0, 32:], 1.5e-3, rtol=1e-12)
    assert tP[0] == 0.0
    s = 1.0 / (1.0 + math.exp(-2.0))
    np.testing.assert_allclose(tD[1, :32], 1.5e-3 * 2.0 * 2.0 * s, rtol=1e-12)
    np.testing.assert_allclose(tD[1, 32:], 1.5e-3 * 2.0 * s * (1.0 + 2.0 * (1.0 - s)), rtol=1e-12)
    np.testing.assert_allclose(tP[1], 32 * 1.5e-3 * 2.0 * s, rtol=1e-12)


# ---------------------------------------------------------------- row-quantised D
def test_quantised_d_hand_worked_block():
    """One row, N = 32: gate = 0 and input = 2 give d_input = 0 and
    d_gate = R * prob * 2 * 1/2 * (1 + 0) = R exactly (prob = 1), with
    R[n] = n + 1 from integer codes (A = [1, 1, 0, ...], B[n] = [x_n, y_n, 0, ...],
    x_n + y_n = n + 1).  The gate block's amax 32 gives the UE8M0 byte
    127 + 5 - 8 = 124 (scale 2^-3), so its codes are E4M3 of 8 (n + 1),
    worked out by hand: 8 -> 0x50, 16 -> 0x58, 24 -> 0x5C, 72 = 64 * 1.125 ->
    0x69, 136 (midway 128 / 144) -> 128 = 0x70, 152 (midway 144 / 160) -> 160 =
    0x72, 200 (midway 192 / 208) -> 192 = 0x74, 256 -> 0x78.  The all-zero
    input block takes byte 0 and +0 codes."""
    N, K = 32, 64
    rv = np.arange(1, N + 1)
    x = np.minimum(rv, 16)
    y = rv - x
    bv = np.zeros((1, N, K), np.int64)
    bv[0, :, 0], bv[0, :, 1] = x, y
    av = np.zeros((1, K), np.int64)
    av[0, :2] = 1
    a = _int_codes(av, "mxfp8")
    b = _int_codes(bv.reshape(N, K), "mxfp8").reshape(1, N, K)
    sfa = np.full((1, K // 32), 127, np.uint8)
    sfb = np.full((1, N, K // 32), 127, np.uint8)
    c = np.zeros((1, 2 * N), np.uint16)
    c[0, :N] = 0x4000                                   # input block: 2.0; gate block: +0
    q, sf, dp, written = DG.grouped_gemm_dswiglu_quant("mxfp8", a, sfa, b, sfb, np.array([1], np.int32), c,
                                                        np.ones(1, np.float32))
    assert written.all() and dp[0] == 0.0
    assert list(sf[0]) == [0, 124]
    assert np.all(q[0, :N] == 0)
    want = {1: 0x50, 2: 0x58, 3: 0x5C, 9: 0x69, 17: 0x70, 19: 0x72, 25: 0x74, 32: 0x78}
    for r, code in want.items():
        assert q[0, N + r - 1] == code, (r, hex(q[0, N + r - 1]))


def test_quantised_d_within_half_an_e4m3_step_and_untouched_rows():
    """Random case: every code times its scale is within half an E4M3 step
    of the BF16 D (relative 2^-4 for normal codes, 2^-10 absolute times the
    scale below 2^-6, 448 times the scale when saturated), and rows past the
    last end keep the caller's bytes."""
    cs = _case("mxfp8", seed=7)
    Dbits, _, written = DG.grouped_gemm_dswiglu(cs["mode"], cs["a"], cs["sfa"], cs["b"], cs["sfb"], cs["ends"],
                                                cs["c"], cs["prob"], cs["alpha"], cs["beta"])
    M, N2 = Dbits.shape
    q0 = np.full((M, N2), 0xA5, np.uint8)
    s0 = np.full((M, N2 // 32), 0x5A, np.uint8)
    q, sf, _, w2 = DG.grouped_gemm_dswiglu_quant(cs["mode"], cs["a"], cs["sfa"], cs["b"], cs["sfb"], cs["ends"],
                                                 cs["c"], cs["prob"], cs["alpha"], cs["beta"], q_out=q0, sf_out=s0)
    assert np.array_equal(w2, written)
    assert np.all(q[~written] == 0xA5) and np.all(sf[~written] == 0x5A)
    D = F.bf16_decode(Dbits[written])
    scale = np.exp2(sf[written].astype(np.float64) - 127).repeat(32, axis=1)
    deq = F.e4m3_decode(q[written]) * scale
    v = np.abs(D) / scale
    tol = np.where(v >= 2.0 ** -6, 2.0 ** -4 * np.abs(D), 2.0 ** -10 * scale)
    sat = v > 448
    assert np.all(np.abs(deq - D)[~sat] <= tol[~sat] * (1 + 1e-12))
    assert np.all(np.abs(deq[sat]) == 448 * scale[sat])
    assert np.all(np.sign(deq)[D != 0] == np.sign(D)[D != 0])
