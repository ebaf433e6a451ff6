"""GPU parity of hq_group_contiguous_gemm_dswiglu (the backward block-scaled
grouped GEMM with the dSwiGLU epilogue; cuDNN FE "Grouped GEMM + dGLU
(SM100)", Steps 1 and 2) against oracle.dglu.

* Integer-exact: small-integer codes with unit scales (R exact in FP32),
  alpha a power of two, the gate half of X = beta C at 64 (sigmoid is exactly
  1 in FP32 and rounds to 1 from float64), input values in {-1, 1/2, 1, 2}, prob
  1: D = [64 R, R input] and dprob = 64 sum R input are exact, so the device's
  bits must equal the oracle's -- this pins the R lane layout, the block
  interleave of C and D, the alpha / beta per group and the dprob reduction.
* Random inputs (MXFP8 and MXFP4, both scale-load layouts, ragged and empty
  groups, a partial n-tile): per element
  |D - D_ref| <= 2^-7 |D_ref| + t_D (t_D: the GEMM bound's absolute term
  carried through the epilogue factor), relative Frobenius error <= 2e-3;
  dprob within 2^-7 sum |swish input R| + t_P + an FP32 summation term.
* Rows past the last end keep their sentinel (d) and value (dprob); dprob
  accumulates onto what it held.
* The full backward MoE shape (32 experts, 65536 routed rows, K = 4096,
  N = 1536): sampled rows of four experts against the oracle.
* The row-quantised form (hq_group_contiguous_gemm_dswiglu_quant): its codes
  and scales equal the MXFP8 quantisation of the BF16 call's D, bit for bit,
  on every written row (the oracle's too where D is integer-exact); rows past
  the last end keep their sentinels; dprob within the same bound.
"""
import numpy as np
import pytest
import torch

import fp4_gemm_moe_amd as hq
import synth
from oracle import dglu as DG
from oracle import formats as F
from oracle import quant as Q
from tests import _gpu as U
from tests.test_oracle_gemm import INT_E2M1, INT_E4M3

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1


def _int_codes(vals, mode):
    table = INT_E4M3 if mode == "mxfp8" else INT_E2M1
    lut = np.zeros(int(max(table)) + 1, np.uint8)
    for v, c in table.items():
        lut[int(v)] = c
    sign = 0x80 if mode == "mxfp8" else 0x8
    c = lut[np.abs(vals)] | np.where(vals < 0, sign, 0).astype(np.uint8)
    return c if mode == "mxfp8" else F.pack_nibbles(c)


def _run(mode, a, sfa, b, sfb, ends, c, prob, alpha, beta, dprob0, dev, cu_limit=0):
    M, N = c.shape[0], b.shape[1]
    d = torch.full((M, 2 * N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    dprob = torch.from_numpy(np.asarray(dprob0, np.float32)).to(dev)
    hq.hq_group_contiguous_gemm_dswiglu(
        mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev), U.dev_u8(sfb, dev), U.dev_i32(ends, dev),
        U.dev_bf16(c, dev), torch.from_numpy(np.asarray(prob, np.float32)).to(dev), dprob, d,
        alpha=None if alpha is None else torch.from_numpy(np.asarray(alpha, np.float32)).to(dev),
        beta=None if beta is None else torch.from_numpy(np.asarray(beta, np.float32)).to(dev), cu_limit=cu_limit)
    torch.cuda.synchronize()
    return U.host_bits(d), dprob.cpu().numpy()


def _run_q(mode, a, sfa, b, sfb, ends, c, prob, alpha, beta, dprob0, dev):
    M, N = c.shape[0], b.shape[1]
    dq = torch.full((M, 2 * N), 0xA5, dtype=torch.uint8, device=dev)
    dsf = torch.full((M, 2 * N // 32), 0x5A, dtype=torch.uint8, device=dev)
    dprob = torch.from_numpy(np.asarray(dprob0, np.float32)).to(dev)
    hq.hq_group_contiguous_gemm_dswiglu_quant(
        mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev), U.dev_u8(sfb, dev), U.dev_i32(ends, dev),
        U.dev_bf16(c, dev), torch.from_numpy(np.asarray(prob, np.float32)).to(dev), dprob, dq, dsf,
        alpha=None if alpha is None else torch.from_numpy(np.asarray(alpha, np.float32)).to(dev),
        beta=None if beta is None else torch.from_numpy(np.asarray(beta, np.float32)).to(dev))
    torch.cuda.synchronize()
    return U.host_u8(dq), U.host_u8(dsf), dprob.cpu().numpy()


def _check_quantised(d_bits, q, sf, written, what):
    """Codes / scales of the written rows = MXFP8 quantisation of the BF16 D
    (bit for bit); the other rows keep the sentinels."""
    wq, ws = Q.mx_quant_bf16(d_bits[written], "mxfp8")
    assert np.array_equal(q[written], wq), f"{what}: {np.sum(q[written] != wq)} codes differ"
    assert np.array_equal(sf[written], ws), f"{what}: {np.sum(sf[written] != ws)} scales differ"
    assert np.all(q[~written] == 0xA5) and np.all(sf[~written] == 0x5A), f"{what}: rows past the end written"


INT_CASES = [("mxfp8", (40, 0, 300, 17), 96, 512), ("mxfp8", (256, 33), 320, 384),
             ("mxfp4", (40, 0, 300, 17), 96, 512), ("mxfp4", (129, 1), 64, 768)]


@pytest.mark.parametrize("case", INT_CASES, ids=lambda c: f"{c[0]}-N{c[2]}-K{c[3]}")
def test_dswiglu_integer_exact(case):
    mode, counts, N, K = case
    dev = U.require_gpu()
    U.banner(f"dswiglu int-exact {mode} counts={counts} N={N} K={K}")
    rng = np.random.default_rng(N + K)
    G = len(counts)
    ends = np.cumsum(counts).astype(np.int32)
    M = int(ends[-1]) + 7
    av = rng.choice(np.array([-1, 0, 1]), (M, K))
    bv = rng.choice(np.array([-1, 0, 1]), (G * N, K))
    a, b = _int_codes(av, mode), _int_codes(bv, mode).reshape(G, N, -1)
    sfa = np.full((M, K // 32), 127, np.uint8)
    sfb = np.full((G, N, K // 32), 127, np.uint8)
    alpha = np.array([2.0, 0.5, 1.0, 4.0][:G], np.float32)
    beta = np.array([0.5, 1.0, 2.0, 0.25][:G], np.float32)
    # X = beta C: gate 64, input in {-1, 1/2, 1, 2}
    c = np.zeros((M, 2 * N), np.float32)
    ic, gc = DG.pair_columns(N)
    rb = np.ones(M, np.float32)
    prev = 0
    for g, e in enumerate(ends):
        rb[prev:e] = beta[g]
        prev = e
    c[:, gc] = 64.0 / rb[:, None]
    c[:, ic] = rng.choice(np.array([-1.0, 0.5, 1.0, 2.0], np.float32), (M, N)) / rb[:, None]
    cb = synth.to_bf16_bits(c)
    prob = np.ones(M, np.float32)
    dprob0 = np.zeros(M, np.float32)
    got, gp = _run(mode, a, sfa, b, sfb, ends, cb, prob, alpha, beta, dprob0, dev)
    want, wp, written = DG.grouped_gemm_dswiglu(mode, a, sfa, b, sfb, ends, cb, prob, alpha, beta,
                                                out=np.full((M, 2 * N), SENTINEL, np.uint16))
    assert np.array_equal(got, want), f"{np.sum(got != want)} of {got.size} D values differ"
    assert np.array_equal(gp[written].astype(np.float64), wp[written]), "dprob differs"
    assert np.all(gp[~written] == 0.0)
    # the row-quantised form: the oracle's codes and scales, exactly
    q, sf, gp2 = _run_q(mode, a, sfa, b, sfb, ends, cb, prob, alpha, beta, dprob0, dev)
    oq, osf, _, _ = DG.grouped_gemm_dswiglu_quant(mode, a, sfa, b, sfb, ends, cb, prob, alpha, beta)
    assert np.array_equal(q[written], oq[written]) and np.array_equal(sf[written], osf[written]), \
        "row-quantised D differs from the oracle"
    _check_quantised(got, q, sf, written, "int-exact")
    assert np.array_equal(gp2[written].astype(np.float64), wp[written]), "dprob of the quantised form differs"


def _random_case(mode, counts, N, K, seed, with_ab=True):
    rng = np.random.default_rng(seed)
    G = len(counts)
    ends = np.cumsum(counts).astype(np.int32)
    M = int(ends[-1]) + 5
    x = synth.normal_bf16(rng, (M, K))
    w = synth.normal_bf16(rng, (G * N, K), 0.05)
    a, sfa = Q.mx_quant_bf16(x, mode)
    b, sfb = Q.mx_quant_bf16(w, mode)
    b, sfb = b.reshape(G, N, -1), sfb.reshape(G, N, -1)
    c = synth.normal_bf16(rng, (M, 2 * N), 2.0)
    prob = rng.random(M).astype(np.float32)
    alpha = rng.uniform(0.5, 2.0, G).astype(np.float32) if with_ab else None
    beta = rng.uniform(0.5, 1.5, G).astype(np.float32) if with_ab else None
    return a, sfa, b, sfb, ends, c, prob, alpha, beta, M


def _check(mode, a, sfa, b, sfb, ends, c, prob, alpha, beta, dprob0, got, gp, what, rows=None):
    """got / gp: the device's D bits and dprob for `rows` (all rows if None)."""
    want, wp, written = DG.grouped_gemm_dswiglu(mode, a, sfa, b, sfb, ends, c, prob, alpha, beta, dprob_in=dprob0)
    tD, tP = DG.d_tolerance(mode, a, sfa, b, sfb, ends, c, prob, alpha, beta)
    sel = written if rows is None else rows
    gD, wD = F.bf16_decode(got), F.bf16_decode(want[sel])
    assert np.all(np.isfinite(gD)), f"{what}: non-finite D"
    bad = np.abs(gD - wD) > 2.0 ** -7 * np.abs(wD) + tD[sel]
    assert not bad.any(), f"{what}: {bad.sum()} D values out of bound"
    nref = np.linalg.norm(wD)
    if nref > 0:
        assert np.linalg.norm(gD - wD) / nref <= 2e-3, f"{what}: relative Frobenius error of D"
    # dprob: each term within its own bound, summed; plus FP32 summation over the row
    R, D64, _, _ = DG.grouped_gemm_dswiglu_f64(mode, a, sfa, b, sfb, ends, c, prob, alpha, beta)
    ic, gc = DG.pair_columns(b.shape[1])
    absterm = np.zeros(len(prob))
    for g, lo, hi in DG._groups(ends, len(prob)):
        if hi > lo:
            be = 1.0 if beta is None else float(beta[g])
            X = be * F.bf16_decode(c[lo:hi])
            with np.errstate(over="ignore"):
                sg = 1.0 / (1.0 + np.exp(-X[:, gc]))
            absterm[lo:hi] = np.sum(np.abs(X[:, gc] * sg * X[:, ic] * R[lo:hi]), axis=1)
    n_terms = b.shape[1]
    pbound = 2.0 ** -7 * absterm + tP + n_terms * 2.0 ** -22 * absterm + 1e-30
    pb = np.abs(gp.astype(np.float64) - wp[sel]) > pbound[sel]
    assert not pb.any(), f"{what}: {pb.sum()} dprob values out of bound"


RANDOM_CASES = [("mxfp8", (40, 0, 300, 17), 96, 512), ("mxfp8", (17, 129, 0, 5), 288, 384),
                ("mxfp4", (40, 0, 300, 17), 96, 512), ("mxfp4", (200, 60), 160, 768)]


@pytest.mark.parametrize("case", RANDOM_CASES, ids=lambda c: f"{c[0]}-N{c[2]}-K{c[3]}")
def test_dswiglu_random_against_oracle(case):
    mode, counts, N, K = case
    dev = U.require_gpu()
    U.banner(f"dswiglu random {mode} counts={counts} N={N} K={K}")
    a, sfa, b, sfb, ends, c, prob, alpha, beta, M = _random_case(mode, counts, N, K, seed=N * 7 + K)
    dprob0 = np.linspace(-0.5, 0.5, M).astype(np.float32)       # accumulates onto this
    got, gp = _run(mode, a, sfa, b, sfb, ends, c, prob, alpha, beta, dprob0, dev)
    written = np.zeros(M, bool)
    written[:int(ends[-1])] = True
    assert np.all(got[~written] == SENTINEL), "rows past the last end were written"
    assert np.array_equal(gp[~written], dprob0[~written]), "dprob past the last end changed"
    _check(mode, a, sfa, b, sfb, ends, c, prob, alpha, beta, dprob0, got[written], gp[written],
           f"{mode} N{N} K{K}")
    q, sf, gp2 = _run_q(mode, a, sfa, b, sfb, ends, c, prob, alpha, beta, dprob0, dev)
    _check_quantised(got, q, sf, written, f"{mode} N{N} K{K} quantised")
    _check(mode, a, sfa, b, sfb, ends, c, prob, alpha, beta, dprob0, got[written], gp2[written],
           f"{mode} N{N} K{K} (dprob of the quantised form)")


def test_dswiglu_without_alpha_beta():
    dev = U.require_gpu()
    mode, counts, N, K = "mxfp8", (64, 100), 64, 256
    U.banner("dswiglu alpha = beta = NULL")
    a, sfa, b, sfb, ends, c, prob, _, _, M = _random_case(mode, counts, N, K, seed=3, with_ab=False)
    dprob0 = np.zeros(M, np.float32)
    got, gp = _run(mode, a, sfa, b, sfb, ends, c, prob, None, None, dprob0, dev)
    w = np.zeros(M, bool)
    w[:int(ends[-1])] = True
    _check(mode, a, sfa, b, sfb, ends, c, prob, None, None, dprob0, got[w], gp[w], "no alpha / beta")


def test_dswiglu_rejects_what_it_cannot_run():
    dev = U.require_gpu()
    lib = hq.load()
    z = torch.zeros(4096, dtype=torch.uint8, device=dev)
    f = torch.zeros(64, dtype=torch.float32, device=dev)
    P = hq._p
    st = hq._stream(z)
    args = lambda mode, n, k: (st, mode, P(z), P(z), P(z), P(z), P(z), 1, P(z), None, None, P(f), P(f), P(z), 8,
                               n, k, 0)
    assert lib.hq_group_contiguous_gemm_dswiglu(*args(2, 64, 512)) == -4      # NVFP4
    assert lib.hq_group_contiguous_gemm_dswiglu(*args(0, 48, 512)) == -2      # n % 32
    assert lib.hq_group_contiguous_gemm_dswiglu(*args(0, 64, 128)) == -2      # one K step
    assert lib.hq_group_contiguous_gemm_dswiglu(*args(1, 64, 256)) == -2      # one FP4 K step
    qargs = lambda mode, n, k, dq, dsf: (st, mode, P(z), P(z), P(z), P(z), P(z), 1, P(z), None, None, P(f), P(f),
                                         dq, dsf, 8, n, k, 0)
    fq = lib.hq_group_contiguous_gemm_dswiglu_quant
    assert fq(*qargs(2, 64, 512, P(z), P(z))) == -4          # NVFP4
    assert fq(*qargs(0, 64, 512, None, P(z))) == -1          # no dq
    assert fq(*qargs(0, 64, 512, P(z), None)) == -1          # no dsf
    assert fq(*qargs(0, 48, 512, P(z), P(z))) == -2          # n % 32


def test_dswiglu_moe_backward_full_size_sampled():
    """The backward of the MoE down projection's input: 32 experts, the 65536
    routed rows padded to 128 per expert, upstream gradient [R, 4096] N(0,1)
    as A, weights [32, 1536, 4096] N(0, 0.02) as B, forward activations C
    [R, 3072] N(0, 1), prob U(0, 1): sampled rows of four experts."""
    dev = U.require_gpu()
    U.banner("dswiglu MoE backward E=32 R=67840 K=4096 N=1536 (full size, sampled)")
    d = synth.moe_dglu_backward(threads=16)
    counts, ends, starts = d["counts"], d["group_end"], d["starts"]
    R, K, N, E = int(ends[-1]), d["K"], d["N"], len(counts)
    qa, sa, _ = hq.quantize(U.dev_bf16(d["a"], dev), "mxfp8")
    wbits = d["b"].reshape(E * N, K)
    qw, sw, _ = hq.quantize(U.dev_bf16(wbits, dev), "mxfp8")
    c = U.dev_bf16(d["c"], dev)
    prob = torch.from_numpy(d["prob"]).to(dev)
    alpha = torch.from_numpy(d["alpha"]).to(dev)
    beta = torch.from_numpy(d["beta"]).to(dev)
    dprob = torch.zeros(R, dtype=torch.float32, device=dev)
    out = torch.full((R, 2 * N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    hq.hq_group_contiguous_gemm_dswiglu("mxfp8", qa, sa, qw.view(E, N, K), sw.view(E, N, K // 32),
                                        U.dev_i32(ends, dev), c, prob, dprob, out, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    rng = np.random.default_rng(66)
    experts = sorted({0, E - 1, int(np.argmin(counts)), int(np.argmax(counts))})
    for g in experts:
        lo, c_ = int(starts[g]), int(counts[g])
        local = sorted({0, c_ - 1, min(255, c_ - 1), min(256, c_ - 1)} | {int(v) for v in rng.integers(0, c_, 4)})
        rows = np.array([lo + v for v in local], np.int64)
        rt = torch.from_numpy(rows).to(dev)
        ac, asc = Q.mx_quant_bf16(d["a"][rows], "mxfp8")
        wc, wsc = Q.mx_quant_bf16(wbits[g * N:(g + 1) * N], "mxfp8")
        assert np.array_equal(U.host_u8(qa[rt]), ac), f"expert {g}: A codes"
        one = np.array([len(rows)], np.int32)
        _check("mxfp8", ac, asc, wc[None], wsc[None], one, d["c"][rows], d["prob"][rows], d["alpha"][g:g + 1],
               d["beta"][g:g + 1], np.zeros(len(rows), np.float32), U.host_bits(out[rt]), dprob[rt].cpu().numpy(),
               f"expert {g} (count {c_})")
    # the row-quantised form at full size: codes / scales of every sampled row
    # = MXFP8 quantisation of the BF16 call's D
    dq = torch.full((R, 2 * N), 0xA5, dtype=torch.uint8, device=dev)
    dsf = torch.full((R, 2 * N // 32), 0x5A, dtype=torch.uint8, device=dev)
    hq.hq_group_contiguous_gemm_dswiglu_quant("mxfp8", qa, sa, qw.view(E, N, K), sw.view(E, N, K // 32),
                                              U.dev_i32(ends, dev), c, prob, torch.zeros_like(dprob), dq, dsf,
                                              alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.integers(0, R, 64), [0, R - 1], starts[np.asarray(counts) > 0]]))
    rt = torch.from_numpy(rows.astype(np.int64)).to(dev)
    valid = np.zeros(R, bool)
    for g in range(E):
        valid[int(starts[g]):int(ends[g])] = True      # padded rows are rows of their group too
    sel = valid[rows]
    _check_quantised(U.host_bits(out[rt])[sel], U.host_u8(dq[rt])[sel], U.host_u8(dsf[rt])[sel],
                     np.ones(int(sel.sum()), bool), "full size, quantised")
    del qa, qw, c, out, dq, dsf
    torch.cuda.empty_cache()
