"""Backward grouped GEMM with the dSwiGLU epilogue (oracle; test
infrastructure only).

Source: cuDNN Frontend "Grouped GEMM + dGLU (SM100)" page --
  * "Tensors, layouts, and equation": for expert g, the compact GEMM
    gradient R_g = alpha_g^2 A_g B_g^T and the scaled forward activation
    X_g = beta_g C_g; X splits into alternating 32-wide blocks of the two GLU
    halves; with s = sigmoid(gate), dinput = R prob (gate s) and
    dgate = R prob input s (1 + gate (1 - s)).
  * "Step 1: Block-scaled grouped GEMM": ref[m, n] = alpha_g^2 times the sum
    over k of dequantize(A[m, k]) dequantize(B[n, k, g]) for the rows m of
    group g.
  * "Step 2: dGLU backward epilogue", "For dSwiGLU": swish = gate
    sigmoid(gate); dprob accumulates the sum of swish * input * ref over the
    row; ab = ref prob swish; dswiglu = ref prob input sigmoid(gate)
    (1 + gate (1 - sigmoid(gate))); [ab, dswiglu] are interleaved back in
    32-column blocks.
The steps below follow that order.  Everything is float64 from the exact
decoded codes, scales and the BF16 / FP32 inputs; the BF16 output is rounded
once (nearest even).

Readings (the page leaves these open or states them twice):
  1. Block order inside a 64-column pair of C and D: the input ("up") block
     first, then the gate block -- C holds "interleaved input/gate blocks"
     and D interleaves [ab, dswiglu] = [dinput, dgate] in the same places.
     R column n = 32 j + t pairs with C / D columns 64 j + t (input) and
     64 j + 32 + t (gate).
  2. Groups are rows [end[g-1], end[g]) of cumulative int32 ends (the page's
     padded_offsets, with any alignment, as the forward grouped GEMM takes
     them); ends are clamped to [previous end, rows]; rows at or past the
     last end are not written (neither D nor dprob).
  3. alpha and beta are per-group FP32 values (1 when absent); alpha enters
     squared, beta scales C before the derivative (X = beta C).
  4. dprob is accumulated: the call adds the row's sum to what dprob holds
     (the page's caller-zeroed dprob).
  5. D is BF16 (the page's default d_dtype), rounded once from the exact
     value.
  6. Row-quantised D (the page's optional output quantisation, "Step 3"):
     each row's 32-column groups of the BF16 D -- one input or gate block
     each -- take the MXFP8 rule of group_wise_quant (UE8M0 scale per 32,
     E4M3 codes).  The page's own FP8 recipe (a norm_const times the block
     amax times a reciprocal maximum, with 128x4 scale atoms) is not the
     OCP MX rule the rest of the library follows; the library's rule on the
     BF16 values is the reading taken, so the codes equal group_wise_quant
     applied to the BF16 D output.
"""

import numpy as np

from . import formats as F
from .quant import dequant, mx_quant_bf16

BLOCK = 32


def pair_columns(n):
    """(input columns, gate columns) of C / D for the n columns of R."""
    r = np.arange(n)
    j, t = r // BLOCK, r % BLOCK
    return 2 * BLOCK * j + t, 2 * BLOCK * j + BLOCK + t


def _groups(group_end, rows):
    prev = 0
    for g, end in enumerate(np.asarray(group_end, dtype=np.int64)):
        hi = int(min(max(int(end), prev), rows))
        yield g, prev, hi
        prev = hi


def grouped_gemm_dswiglu_f64(mode, a, sfa, b, sfb, group_end, c_bits, prob, alpha=None, beta=None,
                             dprob_in=None):
    """Returns (R [M, N], D [M, 2N], dprob [M], written [M]) in float64.

    a: codes [M, K'] + sfa; b: codes [G, N, K'] + sfb [G, N, K/gs] (mode
    "mxfp8" or "mxfp4"); c_bits: BF16 bits [M, 2N]; prob: FP32 [M];
    alpha, beta: FP32 [G] or None; dprob_in: the FP32 values dprob holds
    before the call (zeros when None)."""
    a = np.asarray(a)
    M = a.shape[0]
    G, N = b.shape[0], b.shape[1]
    R = np.zeros((M, N))
    D = np.zeros((M, 2 * N))
    dprob = np.zeros(M) if dprob_in is None else np.asarray(dprob_in, np.float32).astype(np.float64)
    written = np.zeros(M, dtype=bool)
    ic, gc = pair_columns(N)
    C = F.bf16_decode(c_bits)
    p = np.asarray(prob, np.float32).astype(np.float64)
    for g, lo, hi in _groups(group_end, M):
        if hi <= lo:
            continue
        al = 1.0 if alpha is None else float(np.float32(alpha[g]))
        be = 1.0 if beta is None else float(np.float32(beta[g]))
        # Step 1: ref = alpha^2 * sum_k dequantize(A) dequantize(B)
        ref = (al * al) * (dequant(a[lo:hi], sfa[lo:hi], mode) @ dequant(b[g], sfb[g], mode).T)
        # Step 2: the two halves of X = beta * C, block by block
        X = be * C[lo:hi]
        inp, gate = X[:, ic], X[:, gc]
        with np.errstate(over="ignore"):
            sig = 1.0 / (1.0 + np.exp(-gate))
        swish = gate * sig
        pr = p[lo:hi, None]
        dprob[lo:hi] += np.sum(swish * inp * ref, axis=1)
        ab = ref * pr * swish
        dsw = ref * pr * inp * sig * (1.0 + gate * (1.0 - sig))
        D[lo:hi, ic] = ab
        D[lo:hi, gc] = dsw
        R[lo:hi] = ref
        written[lo:hi] = True
    return R, D, dprob, written


def grouped_gemm_dswiglu(mode, a, sfa, b, sfb, group_end, c_bits, prob, alpha=None, beta=None,
                         dprob_in=None, out=None):
    """BF16 D bits [M, 2N] (rows not written keep ``out``, zeros when None),
    float64 dprob [M] and the written-row mask."""
    _, D, dprob, written = grouped_gemm_dswiglu_f64(mode, a, sfa, b, sfb, group_end, c_bits, prob,
                                                   alpha, beta, dprob_in)
    M = D.shape[0]
    res = np.zeros(D.shape, np.uint16) if out is None else np.array(out, dtype=np.uint16, copy=True)
    res[written] = F.bf16_round(D[written])
    return res, dprob, written


def d_tolerance(mode, a, sfa, b, sfb, group_end, c_bits, prob, alpha=None, beta=None):
    """Absolute term of the acceptance bound of D [M, 2N] and of dprob [M].

    The GEMM acceptance bound's absolute term, 1e-3 ||a_m|| ||b_n|| alpha^2
    (dequantised rows), carried through the epilogue's factor of R: for the
    input column prob * swish, for the gate column
    prob * input * s * (1 + gate (1 - s)); for dprob the sum over the row of
    |swish * input| times that term."""
    a = np.asarray(a)
    M = a.shape[0]
    N = b.shape[1]
    tD = np.zeros((M, 2 * N))
    tP = np.zeros(M)
    ic, gc = pair_columns(N)
    C = F.bf16_decode(c_bits)
    p = np.asarray(prob, np.float32).astype(np.float64)
    for g, lo, hi in _groups(group_end, M):
        if hi <= lo:
            continue
        al = 1.0 if alpha is None else float(np.float32(alpha[g]))
        be = 1.0 if beta is None else float(np.float32(beta[g]))
        na = np.linalg.norm(dequant(a[lo:hi], sfa[lo:hi], mode), axis=1)
        nb = np.linalg.norm(dequant(b[g], sfb[g], mode), axis=1)
        slack = 1e-3 * np.outer(na, nb) * al * al
        X = be * C[lo:hi]
        inp, gate = X[:, ic], X[:, gc]
        with np.errstate(over="ignore"):
            sig = 1.0 / (1.0 + np.exp(-gate))
        swish = gate * sig
        pr = np.abs(p[lo:hi, None])
        tD[lo:hi, ic] = slack * pr * np.abs(swish)
        tD[lo:hi, gc] = slack * pr * np.abs(inp * sig * (1.0 + gate * (1.0 - sig)))
        tP[lo:hi] = np.sum(slack * np.abs(swish * inp), axis=1)
    return tD, tP


def grouped_gemm_dswiglu_quant(mode, a, sfa, b, sfb, group_end, c_bits, prob, alpha=None, beta=None,
                               dprob_in=None, q_out=None, sf_out=None):
    """Row-quantised D (reading 6): MXFP8 codes [M, 2N] u8 and UE8M0 scales
    [M, 2N / 32] u8 of the BF16 D of grouped_gemm_dswiglu, on the written
    rows (others keep ``q_out`` / ``sf_out``, zeros when None); float64
    dprob [M]; the written-row mask."""
    D, dprob, written = grouped_gemm_dswiglu(mode, a, sfa, b, sfb, group_end, c_bits, prob, alpha, beta,
                                             dprob_in)
    M, N2 = D.shape
    q = np.zeros((M, N2), np.uint8) if q_out is None else np.array(q_out, dtype=np.uint8, copy=True)
    sf = np.zeros((M, N2 // BLOCK), np.uint8) if sf_out is None else np.array(sf_out, dtype=np.uint8, copy=True)
    if written.any():
        qw, sw = mx_quant_bf16(D[written], "mxfp8")
        q[written] = qw
        sf[written] = sw
    return q, sf, dprob, written
