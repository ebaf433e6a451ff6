"""Block-scaled GEMMs (oracle; test infrastructure only).

Definition (HALOps "GEMM" page, dense_gemm section: output = input @
weight^T + bias; cuDNN FE "Grouped GEMM + dGLU (SM100)", Step 1 equation:
the sum over k of dequantize(A) * dequantize(B)):

    out[m, n] = bf16_rne( alpha * sum_k deq(A)[m, k] * deq(B)[n, k] + bias[n] )

deq() multiplies each decoded code by its group scale (UE8M0 per 32 for the
MX modes, UE4M3 per 16 for NVFP4).  The sum is taken in float64 and rounded
once, directly to BF16.  Bias exists only in MXFP8 mode and alpha only in
NVFP4 mode (dense_gemm parameter list), so their order never matters.

Forms:
  * batch (batch_gemm section): out[b] = A[b] @ B[b]^T; batch item b uses
    only weight[b], bias[b], alpha[b].
  * grouped-contiguous (group_contiguous_gemm section; cuDNN FE Step 1):
    group g owns rows [end[g-1], end[g]) (end[-1] = 0) and uses weight[g].
    Rows at or beyond end[E-1] are not written.
  * grouped-masked (group_masked_gemm section): expert e owns rows
    e*Mmax + [0, min(count[e], Mmax)); all other rows are not written.
"""

import numpy as np

from . import formats as F
from .quant import dequant


def _mode_fmt(mode):
    return {"mxfp8": "mxfp8", "mxfp4": "mxfp4", "nvfp4": "nvfp4"}[mode]


def dense_f64(a_deq, b_deq, bias=None, alpha=None):
    """float64 result before the BF16 rounding: alpha * A @ B^T + bias."""
    acc = np.asarray(a_deq, dtype=np.float64) @ np.asarray(b_deq, dtype=np.float64).T
    if alpha is not None:
        acc = acc * np.float64(np.float32(alpha))
    if bias is not None:
        acc = acc + F.bf16_decode(bias)[None, :]
    return acc


def dense_gemm(mode, a, sfa, b, sfb, bias=None, alpha=None, out="bf16"):
    """Dense scaled GEMM -> BF16 bits [M, N] (out="fp16": binary16 bits).

    a: codes [M, K'] (K' = K for mxfp8, K/2 packed for the FP4 modes);
    sfa: [M, K/gs]; b, sfb likewise for [N, K]; bias: BF16 bits [N] or None;
    alpha: FP32 scalar or None."""
    fmt = _mode_fmt(mode)
    acc = dense_f64(dequant(a, sfa, fmt), dequant(b, sfb, fmt), bias, alpha)
    return F.fp16_round(acc) if out == "fp16" else F.bf16_round(acc)


def batch_gemm(mode, a, sfa, b, sfb, bias=None, alpha=None):
    """out[b] = dense_gemm(A[b], B[b]) with bias[b], alpha[b]."""
    B = a.shape[0]
    outs = []
    for i in range(B):
        outs.append(dense_gemm(mode, a[i], sfa[i], b[i], sfb[i],
                               None if bias is None else bias[i],
                               None if alpha is None else alpha[i]))
    return np.stack(outs) if outs else np.zeros((0,), np.uint16)


def group_contiguous_gemm(mode, a, sfa, b, sfb, group_end, bias=None, alpha=None, out=None):
    """Rows [end[g-1], end[g]) of A times weight[g]^T.  Returns (out, written)
    where written[m] says whether row m belongs to some group.  Rows that do
    not keep the value of ``out`` (zeros when out is None)."""
    M = a.shape[0]
    N = b.shape[1]
    res = np.zeros((M, N), np.uint16) if out is None else np.array(out, dtype=np.uint16, copy=True)
    written = np.zeros(M, dtype=bool)
    prev = 0
    for g, end in enumerate(np.asarray(group_end, dtype=np.int64)):
        # device-side ends cannot be validated by the host: each end is
        # clamped to [previous end, M], so groups never overlap or overrun.
        lo, hi = prev, int(min(max(int(end), prev), M))
        if hi > lo:
            res[lo:hi] = dense_gemm(mode, a[lo:hi], sfa[lo:hi], b[g], sfb[g],
                                    None if bias is None else bias[g],
                                    None if alpha is None else alpha[g])
            written[lo:hi] = True
        prev = hi
    return res, written


def group_masked_gemm(mode, a, sfa, b, sfb, masked_m, max_m, bias=None, alpha=None, out=None):
    """For expert e, rows e*max_m + [0, min(masked_m[e], max_m)) times
    weight[e]^T.  Returns (out, written) as group_contiguous_gemm does."""
    M = a.shape[0]
    N = b.shape[1]
    res = np.zeros((M, N), np.uint16) if out is None else np.array(out, dtype=np.uint16, copy=True)
    written = np.zeros(M, dtype=bool)
    for e, cnt in enumerate(np.asarray(masked_m, dtype=np.int64)):
        c = int(min(max(cnt, 0), max_m))
        lo = e * max_m
        if c > 0:
            res[lo:lo + c] = dense_gemm(mode, a[lo:lo + c], sfa[lo:lo + c], b[e], sfb[e],
                                        None if bias is None else bias[e],
                                        None if alpha is None else alpha[e])
            written[lo:lo + c] = True
    return res, written


def dense_gemm_rows_cols(mode, a, sfa, b, sfb, rows, cols, bias=None, alpha=None):
    """Selected outputs out[rows[i], cols[j]] of a dense GEMM, computed one
    row/column pair set at a time (for spot checks at sizes where the full
    product is too large for the CPU).  Returns BF16 bits [len(rows), len(cols)]."""
    fmt = _mode_fmt(mode)
    ad = dequant(a[rows], sfa[rows], fmt)
    bd = dequant(b[cols], sfb[cols], fmt)
    bias_sel = None if bias is None else np.asarray(bias)[cols]
    return F.bf16_round(dense_f64(ad, bd, bias_sel, alpha))


def tolerance(a_deq, b_deq, alpha=None):
    """Per-element absolute slack 1e-3 * ||a_m||_2 * ||b_n||_2 * |alpha| over
    the dequantised rows (the acceptance bound's absolute term)."""
    na = np.linalg.norm(np.asarray(a_deq, np.float64), axis=1)
    nb = np.linalg.norm(np.asarray(b_deq, np.float64), axis=1)
    s = 1.0 if alpha is None else abs(float(np.float32(alpha)))
    return 1e-3 * np.outer(na, nb) * s
