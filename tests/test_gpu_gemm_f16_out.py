"""GPU parity of the GEMMs with binary16 (FP16) output (HQ_OUT_FP16; the
flashrt/fp4-gemm page's *_fp16 GEMMs): every kernel path writes the FP32 result
(+ bias, x alpha) rounded once to FP16.

* Integer-coded inputs: exact sums, so the output must equal the oracle's
  one-rounding FP64 -> FP16 bit for bit -- including sums beyond 65504, which
  must become Inf -- on the direct, tiled, K-split and tail-split paths.
* Random inputs: the acceptance bound against the oracle (FP16 output), dense,
  batch with bias, grouped-contiguous, grouped-masked (untouched padded rows)
  and the discrete-weights call.
"""
import numpy as np
import pytest
import torch

import fp4_gemm_moe_amd as hq
import synth
from oracle import formats as F
from oracle import gemm as G
from tests import _gpu as U
from tests.test_gpu_gemm import _int_operand, _quant

pytestmark = pytest.mark.gpu

SENTINEL = 0x7E01          # an FP16 NaN pattern no kernel writes


def _host16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _assert_close16(got, want, a_deq, b_deq, alpha=None, what=""):
    out, ref = F.fp16_decode(got), F.fp16_decode(want)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - ref)
    bad = err > 2.0 ** -7 * np.abs(ref) + G.tolerance(a_deq, b_deq, alpha)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of bound"
    nref = np.linalg.norm(ref)
    if nref > 0:
        assert np.linalg.norm(out - ref) / nref <= 2e-3, what


def _dense16(mode, a, sfa, b, sfb, m, n, k, dev, bias=None, alpha=None, cu_limit=0):
    """With the workspace the shape asks for, so K-split shapes split."""
    out = torch.full((m, n), SENTINEL, dtype=torch.int16, device=dev).view(torch.float16)
    hq.hq_dense_gemm(mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev), U.dev_u8(sfb, dev),
                     out, bias=None if bias is None else U.dev_bf16(bias, dev),
                     alpha=None if alpha is None else torch.tensor([alpha], dtype=torch.float32, device=dev),
                     cu_limit=cu_limit, workspace=hq.gemm_workspace(mode, m, n, k, cu_limit=cu_limit, device=dev))
    torch.cuda.synchronize()
    return _host16(out)


# (m, n, k, cu_limit): direct (M <= 16), tiled, K-split (few tiles, long K),
# tail split (last round at most half full, long K, with a CU limit)
INT_SHAPES = [(5, 520, 512, 0), (300, 136, 1024, 0), (300, 520, 8704, 0), (520, 1544, 6144, 16)]


# the tail-split shape is an MXFP8 case (its K steps)
INT_CASES = [(mode, s) for s in INT_SHAPES[:3] for mode in ("mxfp8", "mxfp4", "nvfp4")] + [("mxfp8", INT_SHAPES[3])]


@pytest.mark.parametrize("mode,shape", INT_CASES, ids=lambda c: c if isinstance(c, str) else f"{c[0]}x{c[1]}x{c[2]}-cu{c[3]}")
def test_fp16_out_integer_exact(mode, shape):
    m, n, k, cus = shape
    dev = U.require_gpu()
    U.banner(f"fp16-out int-exact {mode} {m}x{n}x{k} cu={cus}")
    rng = np.random.default_rng(m + n + k)
    av, a, sfa = _int_operand(rng, m, k, mode, [-1, 0, 1])
    bv, b, sfb = _int_operand(rng, n, k, mode, [-2, -1, 0, 1, 2])
    got = _dense16(mode, a, sfa, b, sfb, m, n, k, dev, alpha=1.0 if mode == "nvfp4" else None, cu_limit=cus)
    want = F.fp16_round((av @ bv.T).astype(np.float64))
    assert np.array_equal(got, want), f"{np.sum(got != want)} of {got.size} differ"


def test_fp16_out_overflows_to_inf():
    """Sums beyond 65504 (scale 2^10 on A) round to +-Inf, the rest exactly."""
    dev = U.require_gpu()
    m, n, k = 64, 64, 512
    rng = np.random.default_rng(9)
    av, a, sfa = _int_operand(rng, m, k, "mxfp8", [-2, -1, 0, 1, 2])
    bv, b, sfb = _int_operand(rng, n, k, "mxfp8", [-2, -1, 0, 1, 2])
    sfa[:] = 127 + 10
    got = _dense16("mxfp8", a, sfa, b, sfb, m, n, k, dev)
    want = F.fp16_round((av @ bv.T).astype(np.float64) * 1024.0)
    assert (np.abs(F.fp16_decode(want)) == np.inf).any(), "the case must overflow somewhere"
    assert np.array_equal(got, want), f"{np.sum(got != want)} of {got.size} differ"


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
def test_fp16_out_dense_random(mode):
    dev = U.require_gpu()
    rng = np.random.default_rng(44)
    for (m, n, k) in [(3, 136, 512), (200, 264, 1024)]:
        a, sfa, ga = _quant(synth.normal_bf16(rng, (m, k)), mode)
        b, sfb, gb = _quant(synth.normal_bf16(rng, (n, k), 0.05), mode)
        alpha = None if ga is None else np.float32(ga * gb)
        bias = synth.normal_bf16(rng, (n,), 0.1) if mode == "mxfp8" else None
        got = _dense16(mode, a, sfa, b, sfb, m, n, k, dev, bias=bias, alpha=alpha)
        want = G.dense_gemm(mode, a, sfa, b, sfb, bias, alpha, out="fp16")
        _assert_close16(got, want, U.deq(mode, a, sfa), U.deq(mode, b, sfb), alpha, f"dense {mode} {m}x{n}x{k}")


def test_fp16_out_batch_grouped_masked_discrete():
    dev = U.require_gpu()
    rng = np.random.default_rng(45)
    mode, K, N = "mxfp8", 512, 136
    # batch with bias
    Bn, m = 3, 40
    a, sfa, _ = _quant(synth.normal_bf16(rng, (Bn * m, K)), mode)
    b, sfb, _ = _quant(synth.normal_bf16(rng, (Bn * N, K), 0.05), mode)
    bias = synth.normal_bf16(rng, (Bn, N), 0.1)
    out = torch.empty(Bn, m, N, dtype=torch.float16, device=dev)
    hq.hq_batch_gemm(mode, U.dev_u8(a, dev).view(Bn, m, K), U.dev_u8(sfa, dev).view(Bn, m, -1),
                     U.dev_u8(b, dev).view(Bn, N, K), U.dev_u8(sfb, dev).view(Bn, N, -1), out,
                     bias=U.dev_bf16(bias, dev))
    torch.cuda.synchronize()
    got = _host16(out)
    for i in range(Bn):
        rs, ns = slice(i * m, (i + 1) * m), slice(i * N, (i + 1) * N)
        want = G.dense_gemm(mode, a[rs], sfa[rs], b[ns], sfb[ns], bias[i], out="fp16")
        _assert_close16(got[i], want, U.deq(mode, a[rs], sfa[rs]), U.deq(mode, b[ns], sfb[ns]), what=f"batch {i}")
    # grouped-contiguous, packed and discrete weights
    counts = np.array([70, 0, 300], np.int32)
    ends = np.cumsum(counts).astype(np.int32)
    R = int(ends[-1])
    a, sfa, _ = _quant(synth.normal_bf16(rng, (R, K)), mode)
    b, sfb, _ = _quant(synth.normal_bf16(rng, (3 * N, K), 0.05), mode)
    bq, bs = b.reshape(3, N, K), sfb.reshape(3, N, -1)
    out = torch.empty(R, N, dtype=torch.float16, device=dev)
    hq.hq_group_contiguous_gemm(mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(bq, dev), U.dev_u8(bs, dev),
                                U.dev_i32(ends, dev), out)
    out2 = torch.empty(R, N, dtype=torch.float16, device=dev)
    keep = hq.hq_group_contiguous_gemm_ptr_array(mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev),
                                                 [U.dev_u8(bq[g], dev) for g in range(3)],
                                                 [U.dev_u8(bs[g], dev) for g in range(3)],
                                                 U.dev_i32(ends, dev), out2, N)
    torch.cuda.synchronize()
    del keep
    got = _host16(out)
    assert np.array_equal(got, _host16(out2)), "discrete weights differ from packed"
    lo = 0
    for g in range(3):
        hi = int(ends[g])
        if hi > lo:
            want = G.dense_gemm(mode, a[lo:hi], sfa[lo:hi], bq[g], bs[g], out="fp16")
            _assert_close16(got[lo:hi], want, U.deq(mode, a[lo:hi], sfa[lo:hi]), U.deq(mode, bq[g], bs[g]),
                            what=f"group {g}")
        lo = hi
    # grouped-masked: padded rows keep the sentinel
    E, Mmax = 3, 64
    cnt = np.array([64, 0, 9], np.int32)
    a, sfa, _ = _quant(synth.normal_bf16(rng, (E * Mmax, K)), mode)
    out = torch.full((E * Mmax, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.float16)
    hq.hq_group_masked_gemm(mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(bq, dev), U.dev_u8(bs, dev),
                            U.dev_i32(cnt, dev), out, Mmax)
    torch.cuda.synchronize()
    got = _host16(out)
    for e in range(E):
        rows = slice(e * Mmax, e * Mmax + int(cnt[e]))
        if cnt[e] > 0:
            want = G.dense_gemm(mode, a[rows], sfa[rows], bq[e], bs[e], out="fp16")
            _assert_close16(got[rows], want, U.deq(mode, a[rows], sfa[rows]), U.deq(mode, bq[e], bs[e]),
                            what=f"masked {e}")
        assert (got[e * Mmax + int(cnt[e]):(e + 1) * Mmax] == SENTINEL).all(), f"expert {e}: padded rows written"
