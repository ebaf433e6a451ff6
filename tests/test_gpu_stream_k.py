"""GPU parity of the stream-K form of the dense GEMM (hq_dense_gemm_ws).

A dense launch whose tiles make one round of more than a third of the grid
(and at most all of it) deals the K units of all tiles out in equal runs, one
per workgroup, where that saves enough matrix time (long K, or NVFP4's slower
steps).  The workgroups form 8 groups (every eighth one), each taking an
eighth of the tiles; a tile's pieces sit in two or more workgroups of its
group, which hand their FP32 partial tiles to the tile's last piece.  A CU
limit sets the grid at these sizes:
  * MXFP8 256 x 4096 x 6144 on 32 CUs: 16 tiles of 12 units of 4 steps, 2 per
    group of 4 workgroups, runs of 6 units (each tile in two pieces);
  * MXFP8 256 x 2816 x 6144 on 32 CUs: 11 tiles, so five groups hold one tile
    over their 4 workgroups (four pieces, three partials per tile) and three
    hold two;
  * MXFP4 300 x 2048 x 16384 (a ragged second m-tile; 32 units of 2 steps)
    on 32 CUs, and NVFP4 256 x 2552 x 8192 (a partial last n-tile; 16 units of
    2 steps) on 24 CUs (groups of 3 workgroups: three pieces per tile);
  * MXFP8 512 x 3072 x 8192 on 40 CUs: 24 tiles of 16 units, 3 per group of 5.
Integer-coded inputs make every partial sum exact, so the result is
bit-exact whatever the summation order; random inputs meet the acceptance
bound against the oracle.  Flag words that start at zero are zero again
after a call (every raised flag is consumed and cleared, and the spin-timeout
word stays clear), and left-over workspace contents do not change the result.
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

HEADER = 16384            # flag words at the start of a split workspace
SLOT = 256 * 256 * 4      # one FP32 partial tile

CASES = [("mxfp8", 256, 4096, 6144, 32), ("mxfp8", 256, 2816, 6144, 32), ("mxfp4", 300, 2048, 16384, 32),
         ("nvfp4", 256, 2552, 8192, 24), ("mxfp8", 512, 3072, 8192, 40)]
_IDS = [f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-cu{c[4]}" for c in CASES]


def _grid(cus):
    return cus - cus % 8 if cus >= 8 else cus


def _run(mode, a, sfa, b, sfb, m, n, k, dev, cus, ws, bias=None, alpha=None, f16=False):
    out = torch.zeros(m, n, dtype=torch.float16 if f16 else torch.bfloat16, device=dev)
    hq.hq_dense_gemm(mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev), U.dev_u8(sfb, dev), out,
                     bias=None if bias is None else U.dev_bf16(bias, dev),
                     alpha=None if alpha is None else torch.tensor([alpha], dtype=torch.float32, device=dev),
                     cu_limit=cus, workspace=ws)
    torch.cuda.synchronize()
    return U.host_bits(out)


def _flags_clear(ws):
    flags = ws[:HEADER].cpu().numpy().view(np.uint64)
    return int(np.count_nonzero(flags))


@pytest.mark.parametrize("case", CASES, ids=_IDS)
def test_stream_k_plan_size(case):
    """The size query gives the stream-K workspace: the flag words and two
    partial tiles per workgroup."""
    mode, m, n, k, cus = case
    U.require_gpu()
    assert hq.hq_gemm_workspace_size(mode, m, n, k, cu_limit=cus) == HEADER + 2 * _grid(cus) * SLOT


@pytest.mark.parametrize("case", CASES, ids=_IDS)
def test_stream_k_integer_exact(case):
    mode, m, n, k, cus = case
    dev = U.require_gpu()
    U.banner(f"stream-K int-exact {mode} m={m} n={n} k={k} cu_limit={cus}")
    rng = np.random.default_rng(m + n + k + cus)
    av, a, sfa = _int_operand(rng, m, k, mode, [-1, 0, 1])
    bv, b, sfb = _int_operand(rng, n, k, mode, [-1, 0, 1])
    ws = hq.gemm_workspace(mode, m, n, k, cu_limit=cus, device=dev)
    assert ws is not None
    ws[:HEADER].zero_()
    got = _run(mode, a, sfa, b, sfb, m, n, k, dev, cus, ws, alpha=1.0 if mode == "nvfp4" else None)
    want = F.bf16_round(av.astype(np.float64) @ bv.astype(np.float64).T)   # exact: |sums| <= k
    assert np.array_equal(got, want), f"{np.sum(got != want)} of {got.size} differ"
    assert _flags_clear(ws) == 0, "flag words left set (or the spin-timeout word)"


@pytest.mark.parametrize("case", CASES[1:4], ids=_IDS[1:4])
def test_stream_k_random_with_bias_or_alpha(case):
    mode, m, n, k, cus = case
    dev = U.require_gpu()
    U.banner(f"stream-K random {mode} m={m} n={n} k={k} cu_limit={cus}")
    rng = np.random.default_rng(5 * m + k + cus)
    a, sfa, ga = _quant(synth.normal_bf16(rng, (m, k)), mode)
    b, sfb, gb = _quant(synth.normal_bf16(rng, (n, k), 0.05), mode)
    alpha = None if ga is None else np.float32(ga * gb)
    bias = synth.normal_bf16(rng, (n,), 0.1) if mode == "mxfp8" else None
    ws = hq.gemm_workspace(mode, m, n, k, cu_limit=cus, device=dev)
    ws[:HEADER].zero_()
    got = _run(mode, a, sfa, b, sfb, m, n, k, dev, cus, ws, bias=bias, alpha=alpha)
    want = G.dense_gemm(mode, a, sfa, b, sfb, bias, alpha)
    U.assert_gemm_close(got, want, U.deq(mode, a, sfa), U.deq(mode, b, sfb), alpha, f"stream-K {mode}")
    assert _flags_clear(ws) == 0


def test_stream_k_f16_out():
    """Binary16 output (HQ_OUT_FP16) through the stream-K reduction: equal to
    the unsplit call's binary16 output on integer-coded inputs."""
    dev = U.require_gpu()
    mode, m, n, k, cus = CASES[1]
    rng = np.random.default_rng(99)
    _, a, sfa = _int_operand(rng, m, k, mode, [-2, -1, 0, 1, 2])
    _, b, sfb = _int_operand(rng, n, k, mode, [-1, 0, 1])
    ws = hq.gemm_workspace(mode, m, n, k, cu_limit=cus, device=dev)
    got = _run(mode, a, sfa, b, sfb, m, n, k, dev, cus, ws, f16=True)
    plain = _run(mode, a, sfa, b, sfb, m, n, k, dev, cus, None, f16=True)
    assert np.array_equal(got, plain)


def test_stream_k_left_over_workspace_contents():
    """Whatever the workspace holds before a call -- all ones, random bytes, the
    previous call's partials -- the result is the same, call after call."""
    dev = U.require_gpu()
    mode, m, n, k, cus = CASES[1]
    rng = np.random.default_rng(123)
    a, sfa, _ = _quant(synth.normal_bf16(rng, (m, k)), mode)
    b, sfb, _ = _quant(synth.normal_bf16(rng, (n, k), 0.05), mode)
    ws = hq.gemm_workspace(mode, m, n, k, cu_limit=cus, device=dev)
    ref = _run(mode, a, sfa, b, sfb, m, n, k, dev, cus, ws)
    ws.fill_(0xFF)
    assert np.array_equal(_run(mode, a, sfa, b, sfb, m, n, k, dev, cus, ws), ref)
    ws.copy_(torch.from_numpy(rng.integers(0, 256, ws.numel(), dtype=np.uint8)).to(dev))
    assert np.array_equal(_run(mode, a, sfa, b, sfb, m, n, k, dev, cus, ws), ref)
    for _ in range(3):
        assert np.array_equal(_run(mode, a, sfa, b, sfb, m, n, k, dev, cus, ws), ref)


def test_stream_k_beside_other_work():
    """Stream-K calls while FP32 matrix products run on another stream and
    hold compute units: a piece waits only for workgroups dispatched before
    it, so the results stay those of the idle GPU and no wait gives up (the
    spin-timeout word, the last flag word, stays clear)."""
    dev = U.require_gpu()
    mode, m, n, k, cus = CASES[1]
    rng = np.random.default_rng(321)
    a, sfa, _ = _quant(synth.normal_bf16(rng, (m, k)), mode)
    b, sfb, _ = _quant(synth.normal_bf16(rng, (n, k), 0.05), mode)
    ws = hq.gemm_workspace(mode, m, n, k, cu_limit=cus, device=dev)
    ws[:HEADER].zero_()
    ref = _run(mode, a, sfa, b, sfb, m, n, k, dev, cus, ws)
    other = torch.cuda.Stream()
    x = torch.randn(4096, 4096, device=dev)
    for _ in range(4):
        with torch.cuda.stream(other):
            y = x
            for _ in range(12):
                y = torch.mm(y, x) * 1e-2
        assert np.array_equal(_run(mode, a, sfa, b, sfb, m, n, k, dev, cus, ws), ref)
    torch.cuda.synchronize()
    assert _flags_clear(ws) == 0
