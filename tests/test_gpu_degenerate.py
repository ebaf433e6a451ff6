"""Degenerate grouped calls on the GPU: every group empty.

A grouped call whose groups hold no rows (cumulative ends all 0, masked
counts all 0, valid counts all 0) has nothing to compute. Every kernel path
must then leave its outputs as they were. That covers the tiled kernel (rows
of A above the skinny limit), the direct kernel (16 rows or fewer), the fused
SwiGLU epilogue, both backward dSwiGLU epilogues (D and dprob) and the
standalone SwiGLU + re-quant. The outputs are prefilled with a sentinel and
compared bit for bit.
"""
import numpy as np
import pytest
import torch

import fp4_gemm_moe_amd as hq
from tests import _gpu as U

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1   # a BF16 NaN pattern no kernel produces


def _operands(mode, rows, E, n, k, dev, seed):
    """Random codes with unit scales (the values are never used: no row is valid)."""
    rng = np.random.default_rng(seed)
    kc = k if mode == "mxfp8" else k // 2
    gs = 16 if mode == "nvfp4" else 32
    unit = 0x38 if mode == "nvfp4" else 127
    a = U.dev_u8(rng.integers(0, 256, (rows, kc), dtype=np.uint8), dev)
    sfa = U.dev_u8(np.full((rows, k // gs), unit, np.uint8), dev)
    b = U.dev_u8(rng.integers(0, 256, (E, n, kc), dtype=np.uint8), dev)
    sfb = U.dev_u8(np.full((E, n, k // gs), unit, np.uint8), dev)
    alpha = torch.ones(E, dtype=torch.float32, device=dev) if mode == "nvfp4" else None
    return a, sfa, b, sfb, alpha


def _sentinel_bf16(shape, dev):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("rows", [8, 512], ids=["direct", "tiled"])
def test_contiguous_all_groups_empty(mode, rows):
    dev = U.require_gpu()
    E, n, k = 4, 256, 512
    U.banner(f"contiguous {mode}, {rows} rows, every group empty")
    a, sfa, b, sfb, alpha = _operands(mode, rows, E, n, k, dev, 1)
    out = _sentinel_bf16((rows, n), dev)
    hq.hq_group_contiguous_gemm(mode, a, sfa, b, sfb, U.dev_i32(np.zeros(E, np.int32), dev), out, alpha=alpha)
    torch.cuda.synchronize()
    assert np.all(U.host_bits(out) == SENTINEL), "an empty group wrote output rows"


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("max_m", [16, 256], ids=["direct", "tiled"])
def test_masked_all_counts_zero(mode, max_m):
    dev = U.require_gpu()
    E, n, k = 4, 256, 512
    U.banner(f"masked {mode}, slots of {max_m}, every count 0")
    a, sfa, b, sfb, alpha = _operands(mode, E * max_m, E, n, k, dev, 2)
    out = _sentinel_bf16((E * max_m, n), dev)
    hq.hq_group_masked_gemm(mode, a, sfa, b, sfb, U.dev_i32(np.zeros(E, np.int32), dev), out, max_m, alpha=alpha)
    torch.cuda.synchronize()
    assert np.all(U.host_bits(out) == SENTINEL), "a slot with count 0 wrote output rows"


@pytest.mark.parametrize("ends_zero", [True, False], ids=["ends_zero", "valid_zero"])
def test_gemm_swiglu_nothing_valid(ends_zero):
    """The fused gate|up GEMM: no rows at all, or rows in every group but no
    valid ones: no codes and no scales are written."""
    dev = U.require_gpu()
    E, h, k, rows = 4, 128, 512, 512
    U.banner(f"gemm+swiglu, {'ends 0' if ends_zero else 'valid 0'}")
    a, sfa, b, sfb, _ = _operands("mxfp8", rows, E, 2 * h, k, dev, 3)
    ends = np.zeros(E, np.int32) if ends_zero else np.array([128, 256, 384, 512], np.int32)
    q = torch.full((rows, h), 0xA5, dtype=torch.uint8, device=dev)
    sf = torch.full((rows, h // 32), 0xA5, dtype=torch.uint8, device=dev)
    hq.hq_group_contiguous_gemm_swiglu_quant("mxfp8", a, sfa, b, sfb, U.dev_i32(ends, dev), q, sf,
                                             valid=U.dev_i32(np.zeros(E, np.int32), dev))
    torch.cuda.synchronize()
    assert torch.all(q == 0xA5).item() and torch.all(sf == 0xA5).item(), "codes or scales written for no valid row"


@pytest.mark.parametrize("quantised", [False, True], ids=["bf16_d", "rowquant_d"])
def test_dswiglu_all_groups_empty(quantised):
    """Backward dSwiGLU GEMM with every group empty: D untouched and dprob
    keeps its values (nothing is added)."""
    dev = U.require_gpu()
    E, n, k, rows = 4, 128, 512, 512
    U.banner(f"dswiglu ({'row-quantised' if quantised else 'BF16'} D), every group empty")
    a, sfa, b, sfb, _ = _operands("mxfp8", rows, E, n, k, dev, 4)
    c = torch.zeros(rows, 2 * n, dtype=torch.bfloat16, device=dev)
    prob = torch.ones(rows, dtype=torch.float32, device=dev)
    dprob = torch.full((rows,), 1.5, dtype=torch.float32, device=dev)
    ends = U.dev_i32(np.zeros(E, np.int32), dev)
    if quantised:
        dq = torch.full((rows, 2 * n), 0xA5, dtype=torch.uint8, device=dev)
        dsf = torch.full((rows, 2 * n // 32), 0xA5, dtype=torch.uint8, device=dev)
        hq.hq_group_contiguous_gemm_dswiglu_quant("mxfp8", a, sfa, b, sfb, ends, c, prob, dprob, dq, dsf)
        torch.cuda.synchronize()
        assert torch.all(dq == 0xA5).item() and torch.all(dsf == 0xA5).item(), "D codes or scales written"
    else:
        d = _sentinel_bf16((rows, 2 * n), dev)
        hq.hq_group_contiguous_gemm_dswiglu("mxfp8", a, sfa, b, sfb, ends, c, prob, dprob, d)
        torch.cuda.synchronize()
        assert np.all(U.host_bits(d) == SENTINEL), "D rows written for an empty group"
    assert torch.all(dprob == 1.5).item(), "dprob changed with no rows"


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
def test_swiglu_quant_no_valid_rows(mode):
    dev = U.require_gpu()
    E, h, rows = 4, 128, 256
    U.banner(f"swiglu {mode}, valid counts all 0")
    x = torch.randn(rows, 2 * h, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(dev)
    kc = h if mode == "mxfp8" else h // 2
    gs = 16 if mode == "nvfp4" else 32
    q = torch.full((rows, kc), 0xA5, dtype=torch.uint8, device=dev)
    sf = torch.full((rows, h // gs), 0xA5, dtype=torch.uint8, device=dev)
    g = torch.ones(1, dtype=torch.float32, device=dev) if mode == "nvfp4" else None
    ends = U.dev_i32(np.array([64, 128, 192, 256], np.int32), dev)
    hq.hq_fused_swiglu_quant(mode, x, q, sf, E, ends, 0, U.dev_i32(np.zeros(E, np.int32), dev), global_scale=g)
    torch.cuda.synchronize()
    assert torch.all(q == 0xA5).item() and torch.all(sf == 0xA5).item(), "codes or scales written for no valid row"
