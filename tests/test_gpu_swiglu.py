"""GPU parity of hq_fused_swiglu_quant.

Contract (exp() differs between implementations, so several code tensors can
be correct for one input):
  (a) the FP32 y the device used (y_debug) is within the acceptance bound of
      the oracle's float64 SwiGLU;
  (b) codes and scales are bit-exact against the oracle's quantisation of
      that same y;
  (c) a run without y_debug writes the same codes and scales;
  (d) rows outside the processed set keep their sentinel bytes.
The fraction of codes that differ from the quantisation of the float64 y is
printed, not gated.
"""
import numpy as np
import pytest
import torch

import fp4_gemm_moe_amd as hq
import synth
from oracle import swiglu as S
from tests import _gpu as U

pytestmark = pytest.mark.gpu

MODES = ["mxfp8", "mxfp4", "nvfp4"]


def _alloc(rows, h, mode, dev):
    cols = h if mode == "mxfp8" else h // 2
    gs = 16 if mode == "nvfp4" else 32
    q = torch.full((rows, cols), 0xA5, dtype=torch.uint8, device=dev)
    sf = torch.full((rows, h // gs), 0x5A, dtype=torch.uint8, device=dev)
    return q, sf


def _run_case(mode, x_bits, h, dev, num_groups, group_end=None, slot_rows=0, valid=None, g=None):
    rows = x_bits.shape[0]
    x = U.dev_bf16(x_bits, dev)
    ge = None if group_end is None else U.dev_i32(group_end, dev)
    va = None if valid is None else U.dev_i32(valid, dev)
    gs = None if g is None else torch.tensor([g], dtype=torch.float32, device=dev)
    q1, s1 = _alloc(rows, h, mode, dev)
    y = torch.full((rows, h), float("nan"), dtype=torch.float32, device=dev)
    hq.hq_fused_swiglu_quant(mode, x, q1, s1, num_groups, ge, slot_rows, va, gs, y)
    q2, s2 = _alloc(rows, h, mode, dev)
    hq.hq_fused_swiglu_quant(mode, x, q2, s2, num_groups, ge, slot_rows, va, gs, None)
    torch.cuda.synchronize()
    q1, s1, q2, s2 = (U.host_u8(t) for t in (q1, s1, q2, s2))
    yd = y.cpu().numpy().astype(np.float64)
    mask = S.processed_rows(rows, group_end=group_end, slot_rows=slot_rows, valid=valid,
                            num_groups=num_groups)
    # (d) untouched rows
    assert np.all(q1[~mask] == 0xA5) and np.all(s1[~mask] == 0x5A)
    assert np.all(np.isnan(yd[~mask]))
    # (c) y_debug does not change the result
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    if not mask.any():
        return
    # (a) y within tolerance of float64 SwiGLU
    yref = S.swiglu_f64(x_bits, h)[mask]
    ym = yd[mask]
    err = np.abs(ym - yref)
    assert np.all(err <= 2.0 ** -7 * np.abs(yref) + 1e-6), f"y error {err.max()}"
    # (b) codes exact against the quantisation of the device's y
    c, s = S.quantize_y(ym, mode, None if g is None else np.float32(g))
    assert np.array_equal(s1[mask], s), f"{np.sum(s1[mask] != s)} scale bytes differ"
    assert np.array_equal(q1[mask], c), f"{np.sum(q1[mask] != c)} code bytes differ"
    c_ref, _, _ = S.swiglu_quant(x_bits[mask], h, mode, g=None if g is None else np.float32(g))
    frac = np.mean(c_ref != c)
    print(f"[swiglu {mode}] codes differing from quant(y_f64): {frac:.2e}")


@pytest.mark.parametrize("mode", MODES)
def test_swiglu_contiguous_groups_with_valid(mode):
    dev = U.require_gpu()
    rng = np.random.default_rng(21)
    h = 256
    ends = np.array([5, 5, 40, 64, 100], np.int32)
    valid = np.array([3, 7, 35, 0, 30], np.int32)
    rows = 110
    x = synth.normal_bf16(rng, (rows, 2 * h), 2.0)
    U.banner(f"swiglu contiguous {mode}")
    _run_case(mode, x, h, dev, len(ends), group_end=ends, valid=valid, g=0.003 if mode == "nvfp4" else None)


@pytest.mark.parametrize("mode", MODES)
def test_swiglu_slot_form(mode):
    dev = U.require_gpu()
    rng = np.random.default_rng(22)
    E, M, h = 4, 128, 2048 // 4
    valid = np.array([128, 64, 0, 32], np.int32)
    x = synth.normal_bf16(rng, (E * M, 2 * h))
    U.banner(f"swiglu slots {mode}")
    _run_case(mode, x, h, dev, E, slot_rows=M, valid=valid, g=0.002 if mode == "nvfp4" else None)


def test_swiglu_all_rows_no_valid_and_extreme_gates():
    dev = U.require_gpu()
    h = 96
    rng = np.random.default_rng(23)
    x = synth.normal_bf16(rng, (40, 2 * h), 1.0)
    xf = synth.to_bf16_bits(np.array([0.0, 100.0, -100.0, -0.0], np.float32))
    x[0, :4] = xf                                   # gates 0, +big, -big, -0
    U.banner("swiglu all rows")
    _run_case("mxfp8", x, h, dev, 1, slot_rows=40)


def test_swiglu_moe_layout_sampled():
    """The MoE chain layout: [R, 2*1536] with 128-padded groups (E = 32), only
    the valid rows of each group processed; checked on the full tensor."""
    dev = U.require_gpu()
    d = synth.moe_contiguous(with_weights=False)
    counts, ends = d["counts"], d["group_end"]
    R, H = int(ends[-1]), d["H"]
    rng = np.random.default_rng(24)
    rows = np.sort(rng.choice(R, 2048, replace=False))
    x = synth.normal_bf16(rng, (R, 2 * H))
    U.banner("swiglu moe layout")
    xd = U.dev_bf16(x, dev)
    q, sf = _alloc(R, H, "mxfp8", dev)
    y = torch.empty((R, H), dtype=torch.float32, device=dev)
    hq.hq_fused_swiglu_quant("mxfp8", xd, q, sf, len(ends), U.dev_i32(ends, dev), 0,
                             U.dev_i32(counts.astype(np.int32), dev), None, y)
    torch.cuda.synchronize()
    mask = S.processed_rows(R, group_end=ends, valid=counts)
    qh, sh = U.host_u8(q), U.host_u8(sf)
    assert np.all(qh[~mask] == 0xA5)
    sel = rows[mask[rows]]
    ys = y[torch.from_numpy(sel).to(dev)].cpu().numpy().astype(np.float64)
    yref = S.swiglu_f64(x[sel], H)
    assert np.all(np.abs(ys - yref) <= 2.0 ** -7 * np.abs(yref) + 1e-6)
    c, s = S.quantize_y(ys, "mxfp8")
    assert np.array_equal(qh[sel], c) and np.array_equal(sh[sel], s)
