"""Helpers for the GPU parity tests: host <-> device BF16 bit transfer, the
acceptance bound, and a banner printed (and flushed) before each GPU step so
a failing run names its case."""
import sys

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_gemm_moe_amd as hq
    hq.load()           # fails loudly if the library is missing
    return torch.device("cuda:0")


def dev_bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def dev_u8(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)


def dev_i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def host_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_u8(t):
    return t.detach().cpu().numpy()


def assert_gemm_close(out_bits, ref_bits, a_deq, b_deq, alpha=None, what=""):
    """Acceptance bound: per element |out - ref| <= 2^-7 |ref| +
    1e-3 ||a_m|| ||b_n|| |alpha| (dequantised rows), and relative Frobenius
    error <= 2e-3."""
    out = F.bf16_decode(out_bits)
    ref = F.bf16_decode(ref_bits)
    assert out.shape == ref.shape, what
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    slack = G.tolerance(a_deq, b_deq, alpha)
    err = np.abs(out - ref)
    bad = err > 2.0 ** -7 * np.abs(ref) + slack
    assert not bad.any(), f"{what}: {bad.sum()} elements out of bound; worst {err[bad].max()}"
    nref = np.linalg.norm(ref)
    if nref > 0:
        rel = np.linalg.norm(out - ref) / nref
        assert rel <= 2e-3, f"{what}: relative Frobenius error {rel}"


def deq(mode, codes, sf):
    return Q.dequant(codes, sf, {0: "mxfp8", 1: "mxfp4", 2: "nvfp4"}.get(mode, mode))


SILU_LIPSCHITZ = 1.0999   # max |d silu / d g| (at g ~ 2.4): 1.09985...


def assert_y_close(y, x_bits, h, what=""):
    """SwiGLU contract on the same BF16 gate|up input: per element
    |y - y_ref| <= 2^-7 |y_ref| + 1e-6 against the oracle's float64 SwiGLU,
    and relative Frobenius error <= 2e-3."""
    from oracle import swiglu as S
    y = np.asarray(y, np.float64)
    ref = S.swiglu_f64(x_bits, h)
    bad = np.abs(y - ref) > 2.0 ** -7 * np.abs(ref) + 1e-6
    assert not bad.any(), f"{what}: {bad.sum()} y values out of bound"
    nref = np.linalg.norm(ref)
    if nref > 0:
        assert np.linalg.norm(y - ref) / nref <= 2e-3, f"{what}: relative Frobenius error of y"


def assert_y_close_to_gemm_oracle(y, gu_ref_bits, gu_slack, h, what=""):
    """y of the fused gate|up GEMM + SwiGLU against the oracle's SwiGLU of the
    oracle's GEMM, per element, with the GEMM acceptance bound carried
    through SwiGLU: gate and up may each be off by dG = 2^-7 |g| + slack_g,
    dU = 2^-7 |u| + slack_u (slack: the GEMM bound's absolute term), so
      |y - y_ref| <= L dG (|u| + dU) + |silu(g)| dU + 2^-7 |y_ref| + 1e-6
    with L the Lipschitz constant of silu; plus relative Frobenius error
    <= 2e-3."""
    from oracle import swiglu as S
    x = F.bf16_decode(gu_ref_bits)
    g, u = x[:, :h], x[:, h:2 * h]
    dG = 2.0 ** -7 * np.abs(g) + gu_slack[:, :h]
    dU = 2.0 ** -7 * np.abs(u) + gu_slack[:, h:2 * h]
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    ref = S.swiglu_f64(gu_ref_bits, h)
    bound = SILU_LIPSCHITZ * dG * (np.abs(u) + dU) + np.abs(silu) * dU + 2.0 ** -7 * np.abs(ref) + 1e-6
    y = np.asarray(y, np.float64)
    bad = np.abs(y - ref) > bound
    assert not bad.any(), f"{what}: {bad.sum()} y values outside the propagated bound"
    nref = np.linalg.norm(ref)
    if nref > 0:
        assert np.linalg.norm(y - ref) / nref <= 2e-3, f"{what}: relative Frobenius error of y"
