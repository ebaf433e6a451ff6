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
