"""hq_dense_gemm_scratch -- the dense GEMM for callers that cannot allocate --
against hq_dense_gemm_ws with a caller workspace, through the C ABI.

Two calls in a row (the second with a smaller input) must each give the same
bits as hq_dense_gemm_ws with a workspace of the plan's size (same split plan,
same kernels), and both are within the acceptance bound of the oracle (the
calls include a stream-K plan that fits the scratch).  A shape whose K split
needs more than the library's scratch is refused before any launch (its
output untouched); a stream-K plan that needs more is not taken (the call
runs unsplit); a shape that does not split runs as hq_dense_gemm.
"""
import numpy as np
import pytest
import torch

import fp4_gemm_moe_amd as hq
import synth
from oracle import gemm as G
from oracle import quant as Q
from tests import _gpu as U

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1


def _quant(bits, mode):
    if mode == "nvfp4":
        c, s, g = Q.nvfp4_quant_bf16(bits)
        return c, s, np.float32(g)
    c, s = Q.mx_quant_bf16(bits, mode)
    return c, s, None


def _operands(mode, m, n, k, seed):
    rng = np.random.default_rng(seed)
    a, sfa, ga = _quant(synth.normal_bf16(rng, (m, k)), mode)
    b, sfb, gb = _quant(synth.normal_bf16(rng, (n, k), 0.05), mode)
    alpha = None if ga is None else np.float32(ga * gb)
    bias = synth.normal_bf16(rng, (n,), 0.1) if mode == "mxfp8" else None
    return a, sfa, b, sfb, alpha, bias


def _run(fn, mode, ops, m, n, dev, cu_limit=0):
    a, sfa, b, sfb, alpha, bias = ops
    out = torch.full((m, n), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    kw = dict(bias=None if bias is None else U.dev_bf16(bias, dev),
              alpha=None if alpha is None else torch.tensor([alpha], dtype=torch.float32, device=dev),
              cu_limit=cu_limit)
    args = (mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev), U.dev_u8(sfb, dev), out)
    if fn == "scratch":
        hq.hq_dense_gemm_scratch(*args, **kw)
    else:
        k = a.shape[1] * (1 if mode == "mxfp8" else 2)
        ws = hq.gemm_workspace(mode, m, n, k, cu_limit=cu_limit, device=dev)
        assert ws is not None and ws.numel() <= hq.HQ_SCRATCH_BYTES
        hq.hq_dense_gemm(*args, workspace=ws, **kw)
    torch.cuda.synchronize()
    return U.host_bits(out)


# (mode, m, n, k, cu_limit): a K split of every tile, a smaller one, a tail split, a
# stream-K plan that fits the scratch (16 tiles over 32 workgroups: 16.4 MB of flags and
# partial slots, the flags at the scratch's start zero from load and after every call)
CASES = [("mxfp8", 300, 520, 8576, 0), ("mxfp4", 200, 264, 8448, 0), ("mxfp8", 520, 1544, 6144, 16),
         ("mxfp8", 256, 4096, 6144, 32)]


def test_scratch_equals_workspace_call_twice_in_a_row():
    dev = U.require_gpu()
    for i, (mode, m, n, k, cus) in enumerate(CASES):
        U.banner(f"no-alloc dense gemm call {i}: {mode} {m}x{n}x{k} cu_limit={cus}")
        assert 0 < hq.hq_gemm_workspace_size(mode, m, n, k, cu_limit=cus) <= hq.HQ_SCRATCH_BYTES
        ops = _operands(mode, m, n, k, seed=100 + i)
        got = _run("scratch", mode, ops, m, n, dev, cus)
        ref_dev = _run("ws", mode, ops, m, n, dev, cus)
        assert np.array_equal(got, ref_dev), f"call {i}: {np.sum(got != ref_dev)} outputs differ from the ws call"
        a, sfa, b, sfb, alpha, bias = ops
        want = G.dense_gemm(mode, a, sfa, b, sfb, bias, alpha)
        U.assert_gemm_close(got, want, U.deq(mode, a, sfa), U.deq(mode, b, sfb), alpha, f"call {i} vs oracle")


def test_scratch_refuses_a_split_larger_than_its_array():
    dev = U.require_gpu()
    mode, m, n, k = "mxfp4", 512, 5120, 17408
    need = hq.hq_gemm_workspace_size(mode, m, n, k)
    if need <= hq.HQ_SCRATCH_BYTES:
        pytest.skip(f"this device's split plan for the shape needs {need} bytes: fits")
    U.banner(f"no-alloc dense gemm refuses {mode} {m}x{n}x{k} ({need} bytes)")
    out = torch.full((m, n), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    a = torch.zeros(m, k // 2, dtype=torch.uint8, device=dev)
    sa = torch.zeros(m, k // 32, dtype=torch.uint8, device=dev)
    b = torch.zeros(n, k // 2, dtype=torch.uint8, device=dev)
    sb = torch.zeros(n, k // 32, dtype=torch.uint8, device=dev)
    with pytest.raises(hq.HQError) as e:
        hq.hq_dense_gemm_scratch(mode, a, sa, b, sb, out)
    assert e.value.status == -2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out.view(torch.int16) == SENTINEL).all()), "a refused call wrote its output"


def test_scratch_without_split_equals_plain_call():
    dev = U.require_gpu()
    mode, m, n, k = "mxfp8", 64, 136, 512          # 4 K steps: too short to split
    assert hq.hq_gemm_workspace_size(mode, m, n, k) == 0
    ops = _operands(mode, m, n, k, seed=7)
    got = _run("scratch", mode, ops, m, n, dev)
    a, sfa, b, sfb, alpha, bias = ops
    out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    hq.hq_dense_gemm(mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev), U.dev_u8(sfb, dev), out,
                     bias=U.dev_bf16(bias, dev))
    torch.cuda.synchronize()
    assert np.array_equal(got, U.host_bits(out))


def test_scratch_runs_a_larger_stream_k_plan_unsplit():
    """A stream-K plan that needs more than the scratch is not taken (rather
    than refused): the call runs unsplit, with the bits of hq_dense_gemm
    without a workspace."""
    dev = U.require_gpu()
    mode, m, n, k = "nvfp4", 512, 17408, 5120
    need = hq.hq_gemm_workspace_size(mode, m, n, k)
    if need <= hq.HQ_SCRATCH_BYTES:
        pytest.skip(f"this device's split plan for the shape needs {need} bytes: fits")
    U.banner(f"no-alloc dense gemm runs {mode} {m}x{n}x{k} unsplit ({need} bytes planned)")
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    a = torch.randint(0, 256, (m, k // 2), dtype=torch.uint8, device=dev, generator=g)
    b = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=dev, generator=g)
    sa = torch.randint(0x30, 0x40, (m, k // 16), dtype=torch.uint8, device=dev, generator=g)
    sb = torch.randint(0x30, 0x40, (n, k // 16), dtype=torch.uint8, device=dev, generator=g)
    alpha = torch.ones(1, dtype=torch.float32, device=dev)
    outs = []
    for fn in ("scratch", "plain"):
        out = torch.full((m, n), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
        if fn == "scratch":
            hq.hq_dense_gemm_scratch(mode, a, sa, b, sb, out, alpha=alpha)
        else:
            hq.hq_dense_gemm(mode, a, sa, b, sb, out, alpha=alpha)
        torch.cuda.synchronize()
        outs.append(U.host_bits(out))
    assert np.array_equal(outs[0], outs[1])
