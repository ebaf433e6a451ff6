"""GPU parity of the grouped-contiguous GEMM with discrete expert weights (the
cuDNN FE "Grouped GEMM + dGLU (SM100)" page's b_ptrs form): each expert's
codes and scales in their own allocation, addressed through device arrays of
pointers.

* Against the oracle: every group's rows within the acceptance bound.
* Against hq_group_contiguous_gemm on the same weights packed into one tensor:
  the same output bits (same kernels and K order), rows after the last end
  untouched.
* Tiled path (MXFP8 / MXFP4 / NVFP4, both scale-load layouts) and the direct
  path (16 rows or fewer), empty groups, experts allocated in reverse order.
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


CASES = [
    ("mxfp8", [40, 0, 300, 17], 512, 136),      # tiled, grouped scale loads
    ("mxfp8", [70, 33], 384, 64),               # tiled, per-step scale planes
    ("mxfp4", [129, 0, 64], 1024, 264),
    ("nvfp4", [200, 56], 512, 128),
    ("mxfp4", [5, 0, 7], 512, 72),              # 12 rows: the direct path
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-K{c[2]}-N{c[3]}-rows{sum(c[1])}")
def test_ptr_array_matches_packed_and_oracle(case):
    mode, counts, K, N = case
    dev = U.require_gpu()
    U.banner(f"ptr-array {mode} counts={counts} K={K} N={N}")
    rng = np.random.default_rng(K + N + len(counts))
    E = len(counts)
    ends = np.cumsum(counts).astype(np.int32)
    R = int(ends[-1]) + 3
    a, sfa, ga = _quant(synth.normal_bf16(rng, (R, K)), mode)
    bq, bs, gb = _quant(synth.normal_bf16(rng, (E * N, K), 0.05), mode)
    b, sfb = bq.reshape(E, N, -1), bs.reshape(E, N, -1)
    alpha = None if ga is None else np.full(E, np.float32(ga * gb), np.float32)
    bias = synth.normal_bf16(rng, (E, N), 0.1) if mode == "mxfp8" else None
    da, dsa, ge = U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_i32(ends, dev)
    dbias = None if bias is None else U.dev_bf16(bias, dev)
    dalpha = None if alpha is None else torch.from_numpy(alpha).to(dev)
    # separate allocations, made in reverse order so they are not laid out as one tensor
    bs_list, sfbs_list = [None] * E, [None] * E
    for g in reversed(range(E)):
        bs_list[g] = U.dev_u8(b[g], dev)
        sfbs_list[g] = U.dev_u8(sfb[g], dev)
    out = torch.full((R, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    keep = hq.hq_group_contiguous_gemm_ptr_array(mode, da, dsa, bs_list, sfbs_list, ge, out, N,
                                                 bias=dbias, alpha=dalpha)
    ref = torch.full((R, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    hq.hq_group_contiguous_gemm(mode, da, dsa, U.dev_u8(b, dev), U.dev_u8(sfb, dev), ge, ref,
                                bias=dbias, alpha=dalpha)
    torch.cuda.synchronize()
    del keep
    got = U.host_bits(out)
    assert np.array_equal(got, U.host_bits(ref)), "differs from the packed-weights call"
    lo = 0
    for g in range(E):
        hi = int(ends[g])
        if hi > lo:
            want = G.dense_gemm(mode, a[lo:hi], sfa[lo:hi], b[g], sfb[g],
                                None if bias is None else bias[g], None if alpha is None else alpha[g])
            U.assert_gemm_close(got[lo:hi], want, U.deq(mode, a[lo:hi], sfa[lo:hi]), U.deq(mode, b[g], sfb[g]),
                                None if alpha is None else alpha[g], what=f"group {g}")
        lo = hi
    assert (got[int(ends[-1]):] == SENTINEL).all(), "rows after the last end were written"
