"""GPU parity of the gate|up grouped-contiguous GEMM with the SwiGLU + MXFP8
re-quant applied in its epilogue (HALOps "GEMM" page: group_contiguous_gemm
followed by fused_swiglu_quant, without the BF16 intermediate).

* Against the oracle: per group, the gate|up output within the GEMM bound;
  y per element within 2^-7 |ref| + 1e-6 of the float64 SwiGLU of that BF16
  gate|up, and within the GEMM bound carried through SwiGLU of the oracle's
  own GEMM + SwiGLU (plus relative Frobenius error <= 2e-3); the codes and
  scales are bit-exact with the oracle's quantisation of the device's y
  (several code tensors can be correct, as for hq_fused_swiglu_quant, since
  exp differs between implementations).
* At the full MoE size: sampled rows of four experts against the oracle the
  same way, and every byte against the two-call chain.
* Against the two-call chain on the device: codes, scales and y are the same
  bits (the call's documented contract), rows past a group's valid count and
  after the last end keep their contents.
* Both scale-load layouts of the tiled kernel (K % 512 == 0 and not), bias,
  ragged and empty groups, a group longer than one 256-row tile.
"""
import numpy as np
import pytest
import torch

import fp4_gemm_moe_amd as hq
import synth
from oracle import gemm as G
from oracle import quant as Q
from oracle import swiglu as S
from tests import _gpu as U

pytestmark = pytest.mark.gpu

FILL = 0x5A        # a byte the calls must not write over outside the written rows


def _inputs(counts, align, K, H, seed, bias):
    rng = np.random.default_rng(seed)
    counts = np.asarray(counts, np.int64)
    E = len(counts)
    ends, _ = synth.padded_group_ends(counts, align)
    starts = np.concatenate([[0], ends[:-1]]).astype(np.int64)
    R = int(ends[-1]) + 5                          # trailing rows after the last end
    x = np.zeros((R, K), np.uint16)
    for g in range(E):
        x[starts[g]:starts[g] + counts[g]] = synth.normal_bf16(rng, (int(counts[g]), K))
    w = synth.normal_bf16(rng, (E * 2 * H, K), 0.05)
    b = synth.normal_bf16(rng, (E, 2 * H), 0.1) if bias else None
    return counts, ends, starts, R, x, w, b


def _run_both(dev, counts, ends, R, x, w, b, K, H):
    E = len(counts)
    ge, valid = U.dev_i32(ends, dev), U.dev_i32(counts, dev)
    aq, asf, _ = hq.quantize(U.dev_bf16(x, dev), "mxfp8")
    wq, wsf, _ = hq.quantize(U.dev_bf16(w, dev), "mxfp8")
    wq, wsf = wq.view(E, 2 * H, K), wsf.view(E, 2 * H, K // 32)
    bias = None if b is None else U.dev_bf16(b, dev)
    q = torch.full((R, H), FILL, dtype=torch.uint8, device=dev)
    sf = torch.full((R, H // 32), FILL, dtype=torch.uint8, device=dev)
    y = torch.full((R, H), -7.0, dtype=torch.float32, device=dev)
    hq.hq_group_contiguous_gemm_swiglu_quant("mxfp8", aq, asf, wq, wsf, ge, q, sf, valid=valid,
                                             bias=bias, y_debug=y)
    # the two-call chain
    gu = torch.empty(R, 2 * H, dtype=torch.bfloat16, device=dev)
    hq.hq_group_contiguous_gemm("mxfp8", aq, asf, wq, wsf, ge, gu, bias=bias)
    q2 = torch.full((R, H), FILL, dtype=torch.uint8, device=dev)
    sf2 = torch.full((R, H // 32), FILL, dtype=torch.uint8, device=dev)
    y2 = torch.full((R, H), -7.0, dtype=torch.float32, device=dev)
    hq.hq_fused_swiglu_quant("mxfp8", gu, q2, sf2, E, ge, 0, valid, y_debug=y2)
    torch.cuda.synchronize()
    return (U.host_u8(aq), U.host_u8(asf), U.host_u8(wq).reshape(E * 2 * H, K),
            U.host_u8(wsf).reshape(E * 2 * H, K // 32), (q, sf, y), (q2, sf2, y2), U.host_bits(gu))


CASES = [
    # counts, group alignment, K, H, bias
    ([40, 0, 70, 300], 32, 512, 128, False),      # K % 512 == 0: grouped scale loads; 300 rows > one tile
    ([17, 129, 0, 5], 16, 384, 256, True),        # K % 512 != 0: per-step scale planes; bias
    ([256, 1], 128, 1024, 384, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"K{c[2]}-H{c[3]}-{'bias' if c[4] else 'nobias'}")
def test_gemm_swiglu_quant_against_oracle_and_chain(case):
    counts, align, K, H, with_bias = case
    dev = U.require_gpu()
    U.banner(f"gemm+swiglu counts={counts} K={K} H={H} bias={with_bias}")
    counts, ends, starts, R, x, w, b = _inputs(counts, align, K, H, 5 + K + H, with_bias)
    ac, asc, wc, wsc, fused, chain, gu_dev = _run_both(dev, counts, ends, R, x, w, b, K, H)
    q, sf, y = (U.host_u8(fused[0]), U.host_u8(fused[1]), fused[2].cpu().numpy())
    # the call's contract: the same bits as the two-call chain, everywhere
    assert torch.equal(fused[0], chain[0]), "codes differ from the GEMM + SwiGLU chain"
    assert torch.equal(fused[1], chain[1]), "scales differ from the GEMM + SwiGLU chain"
    assert torch.equal(fused[2], chain[2]), "y differs from the GEMM + SwiGLU chain"
    written = np.zeros(R, bool)
    for g in range(len(counts)):
        lo, c = int(starts[g]), int(counts[g])
        written[lo:lo + c] = True
        if c == 0:
            continue
        rows = slice(lo, lo + c)
        wr = slice(g * 2 * H, (g + 1) * 2 * H)
        gu = G.dense_gemm("mxfp8", ac[rows], asc[rows], wc[wr], wsc[wr], None if b is None else b[g])
        ad, bd = U.deq("mxfp8", ac[rows], asc[rows]), U.deq("mxfp8", wc[wr], wsc[wr])
        # the gate|up output the epilogue rounds (the chain's) is within the GEMM bound
        U.assert_gemm_close(gu_dev[rows], gu, ad, bd, what=f"group {g} gate|up")
        # y per element: against float64 SwiGLU of that same BF16 gate|up ...
        U.assert_y_close(y[rows], gu_dev[rows], H, what=f"group {g} y (device gate|up)")
        # ... and against the oracle's GEMM + SwiGLU, the GEMM bound carried through
        U.assert_y_close_to_gemm_oracle(y[rows], gu, G.tolerance(ad, bd), H, what=f"group {g} y (oracle GEMM)")
        qc, qs = Q.mx_quant_values(y[rows].astype(np.float64), "mxfp8")
        assert np.array_equal(q[rows], qc), f"group {g}: codes are not the quantisation of y"
        assert np.array_equal(sf[rows], qs), f"group {g}: scales are not those of y"
    assert (q[~written] == FILL).all() and (sf[~written] == FILL).all(), "rows past the valid counts were written"


def test_gemm_swiglu_quant_rejects_what_it_cannot_run():
    dev = U.require_gpu()
    E, H, K, R = 2, 128, 512, 64
    a = torch.zeros(R, K, dtype=torch.uint8, device=dev)
    sa = torch.zeros(R, K // 32, dtype=torch.uint8, device=dev)
    b = torch.zeros(E, 2 * H, K, dtype=torch.uint8, device=dev)
    sb = torch.zeros(E, 2 * H, K // 32, dtype=torch.uint8, device=dev)
    ge = torch.tensor([32, 64], dtype=torch.int32, device=dev)
    q = torch.zeros(R, H, dtype=torch.uint8, device=dev)
    sf = torch.zeros(R, H // 32, dtype=torch.uint8, device=dev)
    with pytest.raises(hq.HQError) as e:          # MXFP4 codes: not supported by this call
        hq.hq_group_contiguous_gemm_swiglu_quant("mxfp4", a[:, :K // 2].contiguous(), sa, b[..., :K // 2].contiguous(),
                                                 sb, ge, q, sf)
    assert e.value.status == -4
    lib = hq.load()
    st = hq._stream(a)
    # h not a multiple of 128
    assert lib.hq_group_contiguous_gemm_swiglu_quant(st, 0, hq._p(a), hq._p(sa), hq._p(b), hq._p(sb), hq._p(ge), E,
                                                     None, None, hq._p(q), hq._p(sf), None, R, 96, K, 0) == -2
    # a single K step (the tiled kernel needs two)
    assert lib.hq_group_contiguous_gemm_swiglu_quant(st, 0, hq._p(a), hq._p(sa), hq._p(b), hq._p(sb), hq._p(ge), E,
                                                     None, None, hq._p(q), hq._p(sf), None, R, H, 128, 0) == -2
    torch.cuda.synchronize()
    assert (U.host_u8(q) == 0).all(), "a rejected call wrote its output"


def test_gemm_swiglu_quant_moe_full_size_equals_chain():
    """The MoE workload (32 experts, 65536 routed rows padded to 128, K=4096,
    gate|up N=3072): the fused call writes the same bits as the two calls."""
    dev = U.require_gpu()
    U.banner("gemm+swiglu MoE full size E=32 K=4096 H=1536")
    d = synth.moe_contiguous(threads=16)
    counts, ends = d["counts"], d["group_end"]
    R, K, N, H, E = int(ends[-1]), d["K"], d["N"], d["H"], len(counts)
    qa, sa, _ = hq.quantize(U.dev_bf16(d["a"], dev), "mxfp8")
    qw, sw, _ = hq.quantize(U.dev_bf16(d["b"].reshape(E * N, K), dev), "mxfp8")
    qw, sw = qw.view(E, N, K), sw.view(E, N, K // 32)
    ge, valid = U.dev_i32(ends, dev), U.dev_i32(counts, dev)
    q = torch.full((R, H), FILL, dtype=torch.uint8, device=dev)
    sf = torch.full((R, H // 32), FILL, dtype=torch.uint8, device=dev)
    hq.hq_group_contiguous_gemm_swiglu_quant("mxfp8", qa, sa, qw, sw, ge, q, sf, valid=valid)
    gu = torch.empty(R, N, dtype=torch.bfloat16, device=dev)
    hq.hq_group_contiguous_gemm("mxfp8", qa, sa, qw, sw, ge, gu)
    q2 = torch.full((R, H), FILL, dtype=torch.uint8, device=dev)
    sf2 = torch.full((R, H // 32), FILL, dtype=torch.uint8, device=dev)
    hq.hq_fused_swiglu_quant("mxfp8", gu, q2, sf2, E, ge, 0, valid)
    torch.cuda.synchronize()
    assert torch.equal(q, q2), f"{int((q != q2).sum())} codes differ"
    assert torch.equal(sf, sf2), f"{int((sf != sf2).sum())} scales differ"
    del qa, qw, gu, q, q2
    torch.cuda.empty_cache()


def test_gemm_swiglu_quant_moe_full_size_against_oracle():
    """The MoE workload at full size, sampled rows of the smallest, largest,
    first and last experts (all 1536 y columns of each): the device's y within
    the GEMM bound carried through SwiGLU of the oracle's GEMM + SwiGLU, and
    the codes / scales bit-exact with the oracle's quantisation of that y."""
    dev = U.require_gpu()
    U.banner("gemm+swiglu MoE full size E=32 K=4096 H=1536 against the oracle (sampled rows)")
    d = synth.moe_contiguous(threads=16)
    counts, ends, starts = d["counts"], d["group_end"], d["starts"]
    R, K, N, H, E = int(ends[-1]), d["K"], d["N"], d["H"], len(counts)
    qa, sa, _ = hq.quantize(U.dev_bf16(d["a"], dev), "mxfp8")
    wbits = d["b"].reshape(E * N, K)
    qw, sw, _ = hq.quantize(U.dev_bf16(wbits, dev), "mxfp8")
    ge, valid = U.dev_i32(ends, dev), U.dev_i32(counts, dev)
    q = torch.full((R, H), FILL, dtype=torch.uint8, device=dev)
    sf = torch.full((R, H // 32), FILL, dtype=torch.uint8, device=dev)
    y = torch.full((R, H), -7.0, dtype=torch.float32, device=dev)
    hq.hq_group_contiguous_gemm_swiglu_quant("mxfp8", qa, sa, qw.view(E, N, K), sw.view(E, N, K // 32), ge, q, sf,
                                             valid=valid, y_debug=y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(55)
    experts = sorted({0, E - 1, int(np.argmin(counts)), int(np.argmax(counts))})
    for g in experts:
        lo, c = int(starts[g]), int(counts[g])
        local = sorted({0, c - 1, min(255, c - 1), min(256, c - 1)} | {int(v) for v in rng.integers(0, c, 5)})
        rows = np.array([lo + v for v in local], np.int64)
        rt = torch.from_numpy(rows).to(dev)
        ac, asc = Q.mx_quant_bf16(d["a"][rows], "mxfp8")
        wc, wsc = Q.mx_quant_bf16(wbits[g * N:(g + 1) * N], "mxfp8")
        assert np.array_equal(U.host_u8(qa[rt]), ac) and np.array_equal(U.host_u8(sa[rt]), asc), "A codes"
        gu = G.dense_gemm("mxfp8", ac, asc, wc, wsc)
        ad, bd = U.deq("mxfp8", ac, asc), U.deq("mxfp8", wc, wsc)
        yd = y[rt].cpu().numpy()
        U.assert_y_close_to_gemm_oracle(yd, gu, G.tolerance(ad, bd), H, what=f"expert {g} (count {c})")
        qc, qs = Q.mx_quant_values(yd.astype(np.float64), "mxfp8")
        assert np.array_equal(U.host_u8(q[rt]), qc), f"expert {g}: codes are not the quantisation of y"
        assert np.array_equal(U.host_u8(sf[rt]), qs), f"expert {g}: scales are not those of y"
    del qa, qw, q, y
    torch.cuda.empty_cache()
