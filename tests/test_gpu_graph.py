"""The calls under graph capture (flashrt/fp4-gemm page, large-M tier: a
caller-owned workspace allocated before capture and passed on every replay).

Every tensor -- inputs, outputs, the K-split workspace, the pointer arrays of
the discrete-weights call -- is allocated before capture; the captured
sequence is MXFP8 activation quantisation, NVFP4 quantisation with its amax
pass, the grouped gate|up GEMM with the SwiGLU + re-quant epilogue, a K-split
dense GEMM (workspace), a tail-split dense GEMM (workspace, CU limit), a
stream-K dense GEMM (workspace, CU limit: its flag words are cleared by the
call itself, so every replay starts from the state the previous one left),
the discrete-weights grouped GEMM, a K-split batch GEMM (workspace), the masked
grouped GEMM, the standalone SwiGLU + re-quant and the backward dSwiGLU GEMM
in both output forms (dprob cleared by a fill kernel inside the graph; its
FP32 atomic adds have no fixed order, so dprob is compared within 1e-5
relative, everything else bit for bit).  The graph is replayed several times with the
program's own eager work (outputs overwritten, other launches) and
synchronisations between replays; every replay must give the eager results
bit for bit.  The library records no memset node (its counters and the
NVFP4 amax are cleared by kernels).
"""
import numpy as np
import pytest
import torch

import fp4_gemm_moe_amd as hq
import synth
from tests import _gpu as U

pytestmark = pytest.mark.gpu


def _setup(dev):
    rng = np.random.default_rng(91)
    E, K, H = 4, 512, 128
    counts = np.array([40, 0, 300, 77], np.int64)
    ends, _ = synth.padded_group_ends(counts, 32)
    R = int(ends[-1])
    st = {}
    st["x"] = U.dev_bf16(synth.normal_bf16(rng, (R, K)), dev)
    st["xn"] = U.dev_bf16(synth.normal_bf16(rng, (96, 1024)), dev)
    wq, wsf, _ = hq.quantize(U.dev_bf16(synth.normal_bf16(rng, (E * 2 * H, K), 0.05), dev), "mxfp8")
    st["wq"], st["wsf"] = wq.view(E, 2 * H, K), wsf.view(E, 2 * H, K // 32)
    st["ge"], st["valid"] = U.dev_i32(ends, dev), U.dev_i32(counts, dev)
    st["aq"] = torch.empty(R, K, dtype=torch.uint8, device=dev)
    st["asf"] = torch.empty(R, K // 32, dtype=torch.uint8, device=dev)
    st["nq"] = torch.empty(96, 512, dtype=torch.uint8, device=dev)
    st["nsf"] = torch.empty(96, 64, dtype=torch.uint8, device=dev)
    st["ng"] = torch.empty(1, dtype=torch.float32, device=dev)
    st["yq"] = torch.empty(R, H, dtype=torch.uint8, device=dev)
    st["ysf"] = torch.empty(R, H // 32, dtype=torch.uint8, device=dev)
    # K-split dense: 300 x 520 x 8576 (6 tiles, 67 K steps)
    m, n, k = 300, 520, 8576
    st["da"], st["dsa"], _ = hq.quantize(U.dev_bf16(synth.normal_bf16(rng, (m, k)), dev), "mxfp8")
    st["db"], st["dsb"], _ = hq.quantize(U.dev_bf16(synth.normal_bf16(rng, (n, k), 0.05), dev), "mxfp8")
    st["dout"] = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    st["dws"] = hq.gemm_workspace("mxfp8", m, n, k, device=dev)
    assert st["dws"] is not None
    # tail split: 520 x 1544 x 6144 on 16 CUs
    m2, n2, k2 = 520, 1544, 6144
    st["ta"], st["tsa"], _ = hq.quantize(U.dev_bf16(synth.normal_bf16(rng, (m2, k2)), dev), "mxfp8")
    st["tb"], st["tsb"], _ = hq.quantize(U.dev_bf16(synth.normal_bf16(rng, (n2, k2), 0.05), dev), "mxfp8")
    st["tout"] = torch.empty(m2, n2, dtype=torch.bfloat16, device=dev)
    st["tws"] = hq.gemm_workspace("mxfp8", m2, n2, k2, cu_limit=16, device=dev)
    assert st["tws"] is not None
    # stream-K: 256 x 2560 x 16384 on 24 CUs (10 tiles, 1-2 per group of 3 workgroups, runs of
    # 10-22 of their 32 K units)
    m3, n3, k3 = 256, 2560, 16384
    st["sa"], st["ssa"], _ = hq.quantize(U.dev_bf16(synth.normal_bf16(rng, (m3, k3)), dev), "mxfp8")
    st["sb"], st["ssb"], _ = hq.quantize(U.dev_bf16(synth.normal_bf16(rng, (n3, k3), 0.05), dev), "mxfp8")
    st["skout"] = torch.empty(m3, n3, dtype=torch.bfloat16, device=dev)
    st["skws"] = hq.gemm_workspace("mxfp8", m3, n3, k3, cu_limit=24, device=dev)
    assert st["skws"] is not None
    # discrete weights: per-expert tensors and their address arrays, built now
    st["bs"] = [st["wq"][g].clone() for g in range(E)]
    st["sfbs"] = [st["wsf"][g].clone() for g in range(E)]
    st["bp"], st["sp"] = hq.ptr_arrays("mxfp8", st["bs"], st["sfbs"], 2 * H, K)
    st["pout"] = torch.empty(R, 2 * H, dtype=torch.bfloat16, device=dev)
    # batch: 3 x 64 x 256 x 4096 (K split into the workspace)
    Bn, bm, bn, bk = 3, 64, 256, 4096
    qa, sa, _ = hq.quantize(U.dev_bf16(synth.normal_bf16(rng, (Bn * bm, bk)), dev), "mxfp8")
    qb, sb, _ = hq.quantize(U.dev_bf16(synth.normal_bf16(rng, (Bn * bn, bk), 0.05), dev), "mxfp8")
    st["ba"], st["bsa"] = qa.view(Bn, bm, bk), sa.view(Bn, bm, bk // 32)
    st["bb"], st["bsb"] = qb.view(Bn, bn, bk), sb.view(Bn, bn, bk // 32)
    st["bout"] = torch.empty(Bn, bm, bn, dtype=torch.bfloat16, device=dev)
    st["bws"] = hq.gemm_workspace("mxfp8", bm, bn, bk, batch=Bn, device=dev)
    # masked: 4 slots of 64 rows (counts 10, 0, 64, 33), K = 512, N = 2H
    mq, msf, _ = hq.quantize(U.dev_bf16(synth.normal_bf16(rng, (E * 64, K)), dev), "mxfp8")
    st["ma"], st["msa"] = mq, msf
    st["mcnt"] = U.dev_i32(np.array([10, 0, 64, 33], np.int64), dev)
    st["mout"] = torch.empty(E * 64, 2 * H, dtype=torch.bfloat16, device=dev)
    # standalone SwiGLU + re-quant of a [R, 2H] BF16 gate|up buffer
    st["gu"] = U.dev_bf16(synth.normal_bf16(rng, (R, 2 * H)), dev)
    st["sq"] = torch.empty(R, H, dtype=torch.uint8, device=dev)
    st["ssf"] = torch.empty(R, H // 32, dtype=torch.uint8, device=dev)
    # backward dSwiGLU: R = aq * wq[g]^T (n = 2H), C [R, 4H], prob [R]
    st["cc"] = U.dev_bf16(synth.normal_bf16(rng, (R, 4 * H)), dev)
    st["prob"] = torch.from_numpy(rng.random(R).astype(np.float32)).to(dev)
    st["dprob"] = torch.empty(R, dtype=torch.float32, device=dev)
    st["dprobq"] = torch.empty(R, dtype=torch.float32, device=dev)
    st["dd"] = torch.empty(R, 4 * H, dtype=torch.bfloat16, device=dev)
    st["dq"] = torch.empty(R, 4 * H, dtype=torch.uint8, device=dev)
    st["dsf"] = torch.empty(R, 4 * H // 32, dtype=torch.uint8, device=dev)
    return st


OUTS = ["aq", "asf", "nq", "nsf", "ng", "yq", "ysf", "dout", "tout", "skout", "pout", "bout", "mout", "sq",
        "ssf", "dd", "dq", "dsf"]
CLOSE = ["dprob", "dprobq"]


def _calls(st):
    hq.hq_group_wise_quant("mxfp8", st["x"], st["aq"], st["asf"])
    hq.hq_group_wise_quant("nvfp4", st["xn"], st["nq"], st["nsf"], st["ng"])
    hq.hq_group_contiguous_gemm_swiglu_quant("mxfp8", st["aq"], st["asf"], st["wq"], st["wsf"], st["ge"],
                                             st["yq"], st["ysf"], valid=st["valid"])
    hq.hq_dense_gemm("mxfp8", st["da"], st["dsa"], st["db"], st["dsb"], st["dout"], workspace=st["dws"])
    hq.hq_dense_gemm("mxfp8", st["ta"], st["tsa"], st["tb"], st["tsb"], st["tout"], cu_limit=16,
                     workspace=st["tws"])
    hq.hq_dense_gemm("mxfp8", st["sa"], st["ssa"], st["sb"], st["ssb"], st["skout"], cu_limit=24,
                     workspace=st["skws"])
    hq.hq_group_contiguous_gemm_ptr_array("mxfp8", st["aq"], st["asf"], st["bp"], st["sp"], st["ge"],
                                          st["pout"], n=st["pout"].shape[1])
    hq.hq_batch_gemm("mxfp8", st["ba"], st["bsa"], st["bb"], st["bsb"], st["bout"], workspace=st["bws"])
    hq.hq_group_masked_gemm("mxfp8", st["ma"], st["msa"], st["wq"], st["wsf"], st["mcnt"], st["mout"], 64)
    hq.hq_fused_swiglu_quant("mxfp8", st["gu"], st["sq"], st["ssf"], 4, group_end=st["ge"], valid=st["valid"])
    st["dprob"].zero_()
    st["dprobq"].zero_()
    hq.hq_group_contiguous_gemm_dswiglu("mxfp8", st["aq"], st["asf"], st["wq"], st["wsf"], st["ge"], st["cc"],
                                        st["prob"], st["dprob"], st["dd"])
    hq.hq_group_contiguous_gemm_dswiglu_quant("mxfp8", st["aq"], st["asf"], st["wq"], st["wsf"], st["ge"],
                                              st["cc"], st["prob"], st["dprobq"], st["dq"], st["dsf"])


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.uint8)


def _snapshot(st):
    return {k: st[k].clone() for k in OUTS + CLOSE}


def _scribble(st):
    for k in OUTS + CLOSE:
        v = st[k]
        if v.dtype == torch.float32:
            v.fill_(-3.0)
        else:
            v.view(torch.uint8).fill_(0xA7)


def test_graph_capture_and_replay_equal_eager():
    dev = U.require_gpu()
    U.banner("graph capture: quant, nvfp4 quant, gemm+swiglu, k-split, tail split, ptr-array, batch, masked, "
             "swiglu, dswiglu (bf16 and row-quantised)")
    st = _setup(dev)
    _scribble(st)                   # rows a call does not write hold the fill byte in every run
    _calls(st)                      # eager run (also sets the kernels' launch attributes)
    torch.cuda.synchronize()
    want = _snapshot(st)
    _scribble(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _calls(st)
    torch.cuda.synchronize()
    for rep in range(3):
        U.banner(f"graph replay {rep}")
        _scribble(st)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(_bits(st[k]), _bits(want[k])), f"replay {rep}: {k} differs from the eager run"
        for k in CLOSE:
            assert torch.allclose(st[k], want[k], rtol=1e-5, atol=1e-6), f"replay {rep}: {k}"
        # eager work between replays: the same calls outside the graph, then other launches
        _calls(st)
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(_bits(st[k]), _bits(want[k])), f"eager run after replay {rep}: {k}"
        for k in CLOSE:
            assert torch.allclose(st[k], want[k], rtol=1e-5, atol=1e-6), f"eager run after replay {rep}: {k}"
        torch.randn(1 << 20, device=dev).sum().item()
    del g
