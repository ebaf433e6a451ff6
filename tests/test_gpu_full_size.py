"""GPU parity at the full workload sizes, on sampled outputs.

The launches are the ones bench.py times (same shapes, same forms, same
default CU count); the oracle cannot afford the whole products, so it
recomputes selected rows x columns one by one from its own quantisation of
the same seeded BF16 inputs (quantisation is per row, so quantising only the
sampled rows gives the same codes; the NVFP4 global scale comes from the
oracle's amax over the whole tensor).  The device codes of the sampled rows
must equal the oracle's bit for bit, and the sampled outputs must meet the
acceptance bound.

* Dense MXFP4 / NVFP4: all 24 (N, K, M, mode) shapes of the flashrt/fp4-gemm
  page's qualification grid (M in {1, 16} take the direct kernel, M in
  {512, 4096} the tiled one).
* Grouped-contiguous MXFP8, 32 experts, 65536 routed rows padded to 128 per
  expert, K=4096, N=3072 (the MoE step): sampled rows of the smallest, the
  largest, the first and the last expert, padding rows included.
* Grouped-masked MXFP4, 64 experts x 256-row slots, K=7168, N=4096, with
  random bytes in the padded rows: sampled valid rows, and every padded
  output row keeps its sentinel; and every valid row (all 9291) equals, bit
  for bit, the grouped-contiguous GEMM on the gathered valid rows with
  unpadded offsets (same kernel, same K order).
"""
import numpy as np
import pytest
import torch

import fp4_gemm_moe_amd as hq
import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from tests import _gpu as U

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1


def _cols(n, rng, extra=24):
    """Column sample: both ends, the edges of 256-column tiles, random."""
    base = {0, n - 1}
    for t in (255, 256, 511, 512, n - 256, n - 257):
        if 0 <= t < n:
            base.add(t)
    base.update(int(c) for c in rng.choice(n, size=min(extra, n), replace=False))
    return np.array(sorted(base), np.int64)


def _rows(m, rng, extra=6):
    base = {0, m - 1}
    for t in (15, 16, 255, 256):
        if 0 <= t < m:
            base.add(t)
    base.update(int(r) for r in rng.choice(m, size=min(extra, m), replace=False))
    return np.array(sorted(base), np.int64)


def _oracle_quant(bits, mode, g=None):
    if mode == "nvfp4":
        c, s, gg = Q.nvfp4_quant_bf16(bits, g)
        return c, s, gg
    c, s = Q.mx_quant_bf16(bits, mode)
    return c, s, None


def _amax_bf16(bits):
    """max |x| of a BF16 bit array without decoding it whole: the magnitude
    order of non-negative BF16 patterns is their integer order."""
    mag = np.max(np.asarray(bits, np.uint16) & np.uint16(0x7FFF))
    return F.bf16_decode(np.array([mag], np.uint16))[0]


def _check_block(mode, out_dev, rows, cols, a_bits_rows, b_bits_cols, q_a_dev, q_b_dev, sf_a_dev, sf_b_dev,
                 g_a=None, g_b=None, what="", b_rows=None):
    """out[rows][:, cols] against the oracle; b_rows: the weight rows behind
    cols in q_b_dev (cols itself for a dense GEMM)."""
    b_rows = cols if b_rows is None else b_rows
    ca, sa, _ = _oracle_quant(a_bits_rows, mode, g_a)
    cb, sb, _ = _oracle_quant(b_bits_cols, mode, g_b)
    # device codes of the sampled rows equal the oracle's
    assert np.array_equal(U.host_u8(q_a_dev[torch.from_numpy(rows)]), ca), f"{what}: A codes"
    assert np.array_equal(U.host_u8(sf_a_dev[torch.from_numpy(rows)]), sa), f"{what}: A scales"
    assert np.array_equal(U.host_u8(q_b_dev[torch.from_numpy(b_rows)]), cb), f"{what}: B codes"
    assert np.array_equal(U.host_u8(sf_b_dev[torch.from_numpy(b_rows)]), sb), f"{what}: B scales"
    alpha = None if g_a is None else np.float32(np.float32(g_a) * np.float32(g_b))
    ref = G.dense_gemm_rows_cols(mode, ca, sa, cb, sb, np.arange(len(rows)), np.arange(len(cols)),
                                 alpha=alpha)
    got = U.host_bits(out_dev[torch.from_numpy(rows)][:, torch.from_numpy(cols)])
    U.assert_gemm_close(got, ref, U.deq(mode, ca, sa), U.deq(mode, cb, sb), alpha=alpha, what=what)


# ------------------------------------------------------------- dense grid
_W_CACHE = {}


def _dense_inputs(n, k, m):
    if (n, k) not in _W_CACHE:
        _W_CACHE.clear()
        _W_CACHE[(n, k)] = synth.dense_fp4_large_weights(n, k)
    return {"a": synth.dense_fp4_large_acts(n, k, m), "b": _W_CACHE[(n, k)]}


@pytest.mark.parametrize("mode", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("m", synth.LARGE_M, ids=lambda v: f"M{v}")
@pytest.mark.parametrize("nk", synth.LARGE_NK, ids=lambda t: f"N{t[0]}_K{t[1]}")
def test_dense_qualification_grid_sampled(nk, m, mode):
    dev = U.require_gpu()
    n, k = nk
    U.banner(f"dense {mode} M={m} N={n} K={k} (full size, sampled)")
    d = _dense_inputs(n, k, m)
    a_bits, b_bits = d["a"], d["b"]
    xa, xb = U.dev_bf16(a_bits, dev), U.dev_bf16(b_bits, dev)
    qa, sa, ga = hq.quantize(xa, mode)
    qb, sb, gb = hq.quantize(xb, mode)
    alpha = (ga * gb) if mode == "nvfp4" else None
    out = torch.full((m, n), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    # with the workspace the shape asks for, as bench.py runs it (K split at M = 512, tail split at 4096)
    hq.hq_dense_gemm(mode, qa, sa, qb, sb, out, alpha=alpha, workspace=hq.gemm_workspace(mode, m, n, k, device=dev))
    torch.cuda.synchronize()
    g_a = g_b = None
    if mode == "nvfp4":
        g_a = Q.nvfp4_global_scale(_amax_bf16(a_bits))
        g_b = Q.nvfp4_global_scale(_amax_bf16(b_bits))
        assert np.float32(ga.item()) == g_a and np.float32(gb.item()) == g_b, "global scales"
    rng = np.random.default_rng(1000 + m)
    rows, cols = _rows(m, rng), _cols(n, rng)
    _check_block(mode, out, rows, cols, a_bits[rows], b_bits[cols], qa, qb, sa, sb, g_a, g_b,
                 what=f"{mode} M{m} N{n} K{k}")
    del xa, xb, qa, qb, out
    torch.cuda.empty_cache()


# ------------------------------------------------------- MoE contiguous
def test_moe_contiguous_mxfp8_full_size_sampled():
    dev = U.require_gpu()
    U.banner("grouped-contiguous MXFP8 E=32 R=67840 K=4096 N=3072 (full size, sampled)")
    d = synth.moe_contiguous(threads=16)
    counts, ends, starts = d["counts"], d["group_end"], d["starts"]
    R, K, N, E = int(ends[-1]), d["K"], d["N"], len(counts)
    xa = U.dev_bf16(d["a"], dev)
    xw = U.dev_bf16(d["b"].reshape(E * N, K), dev)
    qa, sa, _ = hq.quantize(xa, "mxfp8")
    qw, sw, _ = hq.quantize(xw, "mxfp8")
    del xa, xw
    out = torch.full((R, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    hq.hq_group_contiguous_gemm("mxfp8", qa, sa, qw.view(E, N, K), sw.view(E, N, K // 32),
                                U.dev_i32(ends, dev), out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    experts = sorted({0, E - 1, int(np.argmin(counts)), int(np.argmax(counts))})
    for g in experts:
        lo, hi, c = int(starts[g]), int(ends[g]), int(counts[g])
        # valid rows (ends, tile edges, random) and padding rows of the group
        local = {0, c - 1, min(c, hi - lo - 1)} | {int(v) for v in rng.integers(0, max(c, 1), 4)}
        local |= {t for t in (255, 256) if t < hi - lo}
        rows = np.array(sorted(lo + v for v in local if 0 <= v < hi - lo), np.int64)
        cols = _cols(N, rng, 16)
        wrows = g * N + cols
        _check_block("mxfp8", out, rows, cols, d["a"][rows], d["b"].reshape(E * N, K)[wrows],
                     qa, qw, sa, sw, what=f"expert {g} (count {c})", b_rows=wrows)
    del qa, qw, out
    torch.cuda.empty_cache()


# ----------------------------------------------------------- MoE masked
def test_moe_masked_mxfp4_full_size_sampled():
    dev = U.require_gpu()
    U.banner("grouped-masked MXFP4 E=64 Mmax=256 K=7168 N=4096 (full size, sampled, garbage padding)")
    d = synth.moe_masked(threads=16)
    counts, Mmax, K, N = d["counts"], d["max_m"], d["K"], d["N"]
    E = len(counts)
    xa = U.dev_bf16(d["a"], dev)
    qa, sa, _ = hq.quantize(xa, "mxfp4")
    del xa
    # padded rows of every slot: random code and scale bytes
    garb_q = synth.garbage_bytes(d["garbage_seed"], (E * Mmax, K // 2))
    garb_s = synth.garbage_bytes(d["garbage_seed"] + 1, (E * Mmax, K // 32))
    pad = np.ones(E * Mmax, bool)
    for e in range(E):
        pad[e * Mmax:e * Mmax + int(counts[e])] = False
    pad_t = torch.from_numpy(pad).to(dev)
    qa[pad_t] = U.dev_u8(garb_q[pad], dev)
    sa[pad_t] = U.dev_u8(garb_s[pad], dev)
    xw = U.dev_bf16(d["b"].reshape(E * N, K), dev)
    qw, sw, _ = hq.quantize(xw, "mxfp4")
    del xw
    out = torch.full((E * Mmax, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    hq.hq_group_masked_gemm("mxfp4", qa, sa, qw.view(E, N, K // 2), sw.view(E, N, K // 32),
                            U.dev_i32(counts, dev), out, Mmax)
    torch.cuda.synchronize()
    # padded rows are untouched
    o = out.view(torch.int16)
    assert bool((o[pad_t] == SENTINEL).all()), "a padded row was written"
    rng = np.random.default_rng(44)
    nz = np.flatnonzero(counts)
    experts = sorted({int(nz[0]), int(nz[-1]), int(nz[np.argmin(counts[nz])]), int(np.argmax(counts))})
    for e in experts:
        c = int(counts[e])
        local = {0, c - 1} | {int(v) for v in rng.integers(0, c, 4)}
        rows = np.array(sorted(e * Mmax + v for v in local), np.int64)
        cols = _cols(N, rng, 16)
        wrows = e * N + cols
        _check_block("mxfp4", out, rows, cols, d["a"][rows], d["b"].reshape(E * N, K)[wrows],
                     qa, qw, sa, sw, what=f"expert {e} (count {c})", b_rows=wrows)
    # the masked form equals the contiguous form on the gathered valid rows
    valid_t = torch.from_numpy(np.flatnonzero(~pad)).to(dev)
    T = int(counts.sum())
    assert valid_t.numel() == T
    ends = np.cumsum(counts).astype(np.int32)
    qa_c, sa_c = qa[valid_t].contiguous(), sa[valid_t].contiguous()
    out_c = torch.full((T, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    hq.hq_group_contiguous_gemm("mxfp4", qa_c, sa_c, qw.view(E, N, K // 2), sw.view(E, N, K // 32),
                                U.dev_i32(ends, dev), out_c)
    torch.cuda.synchronize()
    same = torch.equal(out[valid_t].view(torch.int16), out_c.view(torch.int16))
    ndiff = int((out[valid_t].view(torch.int16) != out_c.view(torch.int16)).sum())
    assert same, f"masked != contiguous on the gathered valid rows: {ndiff} of {T * N} outputs differ"
    del qa, qw, out, out_c, qa_c
    torch.cuda.empty_cache()
