"""GPU parity of the scaled GEMMs (dense, batch, grouped-contiguous,
grouped-masked) against the oracle.

* Integer-coded inputs (small-integer codes, unit scales) make every product
  and partial sum exact in FP32, so the result must be bit-exact; this pins
  the matrix-core lane layout, the scale operand and the output layout.
* Random inputs: the acceptance bound (2^-7 relative + 1e-3 ||a|| ||b||
  absolute, relative Frobenius <= 2e-3).
* Rows a call must not write keep a sentinel; padded rows hold garbage
  (random codes, 0xFF scales) that must not leak into valid rows.
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
from tests.test_oracle_gemm import INT_E2M1, INT_E4M3

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1   # a BF16 NaN pattern no kernel produces


def _code_lut(table):
    lut = np.zeros(int(max(table)) + 1, np.uint8)
    for v, c in table.items():
        lut[int(v)] = c
    return lut


def _int_operand(rng, rows, k, mode, choices):
    vals = rng.choice(np.array(choices), (rows, k))
    mag = np.abs(vals)
    if mode == "mxfp8":
        codes = _code_lut(INT_E4M3)[mag] | np.where(vals < 0, 0x80, 0).astype(np.uint8)
        sf = np.full((rows, k // 32), 127, np.uint8)
    else:
        c = _code_lut(INT_E2M1)[mag] | np.where(vals < 0, 0x8, 0).astype(np.uint8)
        codes = F.pack_nibbles(c)
        sf = np.full((rows, k // (16 if mode == "nvfp4" else 32)), 0x38 if mode == "nvfp4" else 127, np.uint8)
    return vals, codes, sf


def _quant(bits, mode):
    if mode == "nvfp4":
        c, s, g = Q.nvfp4_quant_bf16(bits)
        return c, s, np.float32(g)
    c, s = Q.mx_quant_bf16(bits, mode)
    return c, s, None


def _dense_gpu(mode, a, sfa, b, sfb, m, n, k, dev, bias=None, alpha=None, cu_limit=0, ws=False):
    """ws=True: with the workspace the shape asks for (which must be > 0: the
    case is meant to split K)."""
    out = torch.full((m, n), 0, dtype=torch.int16, device=dev).view(torch.bfloat16)
    workspace = None
    if ws:
        workspace = hq.gemm_workspace(mode, m, n, k, cu_limit=cu_limit, device=dev)
        assert workspace is not None, "the shape was expected to split K"
    hq.hq_dense_gemm(mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev), U.dev_u8(sfb, dev),
                     out, bias=None if bias is None else U.dev_bf16(bias, dev),
                     alpha=None if alpha is None else torch.tensor([alpha], dtype=torch.float32, device=dev),
                     cu_limit=cu_limit, workspace=workspace)
    torch.cuda.synchronize()
    return U.host_bits(out)


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("mnk", [(16, 16, 128), (64, 64, 256), (37, 72, 96), (5, 520, 512), (300, 136, 1024)])
def test_integer_exact_dense(mode, mnk):
    dev = U.require_gpu()
    m, n, k = mnk
    U.banner(f"int-exact dense {mode} m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 1000 + n + k)
    ch = [-2, -1, 0, 1, 2] if k <= 256 else [-1, 0, 1]
    av, a, sfa = _int_operand(rng, m, k, mode, ch)
    bv, b, sfb = _int_operand(rng, n, k, mode, ch)
    exact = av @ bv.T          # exact in FP32 partial sums; one rounding to BF16 on both sides
    got = _dense_gpu(mode, a, sfa, b, sfb, m, n, k, dev, alpha=1.0 if mode == "nvfp4" else None)
    want = F.bf16_round(exact.astype(np.float64))
    assert np.array_equal(got, want), f"{np.sum(got != want)} of {got.size} differ"


def test_integer_exact_scales_and_positions():
    """Distinct power-of-two scales per row and per K-group with one-hot codes:
    each output picks out exactly one product, exposing any scale/lane mix-up."""
    dev = U.require_gpu()
    m, n, k = 32, 32, 256
    rng = np.random.default_rng(1)
    a = np.zeros((m, k), np.uint8)
    b = np.zeros((n, k), np.uint8)
    hot_a = rng.integers(0, k, m)
    hot_b = hot_a[rng.integers(0, m, n)]
    a[np.arange(m), hot_a] = 0x38           # 1.0 in E4M3
    b[np.arange(n), hot_b] = 0x40           # 2.0
    sfa = rng.integers(120, 134, (m, k // 32)).astype(np.uint8)
    sfb = rng.integers(120, 134, (n, k // 32)).astype(np.uint8)
    got = _dense_gpu("mxfp8", a, sfa, b, sfb, m, n, k, dev)
    want = G.dense_gemm("mxfp8", a, sfa, b, sfb)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
def test_dense_random_small(mode):
    dev = U.require_gpu()
    d = synth.dense_mxfp8_256()
    for (m, n, k) in [(256, 256, 256), (33, 40, 160), (1, 64, 512), (16, 136, 4096)]:
        U.banner(f"dense {mode} m={m} n={n} k={k}")
        rng = np.random.default_rng(m + n + k)
        xa = d["a"][:m, :k] if (m, k) == (256, 256) else synth.normal_bf16(rng, (m, k))
        xb = d["b"][:n, :k] if (n, k) == (256, 256) else synth.normal_bf16(rng, (n, k), 0.5)
        a, sfa, ga = _quant(xa, mode)
        b, sfb, gb = _quant(xb, mode)
        alpha = None if ga is None else np.float32(ga * gb)
        got = _dense_gpu(mode, a, sfa, b, sfb, m, n, k, dev, alpha=alpha)
        want = G.dense_gemm(mode, a, sfa, b, sfb, alpha=alpha)
        U.assert_gemm_close(got, want, U.deq(mode, a, sfa), U.deq(mode, b, sfb), alpha, f"{mode} {m}x{n}x{k}")


@pytest.mark.parametrize("mnk", [(5, 520, 512), (300, 264, 512)], ids=["direct", "tiled"])
def test_nvfp4_scale_sign_bit_ignored(mnk):
    """UE4M3 scales are unsigned: a scale byte with bit 7 set decodes as the
    byte without it, in both the skinny and the tiled kernels."""
    dev = U.require_gpu()
    m, n, k = mnk
    U.banner(f"nvfp4 scale bit 7 m={m} n={n} k={k}")
    rng = np.random.default_rng(m + 17)
    a = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    sfa = (rng.integers(0x20, 0x48, (m, k // 16)) | (rng.integers(0, 2, (m, k // 16)) << 7)).astype(np.uint8)
    sfb = (rng.integers(0x20, 0x48, (n, k // 16)) | (rng.integers(0, 2, (n, k // 16)) << 7)).astype(np.uint8)
    got = _dense_gpu("nvfp4", a, sfa, b, sfb, m, n, k, dev, alpha=1.0)
    want = G.dense_gemm("nvfp4", a, sfa, b, sfb, alpha=np.float32(1.0))
    U.assert_gemm_close(got, want, U.deq("nvfp4", a, sfa), U.deq("nvfp4", b, sfb), np.float32(1.0), "scale bit 7")


# Few tiles and a long K: the tiled kernel splits K into slices (uneven here)
# whose FP32 partial tiles a second kernel sums before the BF16 rounding.
# K % 512 == 0 (MX) makes a row's scale bytes a multiple of 16, so the kernel
# loads each row's scales 16 bytes (several K steps) at a time and the slices
# start on those groups (17 groups over 8 slices here); other K take the
# per-step scale planes.
K_SPLIT_SHAPES = [("mxfp8", 300, 520, 8576), ("mxfp4", 200, 264, 8448), ("nvfp4", 130, 512, 8448),
                  ("mxfp8", 300, 520, 8704), ("mxfp4", 200, 264, 8704)]
_KS_IDS = [f"{c[0]}-k{c[3]}" for c in K_SPLIT_SHAPES]


@pytest.mark.parametrize("case", K_SPLIT_SHAPES, ids=_KS_IDS)
def test_k_split_integer_exact(case):
    dev = U.require_gpu()
    mode, m, n, k = case
    U.banner(f"k-split int-exact {mode} m={m} n={n} k={k}")
    rng = np.random.default_rng(k + m)
    av, a, sfa = _int_operand(rng, m, k, mode, [-1, 0, 1])
    bv, b, sfb = _int_operand(rng, n, k, mode, [-1, 0, 1])
    got = _dense_gpu(mode, a, sfa, b, sfb, m, n, k, dev, alpha=1.0 if mode == "nvfp4" else None, ws=True)
    want = F.bf16_round((av @ bv.T).astype(np.float64))
    assert np.array_equal(got, want), f"{np.sum(got != want)} of {got.size} differ"


@pytest.mark.parametrize("case", K_SPLIT_SHAPES, ids=_KS_IDS)
def test_k_split_random(case):
    dev = U.require_gpu()
    mode, m, n, k = case
    U.banner(f"k-split random {mode} m={m} n={n} k={k}")
    rng = np.random.default_rng(7 * k + n)
    a, sfa, ga = _quant(synth.normal_bf16(rng, (m, k)), mode)
    b, sfb, gb = _quant(synth.normal_bf16(rng, (n, k), 0.05), mode)
    alpha = None if ga is None else np.float32(ga * gb)
    bias = synth.normal_bf16(rng, (n,), 0.1) if mode == "mxfp8" else None
    got = _dense_gpu(mode, a, sfa, b, sfb, m, n, k, dev, bias=bias, alpha=alpha, ws=True)
    want = G.dense_gemm(mode, a, sfa, b, sfb, bias, alpha)
    U.assert_gemm_close(got, want, U.deq(mode, a, sfa), U.deq(mode, b, sfb), alpha, f"k-split {mode}")
    # without a workspace the same call runs unsplit, within the same bound
    plain = _dense_gpu(mode, a, sfa, b, sfb, m, n, k, dev, bias=bias, alpha=alpha)
    U.assert_gemm_close(plain, want, U.deq(mode, a, sfa), U.deq(mode, b, sfb), alpha, f"unsplit {mode}")


# A dense launch whose last round of tiles is at most half full: the leading
# tiles run unsplit and the last ones -- whole n-tile columns of the last
# block of 4 m-tiles -- run K-split as a sub-problem whose reduce writes into
# the full-width output.  It is taken for long K only (48 FP8, 40 FP4 or 12
# NVFP4 steps and more).  A CU limit sets the round size at these sizes:
#   520 x 1544 (3 x 7 tiles, 16 CUs): 5 tail tiles -> 2 columns x 3 m-tiles,
#     the rectangle spans every row, 2 slices; 1100 x 1544 (5 x 7 tiles, 32
#     CUs): 3 tail tiles -> 3 columns of the ragged fifth m-tile (rows
#     1024..1099), 8 uneven slices of 49 or 41 K steps.
TAIL_SPLIT_CASES = [("mxfp8", 520, 1544, 6144, 16), ("mxfp8", 1100, 1544, 6272, 32),
                    ("mxfp4", 1100, 1544, 10496, 32), ("nvfp4", 520, 1544, 3072, 16)]


@pytest.mark.parametrize("case", TAIL_SPLIT_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-cu{c[4]}")
def test_tail_split_integer_exact(case):
    mode, m, n, k, cus = case
    dev = U.require_gpu()
    U.banner(f"tail split int-exact {mode} m={m} n={n} k={k} cu_limit={cus}")
    rng = np.random.default_rng(m + n + k)
    av, a, sfa = _int_operand(rng, m, k, mode, [-1, 0, 1])
    bv, b, sfb = _int_operand(rng, n, k, mode, [-1, 0, 1])
    got = _dense_gpu(mode, a, sfa, b, sfb, m, n, k, dev, alpha=1.0 if mode == "nvfp4" else None, cu_limit=cus,
                     ws=True)
    want = F.bf16_round(av.astype(np.float64) @ bv.astype(np.float64).T)   # exact: |sums| <= k
    assert np.array_equal(got, want), f"{np.sum(got != want)} of {got.size} differ"


@pytest.mark.parametrize("case", TAIL_SPLIT_CASES[1:2] + TAIL_SPLIT_CASES[3:],
                         ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-cu{c[4]}")
def test_tail_split_random_with_bias_or_alpha(case):
    mode, m, n, k, cus = case
    dev = U.require_gpu()
    U.banner(f"tail split random {mode} m={m} n={n} k={k} cu_limit={cus}")
    rng = np.random.default_rng(3 * m + k)
    a, sfa, ga = _quant(synth.normal_bf16(rng, (m, k)), mode)
    b, sfb, gb = _quant(synth.normal_bf16(rng, (n, k), 0.05), mode)
    alpha = None if ga is None else np.float32(ga * gb)
    bias = synth.normal_bf16(rng, (n,), 0.1) if mode == "mxfp8" else None
    got = _dense_gpu(mode, a, sfa, b, sfb, m, n, k, dev, bias=bias, alpha=alpha, cu_limit=cus, ws=True)
    want = G.dense_gemm(mode, a, sfa, b, sfb, bias, alpha)
    U.assert_gemm_close(got, want, U.deq(mode, a, sfa), U.deq(mode, b, sfb), alpha, f"tail split {mode}")


def test_workspace_size_query():
    """The size query follows the split plan: 16 KB of stream-K flag words,
    then S slices x rows x columns FP32 (K split: the whole output; tail
    split: the last round's rectangle), 0 where the call never splits (many
    tiles, short K, the direct kernel, the grouped forms' shapes)."""
    U.require_gpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    hdr = 16384
    # (mxfp8, 300 x 520 x 8576): 2 x 3 = 6 tiles, 67 K steps -> S = min(cus / 6, 16, 8) = 8
    assert hq.hq_gemm_workspace_size("mxfp8", 300, 520, 8576) == hdr + min(cus // 6, 8) * 300 * 520 * 4
    # tail split of 520 x 1544 x 6144 on 16 CUs: a 2-column x 3-m-tile rectangle, S = 2
    assert hq.hq_gemm_workspace_size("mxfp8", 520, 1544, 6144, cu_limit=16) == hdr + 2 * 520 * (1544 - 1280) * 4
    assert hq.hq_gemm_workspace_size("mxfp8", 4096, 4096, 256) == 0         # short K
    assert hq.hq_gemm_workspace_size("mxfp4", 16, 4096, 8192) == 0          # direct kernel
    assert hq.hq_gemm_workspace_size("mxfp8", 100, 128, 4096, batch=3) == hdr + min(cus // 3, 8) * 300 * 128 * 4
    assert hq.hq_gemm_workspace_size("mxfp8", 0, 128, 4096) == 0
    with pytest.raises(hq.HQError):
        hq.hq_gemm_workspace_size("mxfp8", 16, 12, 4096)                       # n % 8


def test_too_small_workspace_runs_unsplit():
    """A workspace smaller than the plan's is not used: the call runs unsplit
    and gives the unsplit call's bits."""
    dev = U.require_gpu()
    mode, m, n, k = "mxfp8", 300, 520, 8576
    rng = np.random.default_rng(77)
    a, sfa, _ = _quant(synth.normal_bf16(rng, (m, k)), mode)
    b, sfb, _ = _quant(synth.normal_bf16(rng, (n, k), 0.05), mode)
    need = hq.hq_gemm_workspace_size(mode, m, n, k)
    small = torch.empty(need - 16, dtype=torch.uint8, device=dev)
    outs = []
    for ws in (None, small):
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        hq.hq_dense_gemm(mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev), U.dev_u8(sfb, dev),
                         out, workspace=ws)
        outs.append(U.host_bits(out))
    assert np.array_equal(outs[0], outs[1])


def test_k_split_batch_with_bias():
    """Batch form: each batch's rows take its own weights and bias after the
    slices are summed."""
    dev = U.require_gpu()
    Bn, m, n, k = 3, 100, 128, 4096
    rng = np.random.default_rng(31)
    a, sfa = Q.mx_quant_bf16(synth.normal_bf16(rng, (Bn * m, k)), "mxfp8")
    b, sfb = Q.mx_quant_bf16(synth.normal_bf16(rng, (Bn * n, k), 0.05), "mxfp8")
    bias = synth.normal_bf16(rng, (Bn, n), 0.1)
    out = torch.empty(Bn, m, n, dtype=torch.bfloat16, device=dev)
    U.banner("k-split batch mxfp8")
    ws = hq.gemm_workspace("mxfp8", m, n, k, batch=Bn, device=dev)
    assert ws is not None
    hq.hq_batch_gemm("mxfp8", U.dev_u8(a, dev).view(Bn, m, k), U.dev_u8(sfa, dev).view(Bn, m, -1),
                     U.dev_u8(b, dev).view(Bn, n, k), U.dev_u8(sfb, dev).view(Bn, n, -1), out,
                     bias=U.dev_bf16(bias, dev), workspace=ws)
    torch.cuda.synchronize()
    want = G.batch_gemm("mxfp8", a.reshape(Bn, m, k), sfa.reshape(Bn, m, -1), b.reshape(Bn, n, k),
                        sfb.reshape(Bn, n, -1), bias=bias)
    got = U.host_bits(out)
    for i in range(Bn):
        U.assert_gemm_close(got[i], want[i], U.deq("mxfp8", a[i * m:(i + 1) * m], sfa[i * m:(i + 1) * m]),
                            U.deq("mxfp8", b[i * n:(i + 1) * n], sfb[i * n:(i + 1) * n]), what=f"batch {i}")


def test_k_split_batch_nvfp4_alpha():
    """Batch NVFP4 with a different alpha per item: the slice sum of each row is
    scaled by its own item's alpha."""
    dev = U.require_gpu()
    Bn, m, n, k = 2, 96, 256, 8192
    rng = np.random.default_rng(32)
    a, sfa, ga = _quant(synth.normal_bf16(rng, (Bn * m, k)), "nvfp4")
    b, sfb, gb = _quant(synth.normal_bf16(rng, (Bn * n, k), 0.05), "nvfp4")
    alpha = np.array([ga * gb, np.float32(3.0) * ga * gb], np.float32)
    out = torch.empty(Bn, m, n, dtype=torch.bfloat16, device=dev)
    U.banner("k-split batch nvfp4")
    ws = hq.gemm_workspace("nvfp4", m, n, k, batch=Bn, device=dev)
    assert ws is not None
    hq.hq_batch_gemm("nvfp4", U.dev_u8(a, dev).view(Bn, m, -1), U.dev_u8(sfa, dev).view(Bn, m, -1),
                     U.dev_u8(b, dev).view(Bn, n, -1), U.dev_u8(sfb, dev).view(Bn, n, -1), out,
                     alpha=torch.from_numpy(alpha).to(dev), workspace=ws)
    torch.cuda.synchronize()
    got = U.host_bits(out)
    for i in range(Bn):
        rows, cols = slice(i * m, (i + 1) * m), slice(i * n, (i + 1) * n)
        want = G.dense_gemm("nvfp4", a[rows], sfa[rows], b[cols], sfb[cols], alpha=alpha[i])
        U.assert_gemm_close(got[i], want, U.deq("nvfp4", a[rows], sfa[rows]), U.deq("nvfp4", b[cols], sfb[cols]),
                            alpha[i], f"batch {i}")


def test_config0_dense_mxfp8_256_with_gpu_quant():
    """256^3 MXFP8, seed 0: quantised on the GPU (bit-exact to the oracle),
    then the GEMM within tolerance."""
    dev = U.require_gpu()
    d = synth.dense_mxfp8_256()
    qa, sa, _ = hq.quantize(U.dev_bf16(d["a"], dev), "mxfp8")
    qb, sb, _ = hq.quantize(U.dev_bf16(d["b"], dev), "mxfp8")
    out = torch.empty(256, 256, dtype=torch.bfloat16, device=dev)
    hq.hq_dense_gemm("mxfp8", qa, sa, qb, sb, out)
    torch.cuda.synchronize()
    a, sfa = Q.mx_quant_bf16(d["a"], "mxfp8")
    b, sfb = Q.mx_quant_bf16(d["b"], "mxfp8")
    assert np.array_equal(U.host_u8(qa), a) and np.array_equal(U.host_u8(sb), sfb)
    want = G.dense_gemm("mxfp8", a, sfa, b, sfb)
    U.assert_gemm_close(U.host_bits(out), want, U.deq("mxfp8", a, sfa), U.deq("mxfp8", b, sfb))


@pytest.mark.parametrize("with_bias", [False, True])
def test_config1_batch_mxfp8(with_bias):
    dev = U.require_gpu()
    d = synth.batch_mxfp8()
    Bn, m, k = d["a"].shape
    n = d["b"].shape[1]
    a, sfa = Q.mx_quant_bf16(d["a"].reshape(Bn * m, k), "mxfp8")
    b, sfb = Q.mx_quant_bf16(d["b"].reshape(Bn * n, k), "mxfp8")
    bias = d["bias"] if with_bias else None
    out = torch.empty(Bn, m, n, dtype=torch.bfloat16, device=dev)
    U.banner(f"batch mxfp8 bias={with_bias}")
    hq.hq_batch_gemm("mxfp8", U.dev_u8(a, dev).view(Bn, m, k), U.dev_u8(sfa, dev).view(Bn, m, -1),
                     U.dev_u8(b, dev).view(Bn, n, k), U.dev_u8(sfb, dev).view(Bn, n, -1), out,
                     bias=None if bias is None else U.dev_bf16(bias, dev))
    torch.cuda.synchronize()
    want = G.batch_gemm("mxfp8", a.reshape(Bn, m, k), sfa.reshape(Bn, m, -1), b.reshape(Bn, n, k),
                        sfb.reshape(Bn, n, -1), bias=bias)
    got = U.host_bits(out)
    for i in range(Bn):
        U.assert_gemm_close(got[i], want[i], U.deq("mxfp8", a[i * m:(i + 1) * m], sfa[i * m:(i + 1) * m]),
                            U.deq("mxfp8", b[i * n:(i + 1) * n], sfb[i * n:(i + 1) * n]), what=f"batch {i}")


def test_config1_dense_mxfp4_32x512x256():
    dev = U.require_gpu()
    d = synth.dense_mxfp4_small()
    a, sfa = Q.mx_quant_bf16(d["a"], "mxfp4")
    b, sfb = Q.mx_quant_bf16(d["b"], "mxfp4")
    got = _dense_gpu("mxfp4", a, sfa, b, sfb, 32, 512, 256, dev)
    want = G.dense_gemm("mxfp4", a, sfa, b, sfb)
    U.assert_gemm_close(got, want, U.deq("mxfp4", a, sfa), U.deq("mxfp4", b, sfb))


def _grouped_inputs(mode, counts, K, N, seed, trailing=0):
    rng = np.random.default_rng(seed)
    E = len(counts)
    ends = np.cumsum(counts).astype(np.int32)
    R = int(ends[-1]) + trailing
    xa = synth.normal_bf16(rng, (R, K))
    xb = synth.normal_bf16(rng, (E * N, K), 0.05)
    a, sfa, ga = _quant(xa, mode)
    bq, bs, gb = _quant(xb, mode)
    b = bq.reshape(E, N, -1)
    sfb = bs.reshape(E, N, -1)
    return ends, a, sfa, b, sfb, ga, gb


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("case", ["ragged", "aligned"])
def test_group_contiguous(mode, case):
    dev = U.require_gpu()
    if case == "ragged":
        counts, K, N, trailing = [7, 0, 33, 1, 160, 0, 17], 96, 40, 9
    else:
        counts, K, N, trailing = [128, 256, 0, 384], 512, 256, 0
    U.banner(f"contiguous {mode} {case}")
    ends, a, sfa, b, sfb, ga, gb = _grouped_inputs(mode, counts, K, N, 42, trailing)
    E = len(counts)
    R = a.shape[0]
    alpha = None if ga is None else np.full(E, np.float32(ga * gb), np.float32)
    bias = synth.normal_bf16(np.random.default_rng(3), (E, N), 0.1) if mode == "mxfp8" else None
    out = torch.full((R, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    hq.hq_group_contiguous_gemm(mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev),
                                U.dev_u8(sfb, dev), U.dev_i32(ends, dev), out,
                                bias=None if bias is None else U.dev_bf16(bias, dev),
                                alpha=None if alpha is None else torch.from_numpy(alpha).to(dev))
    torch.cuda.synchronize()
    got = U.host_bits(out)
    want, written = G.group_contiguous_gemm(mode, a, sfa, b, sfb, ends, bias=bias, alpha=alpha,
                                            out=np.full((R, N), SENTINEL, np.uint16))
    assert np.all(got[~written] == SENTINEL), "rows outside every group were written"
    starts = np.concatenate([[0], ends[:-1]])
    for g in range(E):
        lo, hi = int(starts[g]), int(ends[g])
        if hi > lo:
            U.assert_gemm_close(got[lo:hi], want[lo:hi], U.deq(mode, a[lo:hi], sfa[lo:hi]),
                                U.deq(mode, b[g], sfb[g]), None if alpha is None else alpha[g], f"group {g}")


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
def test_group_contiguous_many_tiles_per_workgroup(mode):
    """A CU limit of 3 makes each workgroup walk about five tiles in turn, each
    of four K steps (K = 512, whole 16-byte scale groups), so every tile
    boundary carries the next tile's loads; partial last tiles leave waves
    without rows.  Integer-valued operands: exact against the exact sums."""
    dev = U.require_gpu()
    counts, K, N, trailing = [128, 300, 0, 77, 256, 1, 200], 512, 512, 5
    U.banner(f"contiguous {mode} many tiles per workgroup")
    rng = np.random.default_rng(2024)
    E = len(counts)
    ends = np.cumsum(counts).astype(np.int32)
    R = int(ends[-1]) + trailing
    av, a, sfa = _int_operand(rng, R, K, mode, [-1, 0, 1])
    bv, b, sfb = _int_operand(rng, E * N, K, mode, [-1, 0, 1])
    alpha = torch.ones(E, dtype=torch.float32, device=dev) if mode == "nvfp4" else None
    out = torch.full((R, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    hq.hq_group_contiguous_gemm(mode, U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b.reshape(E, N, -1), dev),
                                U.dev_u8(sfb.reshape(E, N, -1), dev), U.dev_i32(ends, dev), out, alpha=alpha,
                                cu_limit=3)
    torch.cuda.synchronize()
    got = U.host_bits(out)
    assert np.all(got[int(ends[-1]):] == SENTINEL), "rows after the last group were written"
    lo = 0
    for g in range(E):
        hi = int(ends[g])
        want = F.bf16_round((av[lo:hi] @ bv[g * N:(g + 1) * N].T).astype(np.float64))
        assert np.array_equal(got[lo:hi], want), f"group {g}: {np.sum(got[lo:hi] != want)} differ"
        lo = hi


# Slots of at most 256 rows (one m-tile each: the weights are read once and
# take the non-temporal load policy) and slots of 300 rows (two m-tiles each:
# the default policy).
MASKED_CASES = [(48, 256, 64, [48, 0, 13, 1, 30, 47]), (300, 512, 256, [300, 0, 257, 1, 130, 299])]


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("case", MASKED_CASES, ids=lambda c: f"slot{c[0]}")
def test_group_masked_matches_contiguous_with_garbage_padding(mode, case):
    dev = U.require_gpu()
    Mmax, K, N, cl = case
    counts = np.array(cl, np.int32)
    E = len(counts)
    rng = np.random.default_rng(9)
    U.banner(f"masked {mode} slots of {Mmax} rows")
    xa = synth.normal_bf16(rng, (int(counts.sum()), K))
    a_c, sfa_c, ga = _quant(xa, mode)
    xb = synth.normal_bf16(rng, (E * N, K), 0.05)
    bq, bs, gb = _quant(xb, mode)
    b, sfb = bq.reshape(E, N, -1), bs.reshape(E, N, -1)
    # padded layout: garbage codes and 0xFF (NaN) scales in every padded row
    a_m = synth.garbage_bytes(1, (E * Mmax, a_c.shape[1]))
    sfa_m = np.full((E * Mmax, sfa_c.shape[1]), 0xFF, np.uint8)
    ends = np.cumsum(counts)
    starts = ends - counts
    for e in range(E):
        a_m[e * Mmax:e * Mmax + counts[e]] = a_c[starts[e]:ends[e]]
        sfa_m[e * Mmax:e * Mmax + counts[e]] = sfa_c[starts[e]:ends[e]]
    alpha = None if ga is None else torch.full((E,), float(np.float32(ga * gb)), dtype=torch.float32, device=dev)
    out_m = torch.full((E * Mmax, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    hq.hq_group_masked_gemm(mode, U.dev_u8(a_m, dev), U.dev_u8(sfa_m, dev), U.dev_u8(b, dev), U.dev_u8(sfb, dev),
                            U.dev_i32(counts, dev), out_m, Mmax, alpha=alpha)
    out_c = torch.full((len(xa), N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    hq.hq_group_contiguous_gemm(mode, U.dev_u8(a_c, dev), U.dev_u8(sfa_c, dev), U.dev_u8(b, dev),
                                U.dev_u8(sfb, dev), U.dev_i32(ends, dev), out_c, alpha=alpha)
    torch.cuda.synchronize()
    gm, gc = U.host_bits(out_m), U.host_bits(out_c)
    al = None if alpha is None else np.full(E, np.float32(ga * gb), np.float32)
    for e in range(E):
        blk = gm[e * Mmax:(e + 1) * Mmax]
        assert np.all(blk[counts[e]:] == SENTINEL), f"expert {e}: padded rows written"
        assert np.array_equal(blk[:counts[e]], gc[starts[e]:ends[e]]), f"expert {e}: masked != contiguous"
        if counts[e]:
            want = G.dense_gemm(mode, a_c[starts[e]:ends[e]], sfa_c[starts[e]:ends[e]], b[e], sfb[e],
                                alpha=None if al is None else al[e])
            U.assert_gemm_close(blk[:counts[e]], want, U.deq(mode, a_c[starts[e]:ends[e]], sfa_c[starts[e]:ends[e]]),
                                U.deq(mode, b[e], sfb[e]), None if al is None else al[e], f"expert {e}")


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("form", ["contiguous", "masked"])
def test_many_groups(mode, form):
    """1024 groups (the limit): the group table fills every entry, tiles
    outnumber the CUs several times over, and groups end in full, more than
    half-full and at most half-full m-tiles (row counts around 128 and 256)."""
    dev = U.require_gpu()
    E, K, N = 1024, 256, 64
    rng = np.random.default_rng(77)
    if form == "contiguous":
        counts = rng.integers(0, 200, size=E).astype(np.int32)
        counts[rng.choice(E, 100, replace=False)] = 0
        counts[:8] = [128, 129, 256, 257, 300, 1, 127, 383]
    else:
        Mmax = 160
        counts = rng.integers(0, Mmax + 1, size=E).astype(np.int32)
        counts[rng.choice(E, 100, replace=False)] = 0
        counts[:6] = [128, 129, 160, 1, 127, 0]
    U.banner(f"{form} {mode} E={E} rows={int(counts.sum())}")
    ends = np.cumsum(counts).astype(np.int32)
    starts = ends - counts
    xa = synth.normal_bf16(rng, (int(ends[-1]), K))
    a_c, sfa_c, ga = _quant(xa, mode)
    xb = synth.normal_bf16(rng, (E * N, K), 0.05)
    bq, bs, gb = _quant(xb, mode)
    b, sfb = bq.reshape(E, N, -1), bs.reshape(E, N, -1)
    al = None if ga is None else np.full(E, np.float32(ga * gb), np.float32)
    alpha = None if al is None else torch.from_numpy(al).to(dev)
    if form == "contiguous":
        out = torch.full((len(xa), N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
        hq.hq_group_contiguous_gemm(mode, U.dev_u8(a_c, dev), U.dev_u8(sfa_c, dev), U.dev_u8(b, dev),
                                    U.dev_u8(sfb, dev), U.dev_i32(ends, dev), out, alpha=alpha)
        torch.cuda.synchronize()
        got = U.host_bits(out)
        rows = [(starts[e], ends[e]) for e in range(E)]
    else:
        a_m = synth.garbage_bytes(5, (E * Mmax, a_c.shape[1]))
        sfa_m = synth.garbage_bytes(6, (E * Mmax, sfa_c.shape[1]))
        for e in range(E):
            a_m[e * Mmax:e * Mmax + counts[e]] = a_c[starts[e]:ends[e]]
            sfa_m[e * Mmax:e * Mmax + counts[e]] = sfa_c[starts[e]:ends[e]]
        out = torch.full((E * Mmax, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
        hq.hq_group_masked_gemm(mode, U.dev_u8(a_m, dev), U.dev_u8(sfa_m, dev), U.dev_u8(b, dev),
                                U.dev_u8(sfb, dev), U.dev_i32(counts, dev), out, Mmax, alpha=alpha)
        torch.cuda.synchronize()
        gm = U.host_bits(out)
        pad = np.ones(E * Mmax, bool)
        for e in range(E):
            pad[e * Mmax:e * Mmax + counts[e]] = False
        assert np.all(gm[pad] == SENTINEL), "a padded row was written"
        got = np.zeros((len(xa), N), np.uint16)
        for e in range(E):
            got[starts[e]:ends[e]] = gm[e * Mmax:e * Mmax + counts[e]]
        rows = [(starts[e], ends[e]) for e in range(E)]
    for e, (lo, hi) in enumerate(rows):
        if hi > lo:
            want = G.dense_gemm(mode, a_c[lo:hi], sfa_c[lo:hi], b[e], sfb[e],
                                alpha=None if al is None else al[e])
            U.assert_gemm_close(got[lo:hi], want, U.deq(mode, a_c[lo:hi], sfa_c[lo:hi]), U.deq(mode, b[e], sfb[e]),
                                None if al is None else al[e], f"{form} group {e} ({hi - lo} rows)")


def test_device_counts_are_clamped():
    """Out-of-range device values: a masked count above max_m covers the slot
    exactly; a negative count covers nothing; decreasing ends give empty
    groups; ends beyond m_total stop at m_total."""
    dev = U.require_gpu()
    K, N, Mmax = 128, 32, 16
    rng = np.random.default_rng(2)
    xa = synth.normal_bf16(rng, (3 * Mmax, K))
    a, sfa = Q.mx_quant_bf16(xa, "mxfp8")
    xb = synth.normal_bf16(rng, (3 * N, K), 0.1)
    bq, bs = Q.mx_quant_bf16(xb, "mxfp8")
    b, sfb = bq.reshape(3, N, K), bs.reshape(3, N, -1)
    counts = np.array([1000, -5, 3], np.int32)
    out = torch.full((3 * Mmax, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    U.banner("clamp masked")
    hq.hq_group_masked_gemm("mxfp8", U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev), U.dev_u8(sfb, dev),
                            U.dev_i32(counts, dev), out, Mmax)
    torch.cuda.synchronize()
    want, written = G.group_masked_gemm("mxfp8", a, sfa, b, sfb, counts, Mmax,
                                        out=np.full((3 * Mmax, N), SENTINEL, np.uint16))
    got = U.host_bits(out)
    assert np.all(got[~written] == SENTINEL)
    for e, c in [(0, Mmax), (2, 3)]:
        lo, hi = e * Mmax, e * Mmax + c
        assert written[lo:hi].all()
        U.assert_gemm_close(got[lo:hi], want[lo:hi], U.deq("mxfp8", a[lo:hi], sfa[lo:hi]),
                            U.deq("mxfp8", b[e], sfb[e]), what=f"clamped expert {e}")
    ends = np.array([20, 10, 999], np.int32)
    out2 = torch.full((3 * Mmax, N), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    U.banner("clamp contiguous")
    hq.hq_group_contiguous_gemm("mxfp8", U.dev_u8(a, dev), U.dev_u8(sfa, dev), U.dev_u8(b, dev),
                                U.dev_u8(sfb, dev), U.dev_i32(ends, dev), out2)
    torch.cuda.synchronize()
    want2, written2 = G.group_contiguous_gemm("mxfp8", a, sfa, b, sfb, ends,
                                              out=np.full((3 * Mmax, N), SENTINEL, np.uint16))
    got2 = U.host_bits(out2)
    assert written2.all()
    for lo, hi, g in [(0, 20, 0), (20, 48, 2)]:
        U.assert_gemm_close(got2[lo:hi], want2[lo:hi], U.deq("mxfp8", a[lo:hi], sfa[lo:hi]),
                            U.deq("mxfp8", b[g], sfb[g]), what=f"clamped group {g}")
