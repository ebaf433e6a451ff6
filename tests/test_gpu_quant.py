"""GPU parity of hq_group_wise_quant against the oracle: codes, scale bytes
and the NVFP4 global scale must be bit-exact."""
import numpy as np
import pytest
import torch

import fp4_gemm_moe_amd as hq
import synth
from oracle import quant as Q
from tests import _gpu as U
from tests.test_oracle_quant import _random_bf16_blocks

pytestmark = pytest.mark.gpu

MODES = ["mxfp8", "mxfp4", "nvfp4"]


def _run(mode, bits, dev, g=None):
    x = U.dev_bf16(bits, dev)
    gs = None
    if mode == "nvfp4" and g is not None:
        gs = torch.tensor([g], dtype=torch.float32, device=dev)
    q, sf, gout = hq.quantize(x, mode, gs)
    torch.cuda.synchronize()
    return U.host_u8(q), U.host_u8(sf), (None if gout is None else float(gout.cpu()[0]))


def _oracle(mode, bits, g=None):
    if mode == "nvfp4":
        c, s, gg = Q.nvfp4_quant_bf16(bits, None if g is None else np.float32(g))
        return c, s, float(gg)
    c, s = Q.mx_quant_bf16(bits, mode)
    return c, s, None


def _check(mode, bits, dev, g=None, what=""):
    U.banner(f"quant {mode} {bits.shape} {what}")
    qc, qs, qg = _run(mode, bits, dev, g)
    oc, os_, og = _oracle(mode, bits, g)
    assert np.array_equal(qs, os_), f"{mode} {what}: {np.sum(qs != os_)} scale bytes differ"
    assert np.array_equal(qc, oc), f"{mode} {what}: {np.sum(qc != oc)} code bytes differ"
    if mode == "nvfp4":
        assert np.float32(qg) == np.float32(og), (qg, og)


@pytest.mark.parametrize("mode", MODES)
def test_quant_dense_256(mode):
    dev = U.require_gpu()
    d = synth.dense_mxfp8_256()
    _check(mode, d["a"], dev, what="256x256 N(0,1)")
    _check(mode, d["b"], dev, what="256x256 N(0,1) B")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(1, 32), (37, 96), (129, 544), (1024, 256)])
def test_quant_ragged_shapes(mode, shape):
    dev = U.require_gpu()
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    bits = synth.normal_bf16(rng, shape, 3.0)
    _check(mode, bits, dev, what="ragged")


@pytest.mark.parametrize("mode", MODES)
def test_quant_adversarial_blocks(mode):
    """Zeros, negative zeros, BF16 subnormals, exact grid midpoints, outliers,
    values at the top of a binade."""
    dev = U.require_gpu()
    rng = np.random.default_rng(77)
    bits = _random_bf16_blocks(rng, 64, 512)
    if mode == "nvfp4":
        bits[(bits & 0x7F80) == 0] = 0   # NVFP4 recipe is defined on normal BF16 inputs
    _check(mode, bits, dev, what="adversarial")


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4"])
def test_quant_every_bf16_value(mode):
    """Every finite BF16 pattern, shuffled into 32-groups, so every element
    value meets many different group scales."""
    dev = U.require_gpu()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = (bits & 0x7F80) != 0x7F80
    vals = bits[fin]
    rng = np.random.default_rng(5)
    out = np.concatenate([rng.permutation(vals) for _ in range(3)])
    out = out[: (len(out) // 32) * 32].reshape(-1, 32 * 8)[: 4096]
    _check(mode, np.ascontiguousarray(out), dev, what="all finite BF16")


@pytest.mark.parametrize("g", [2.0 ** -100, 2.0 ** -40, 0.0012345, 1.0, 2.0 ** 40, 2.0 ** 100])
def test_quant_nvfp4_every_bf16_value(g):
    """Every normal BF16 pattern of either sign, sorted by magnitude into
    16-groups (so each group's scale is set by values of one size, and every
    value meets an unsaturated scale at some global scale), groups and group
    members shuffled.  The global scales put the effective block scales both
    inside [2^-56, 2^56], where the device divides with a shared reciprocal,
    and outside it, where it divides plainly."""
    dev = U.require_gpu()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ex = bits & 0x7F80
    vals = bits[(ex != 0x7F80) & (ex != 0)]
    vals = vals[np.argsort(vals & 0x7FFF, kind="stable")]
    vals = vals[: (len(vals) // 16) * 16].reshape(-1, 16)
    rng = np.random.default_rng(int(np.log2(g)) + 200)
    vals = rng.permuted(vals, axis=1)[rng.permutation(len(vals))]
    out = np.ascontiguousarray(vals.reshape(-1, 256)[: (vals.size // 256)])
    _check("nvfp4", out, dev, g=g, what=f"all normal BF16, g={g:g}")


def _check_fp16(mode, bits, dev, g=None, what=""):
    """FP16 input (HQ_IN_FP16): the device codes / scales / global scale
    against the oracle's quantisation of the decoded FP16 values."""
    U.banner(f"quant fp16 {mode} {bits.shape} {what}")
    x = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(dev)
    gs = None if g is None else torch.tensor([g], dtype=torch.float32, device=dev)
    q, sf, gout = hq.quantize(x, mode, gs)
    torch.cuda.synchronize()
    if mode == "nvfp4":
        oc, os_, og = Q.nvfp4_quant_fp16(bits, None if g is None else np.float32(g))
        assert np.float32(float(gout.cpu()[0])) == np.float32(og), (float(gout.cpu()[0]), og)
    else:
        oc, os_ = Q.mx_quant_fp16(bits, mode)
    assert np.array_equal(U.host_u8(sf), os_), f"{mode} {what}: {np.sum(U.host_u8(sf) != os_)} scale bytes differ"
    assert np.array_equal(U.host_u8(q), oc), f"{mode} {what}: {np.sum(U.host_u8(q) != oc)} code bytes differ"


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4"])
def test_quant_every_fp16_value(mode):
    """FP16 input: every finite binary16 pattern (subnormals and +-65504
    included), shuffled into 32-groups."""
    dev = U.require_gpu()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits[(bits & 0x7C00) != 0x7C00]
    rng = np.random.default_rng(15)
    out = np.concatenate([rng.permutation(vals) for _ in range(3)])
    out = out[: (len(out) // 256) * 256].reshape(-1, 256)
    _check_fp16(mode, np.ascontiguousarray(out), dev, what="all finite FP16")


@pytest.mark.parametrize("g", [None, 2.0 ** -20, 0.0012345, 2.0 ** 20])
def test_quant_nvfp4_every_fp16_value(g):
    """FP16 input, NVFP4: every normal binary16 pattern of either sign,
    sorted by magnitude into 16-groups and shuffled (as for BF16); the global
    scale computed from the tensor's amax (None) or supplied."""
    dev = U.require_gpu()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ex = bits & 0x7C00
    vals = bits[(ex != 0x7C00) & (ex != 0)]
    vals = vals[np.argsort(vals & 0x7FFF, kind="stable")]
    vals = vals[: (len(vals) // 16) * 16].reshape(-1, 16)
    rng = np.random.default_rng(300 if g is None else int(np.log2(g)) + 400)
    vals = rng.permuted(vals, axis=1)[rng.permutation(len(vals))]
    out = np.ascontiguousarray(vals.reshape(-1, 256)[: (vals.size // 256)])
    _check_fp16("nvfp4", out, dev, g=g, what=f"all normal FP16, g={g}")


def test_quant_fp16_gaussian_rows():
    """FP16 input, N(0, 1) rows of the MoE width in the three modes."""
    dev = U.require_gpu()
    x = torch.randn(96, 4096, generator=torch.Generator().manual_seed(12)).to(torch.float16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    for mode in MODES:
        _check_fp16(mode, bits, dev, what="gaussian")


def test_quant_nvfp4_supplied_global_scale():
    dev = U.require_gpu()
    rng = np.random.default_rng(3)
    bits = synth.normal_bf16(rng, (64, 256), 1.0)
    _check("nvfp4", bits, dev, g=0.0012345, what="supplied g")
    zeros = np.zeros((4, 64), np.uint16)
    _check("nvfp4", zeros, dev, what="all zero -> g = 1")


def test_quant_large_activation_every_byte():
    """MoE activation quantisation at full size [65536, 4096] (MXFP8): every
    code and every scale byte against the oracle (the oracle runs on chunks
    of 4096 rows, several at a time)."""
    from concurrent.futures import ThreadPoolExecutor
    dev = U.require_gpu()
    m, k = 65536, 4096
    U.banner("quant mxfp8 65536x4096 (every byte)")
    x = torch.randn(m, k, generator=torch.Generator(device=dev).manual_seed(31), device=dev).to(torch.bfloat16)
    q, sf, _ = hq.quantize(x, "mxfp8")
    xb, qh, sh = U.host_bits(x), U.host_u8(q), U.host_u8(sf)
    del x, q, sf
    step = 4096

    def chunk(r0):
        oc, os_ = Q.mx_quant_bf16(xb[r0:r0 + step], "mxfp8")
        return (np.array_equal(qh[r0:r0 + step], oc), np.array_equal(sh[r0:r0 + step], os_))

    with ThreadPoolExecutor(max_workers=8) as ex:
        res = list(ex.map(chunk, range(0, m, step)))
    bad_codes = [i * step for i, (c, _) in enumerate(res) if not c]
    bad_scales = [i * step for i, (_, s_) in enumerate(res) if not s_]
    assert not bad_scales, f"scale bytes differ in the row chunks starting at {bad_scales}"
    assert not bad_codes, f"codes differ in the row chunks starting at {bad_codes}"


def test_quant_fp16_input_must_be_contiguous():
    """A float16 x goes through the same contiguity and device checks as a
    bfloat16 one: a transposed or broadcast view is refused before any call."""
    dev = U.require_gpu()
    x = torch.randn(64, 128, device=dev).to(torch.float16)
    q = torch.empty(128, 64, dtype=torch.uint8, device=dev)
    sf = torch.empty(128, 2, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="contiguous"):
        hq.hq_group_wise_quant("mxfp8", x.t(), q, sf)
    row = torch.randn(1, 128, device=dev).to(torch.float16)
    q2 = torch.empty(64, 128, dtype=torch.uint8, device=dev)
    sf2 = torch.empty(64, 4, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="contiguous"):
        hq.hq_group_wise_quant("mxfp8", row.expand(64, 128), q2, sf2)
