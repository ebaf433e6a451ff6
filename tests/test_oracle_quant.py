"""Pins for oracle.quant.

* Brute force on 4 x 4 x 32 inputs (4 rows, 4 groups of 32) reproduces the
  OCP MX rule -- scale = floor(log2 amax) - emax_elem, clamped to the UE8M0
  range; codes = nearest element value of x / 2^scale, ties to even,
  saturating -- computed with exact rationals and a scan for floor(log2).
* NVFP4: every step re-derived with exact rationals and explicit FP32
  rounding (a different route from numpy's float32 arithmetic).
* Properties: idempotence, sign symmetry, power-of-two equivariance, zero
  blocks, saturation.
"""
import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q
from synth import to_bf16_bits
from tests import _exact as X


def _random_bf16_blocks(rng, rows, K):
    """BF16 bit patterns with a spread of magnitudes per 32-group, exact grid
    ties, zeros, negative zeros and subnormals."""
    bits = np.zeros((rows, K), np.uint16)
    for r in range(rows):
        for g in range(K // 32):
            kind = rng.integers(0, 6)
            center = rng.integers(-20, 20)
            if kind == 0:       # plain normals
                v = rng.standard_normal(32).astype(np.float32) * np.float32(2.0 ** center)
                blk = to_bf16_bits(v)
            elif kind == 1:     # all zeros (some negative)
                blk = np.where(rng.random(32) < 0.5, 0x8000, 0).astype(np.uint16)
            elif kind == 2:     # BF16 subnormals and tiny normals
                blk = rng.integers(0, 0x0100, 32).astype(np.uint16) | (rng.integers(0, 2, 32) << 15).astype(np.uint16)
            elif kind == 3:     # exact E2M1/E4M3 midpoints relative to a block max
                base = np.float32(2.0 ** center)
                mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.5, 1.0 / 128, 3.0 / 256], np.float32)
                v = rng.choice(mids, 32) * base * rng.choice(np.array([-1, 1], np.float32), 32)
                v[0] = np.float32(7.9) * base
                blk = to_bf16_bits(v)
            elif kind == 4:     # one huge outlier, the rest tiny (many codes round to 0)
                v = rng.standard_normal(32).astype(np.float32) * np.float32(2.0 ** (center - 14))
                v[rng.integers(0, 32)] = np.float32(2.0 ** center) * 1.9
                blk = to_bf16_bits(v)
            else:               # values near the top of a binade (saturation path)
                v = np.float32(2.0 ** center) * rng.uniform(1.7, 1.999, 32).astype(np.float32)
                v *= rng.choice(np.array([-1, 1], np.float32), 32)
                blk = to_bf16_bits(v)
            bits[r, g * 32:(g + 1) * 32] = blk
    return bits


def _mx_brute(bits, fmt):
    grid = X.E4M3 if fmt == "mxfp8" else X.E2M1
    emax = 8 if fmt == "mxfp8" else 2
    sign_bit = 0x80 if fmt == "mxfp8" else 0x8
    rows, K = bits.shape
    codes = np.zeros((rows, K), np.uint8)
    sf = np.zeros((rows, K // 32), np.uint8)
    for r in range(rows):
        for g in range(K // 32):
            vals = [X.bf16_value(int(b)) for b in bits[r, g * 32:(g + 1) * 32]]
            amax = max(abs(v) for v, _ in vals)
            s = -127 if amax == 0 else min(max(X.floor_log2(amax) - emax, -127), 127)
            sf[r, g] = s + 127
            for j, (v, neg) in enumerate(vals):
                c = X.nearest_code(v / X.Fr(2) ** s, grid)
                codes[r, g * 32 + j] = c | (sign_bit if neg else 0)
    return codes, sf


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("seed", range(6))
def test_mx_rule_brute_force_4x4x32(fmt, seed):
    rng = np.random.default_rng(1000 + seed)
    bits = _random_bf16_blocks(rng, 4, 128)
    want_codes, want_sf = _mx_brute(bits, fmt)
    codes, sf = Q.mx_quant_bf16(bits, fmt)
    assert np.array_equal(sf, want_sf)
    if fmt == "mxfp4":
        want_codes = F.pack_nibbles(want_codes)
    assert np.array_equal(codes, want_codes)


def test_mx_zero_block_and_extremes():
    bits = np.zeros((1, 64), np.uint16)
    bits[0, 32:] = 0x8000                       # -0
    codes, sf = Q.mx_quant_bf16(bits, "mxfp8")
    assert sf.tolist() == [[0, 0]]
    assert codes[0, :32].tolist() == [0] * 32 and codes[0, 32:].tolist() == [0x80] * 32
    # largest finite BF16: floor(log2) = 127 -> scale 119 (MXFP8), 125 (MXFP4)
    big = np.full((1, 32), 0x7F7F, np.uint16)
    assert Q.mx_quant_bf16(big, "mxfp8")[1][0, 0] == 127 + 119
    assert Q.mx_quant_bf16(big, "mxfp4")[1][0, 0] == 127 + 125
    # smallest BF16 subnormal: floor(log2) = -133 -> clamped to -127
    tiny = np.full((1, 32), 0x0001, np.uint16)
    c, s = Q.mx_quant_bf16(tiny, "mxfp8")
    # 2^-133 / 2^-127 = 2^-6, the smallest E4M3 normal (code 0x08)
    assert s[0, 0] == 0 and np.all(c == 0x08)
    c4, s4 = Q.mx_quant_bf16(tiny, "mxfp4")
    # 2^-6 is below half of E2M1's smallest step (0.25) -> code 0
    assert s4[0, 0] == 0 and not c4.any()


def test_mx_saturation_top_of_binade():
    # 1.99 * 2^e scales to 1.99 * 2^8 = 509.4 -> saturates to 448 (0x7E)
    v = np.float32(1.99) * np.ones((1, 32), np.float32)
    bits = to_bf16_bits(v)
    codes, sf = Q.mx_quant_bf16(bits, "mxfp8")
    assert sf[0, 0] == 127 - 8 and np.all(codes == 0x7E)
    codes4, sf4 = Q.mx_quant_bf16(bits, "mxfp4")
    assert sf4[0, 0] == 127 - 2 and np.all(codes4 == 0x77)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_properties(fmt):
    rng = np.random.default_rng(7)
    bits = to_bf16_bits(rng.standard_normal((16, 256)).astype(np.float32))
    codes, sf = Q.mx_quant_bf16(bits, fmt)
    deq = Q.dequant(codes, sf, fmt)
    codes2, sf2 = Q.mx_quant_values(deq, fmt)
    assert np.array_equal(codes, codes2) and np.array_equal(sf, sf2)          # idempotent
    neg = bits ^ np.uint16(0x8000)
    ncodes, nsf = Q.mx_quant_bf16(neg, fmt)
    flip = 0x80 if fmt == "mxfp8" else 0x88
    assert np.array_equal(nsf, sf) and np.array_equal(ncodes, codes ^ np.uint8(flip))
    x = F.bf16_decode(bits)
    for j in (-5, 3, 20):
        c3, s3 = Q.mx_quant_values(np.ldexp(x, j), fmt)
        assert np.array_equal(c3, codes) and np.array_equal(s3.astype(int), sf.astype(int) + j)
    # error bound: half the top-binade step, or the saturation gap
    # (E4M3: [448, 512) -> 448, gap 64; E2M1: [6, 8) -> 6, gap 2), times 2^scale
    err = np.abs(deq - x)
    scale = F.ue8m0_decode(np.repeat(sf, 32, axis=1))
    assert np.all(err <= scale * (64.0 if fmt == "mxfp8" else 2.0))


def _nv_brute(bits, g):
    rows, K = bits.shape
    codes = np.zeros((rows, K), np.uint8)
    sf = np.zeros((rows, K // 16), np.uint8)
    g = X.Fr(float(g))
    d = X.fp32_round(6 * g)
    for r in range(rows):
        for b in range(K // 16):
            vals = [X.bf16_value(int(t)) for t in bits[r, b * 16:(b + 1) * 16]]
            amax = max(abs(v) for v, _ in vals)
            ratio = X.fp32_round(amax / d)
            s = X.nearest_code(ratio, X.E4M3)
            sf[r, b] = s
            s_eff = X.fp32_round(dict(X.E4M3)[s] * g)
            for j, (v, neg) in enumerate(vals):
                c = 0 if s_eff == 0 else X.nearest_code(X.fp32_round(v / s_eff), X.E2M1)
                codes[r, b * 16 + j] = c | (0x8 if neg else 0)
    return F.pack_nibbles(codes), sf


@pytest.mark.parametrize("seed", range(4))
def test_nvfp4_recipe_brute_force(seed):
    rng = np.random.default_rng(2000 + seed)
    bits = _random_bf16_blocks(rng, 4, 64)
    bits[bits & 0x7F80 == 0] = 0                # keep BF16 normals and zeros
    codes, sf, g = Q.nvfp4_quant_bf16(bits)
    x = F.bf16_decode(bits)
    amax = np.max(np.abs(x))
    want_g = np.float32(1.0) if amax == 0 else np.float32(float(X.fp32_round(X.Fr(float(amax)) / 2688)))
    assert g == want_g
    wc, ws = _nv_brute(bits, g)
    assert np.array_equal(sf, ws)
    assert np.array_equal(codes, wc)


def test_nvfp4_global_scale_supplied_and_zero():
    bits = np.zeros((2, 32), np.uint16)
    codes, sf, g = Q.nvfp4_quant_bf16(bits)
    assert g == 1.0 and not sf.any() and not codes.any()
    one = to_bf16_bits(np.ones((1, 16), np.float32))
    codes, sf, g = Q.nvfp4_quant_bf16(one, g=np.float32(1.0 / 6.0))
    # amax/d = 1 / fp32(6 * fp32(1/6)) -> 1.0 -> UE4M3 0x38; x / s_eff = 6 -> code 7
    assert sf[0, 0] == 0x38 or sf[0, 0] in (0x37, 0x39)
    assert np.all(F.unpack_nibbles(codes) == 7)
