"""Group-wise quantisation (oracle; test infrastructure only).

MX recipe (MXFP8 = E4M3 codes, MXFP4 = E2M1 codes, one UE8M0 scale per 32
consecutive K elements of a row): HALOps "GEMM" page, group_wise_quant
section (modes w8a8-mxfp8 / w4a4-mxfp4, scale encodings, nibble order), with
the scale rule of the OCP MX specification: the shared exponent is
floor(log2(amax)) minus the largest exponent of the element format
(8 for E4M3, 2 for E2M1), clamped to the UE8M0 range; elements are divided by
2^scale and rounded to the element grid with saturation.

NVFP4 recipe (E2M1 codes, one UE4M3 scale per 16, an FP32 per-tensor global
scale): HALOps "GEMM" page, group_wise_quant section (UE4M3 per 16) and the
alpha parameter of the GEMM sections (required for w4a4-nvfp4);
flashrt/fp4-gemm page (NVFP4 A4W4 producers).  The pages give only the
global-scale formula alpha = amax / (448 * 6) per operand; the remaining
steps are the plainest two-level reading of it:
    g      = fp32(amax_tensor / 2688)         (g = 1 when amax_tensor == 0)
    d      = fp32(6 * g)
    sf_b   = UE4M3_rne_sat(fp32(amax_block / d))
    s_eff  = fp32(decode(sf_b) * g)
    code   = E2M1_rne_sat(fp32(x / s_eff))     (code = +-0 when s_eff == 0)
Each fp32(...) is one IEEE single-precision operation rounded to nearest
even.  NVFP4 parity against other implementations is unpinned: the pages
print no values.
"""

import numpy as np

from . import formats as F

MX_GROUP = 32
NV_GROUP = 16
E4M3_EMAX = 8   # 448 = 1.75 * 2^8
E2M1_EMAX = 2   # 6   = 1.5  * 2^2


def _floor_log2(a):
    """floor(log2(a)) for a > 0, exact (frexp: a = f * 2^e, f in [0.5, 1))."""
    _, e = np.frexp(a)
    return e.astype(np.int64) - 1


def mx_quant_values(x, fmt):
    """MX quantisation of real values x[..., K] (float64 holding exactly the
    BF16 or FP32 inputs).  fmt is "mxfp8" or "mxfp4".

    Returns (codes, sf): codes is uint8 [..., K] for mxfp8 and packed uint8
    [..., K/2] for mxfp4 (element 2j in the low nibble of byte j); sf is the
    UE8M0 byte per 32-group, shape [..., K/32], row-major."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    assert K % MX_GROUP == 0
    g = x.reshape(x.shape[:-1] + (K // MX_GROUP, MX_GROUP))
    amax = np.max(np.abs(g), axis=-1)
    emax = E4M3_EMAX if fmt == "mxfp8" else E2M1_EMAX
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)), -(1 << 20))
    s = np.clip(e - emax, -127, 127)
    sf = (s + 127).astype(np.uint8)
    v = np.ldexp(g, -s[..., None])                  # exact power-of-two scaling
    if fmt == "mxfp8":
        codes = F.e4m3_encode(v).reshape(x.shape)
        return codes, sf
    if fmt == "mxfp4":
        codes = F.e2m1_encode(v).reshape(x.shape)
        return F.pack_nibbles(codes), sf
    raise ValueError(fmt)


def mx_quant_bf16(x_bits, fmt):
    """MX quantisation of BF16 rows given as uint16 bit patterns."""
    return mx_quant_values(F.bf16_decode(x_bits), fmt)


def mx_quant_fp16(x_bits, fmt):
    """MX quantisation of FP16 rows given as uint16 bit patterns."""
    return mx_quant_values(F.fp16_decode(x_bits), fmt)


def nvfp4_global_scale(amax_tensor):
    """g = fp32(amax / 2688), or 1 when amax == 0 (FP32 arithmetic)."""
    a = np.float32(amax_tensor)
    if a == 0:
        return np.float32(1.0)
    return np.float32(a / np.float32(2688.0))


def nvfp4_quant_values(x, g=None):
    """NVFP4 quantisation of real values x[..., K] (exact FP32/BF16 values as
    float64).  If g (FP32 global scale) is None it is computed from the
    tensor's amax.  Returns (packed codes [..., K/2], sf [..., K/16] UE4M3
    bytes, g as np.float32)."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    assert K % NV_GROUP == 0
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x, equal_nan=True), "inputs must be FP32-exact"
    if g is None:
        g = nvfp4_global_scale(np.max(np.abs(x32)) if x32.size else np.float32(0))
    g = np.float32(g)
    d = np.float32(np.float32(6.0) * g)
    blk = x32.reshape(x32.shape[:-1] + (K // NV_GROUP, NV_GROUP))
    amax_b = np.max(np.abs(blk), axis=-1).astype(np.float32)
    # A quotient may overflow FP32 (a tiny supplied g): it becomes +-Inf and
    # the encoders saturate it, as the device does; the warning is silenced.
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        ratio = (amax_b / d).astype(np.float32)                # one fp32 division
    sf = F.ue4m3_encode(ratio.astype(np.float64))
    with np.errstate(over="ignore"):
        s_eff = (F.ue4m3_decode(sf).astype(np.float32) * g).astype(np.float32)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        q = (blk / s_eff[..., None]).astype(np.float32)        # one fp32 division
    q = np.where(s_eff[..., None] == 0, np.copysign(np.float32(0), blk), q)
    codes = F.e2m1_encode(q.astype(np.float64)).reshape(x.shape)
    return F.pack_nibbles(codes), sf, g


def nvfp4_quant_bf16(x_bits, g=None):
    return nvfp4_quant_values(F.bf16_decode(x_bits), g)


def nvfp4_quant_fp16(x_bits, g=None):
    return nvfp4_quant_values(F.fp16_decode(x_bits), g)


def dequant(codes, sf, fmt, g=None):
    """Real values of quantised rows: decode(code) * scale(group) [* g].

    fmt: "mxfp8" (codes [..,K]), "mxfp4" (packed [..,K/2]) or "nvfp4"
    (packed [..,K/2], UE4M3 sf per 16; g multiplies every element when given,
    otherwise the per-tensor factor is left to the GEMM's alpha)."""
    codes = np.asarray(codes, dtype=np.uint8)
    sf = np.asarray(sf, dtype=np.uint8)
    if fmt == "mxfp8":
        v = F.e4m3_decode(codes)
        gs = MX_GROUP
        scale = F.ue8m0_decode(sf)
    elif fmt == "mxfp4":
        v = F.e2m1_decode(F.unpack_nibbles(codes))
        gs = MX_GROUP
        scale = F.ue8m0_decode(sf)
    elif fmt == "nvfp4":
        v = F.e2m1_decode(F.unpack_nibbles(codes))
        gs = NV_GROUP
        scale = F.ue4m3_decode(sf)
    else:
        raise ValueError(fmt)
    K = v.shape[-1]
    vg = v.reshape(v.shape[:-1] + (K // gs, gs)) * scale[..., None]
    out = vg.reshape(v.shape)
    if g is not None:
        out = out * np.float64(np.float32(g))
    return out
