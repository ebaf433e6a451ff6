"""Element and scale formats, decoded from their bit definitions (oracle; test
infrastructure only).

The pages name the formats but do not print their grids:
  * HALOps "GEMM" page, group_wise_quant section: FP8 codes are
    float8_e4m3fn, FP4 codes are packed E2M1 nibbles (even index in the low
    nibble), MX scales are UE8M0 ("power-of-2 biased exponent"), NVFP4
    scales are UE4M3 (the e4m3fn bit pattern read as an unsigned byte).
  * cuDNN FE "Grouped GEMM + dGLU (SM100)", Data Types table: MXFP8 uses
    e8m0 scales per 32; NVF4 uses e4m3 scales per 16.
The bit-level meanings below follow the OCP MX v1.0 element definitions:

  E4M3 (fn): sign | 4-bit exponent (bias 7) | 3-bit mantissa.  Exponent 0 is
             subnormal (m/8 * 2^-6).  S.1111.111 is NaN; there is no Inf.
             Largest finite magnitude 448.
  E2M1:      sign | 2-bit exponent (bias 1) | 1-bit mantissa.  Exponent 0 is
             subnormal (m/2).  Magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
  UE8M0:     byte b means 2^(b-127); 0xFF is NaN.
  UE4M3:     E4M3 with the sign bit clear.
  BF16:      sign | 8-bit exponent (bias 127) | 7-bit mantissa (IEEE-style,
             with subnormals, Inf and NaN).

Encoders round to nearest with ties to the even code (the code whose
mantissa LSB -- bit 0 of the code -- is 0) and saturate to the largest
finite magnitude.  The sign of the input is kept, also when the magnitude
rounds to zero (-tiny -> the negative-zero code).
"""

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def _e4m3_value(code):
    """Value of one E4M3 code from its fields (Python floats, exact)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def _e2m1_value(code):
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = m * 0.5
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)

# Positive finite grids, indexed by code (codes are monotone in magnitude).
_E4M3_POS = E4M3_TABLE[:127].copy()        # codes 0x00 .. 0x7E
_E2M1_POS = E2M1_TABLE[:8].copy()          # codes 0x0 .. 0x7


def e4m3_decode(codes):
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_decode(codes):
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def ue8m0_decode(b):
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


def ue4m3_decode(b):
    b = np.asarray(b, dtype=np.uint8)
    return E4M3_TABLE[b & 0x7F]


def _encode_grid(v, grid):
    """Nearest grid index for |v| (grid sorted, starts at 0), ties to the even
    index, saturating at the top of the grid."""
    a = np.minimum(np.abs(np.asarray(v, dtype=np.float64)), grid[-1])
    hi = np.searchsorted(grid, a, side="left")          # grid[hi] >= a
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    return idx.astype(np.uint8)


def e4m3_encode(v):
    """float64 -> E4M3 code: round to nearest, ties to even, saturate +-448."""
    v = np.asarray(v, dtype=np.float64)
    idx = _encode_grid(v, _E4M3_POS)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (idx | sign).astype(np.uint8)


def e2m1_encode(v):
    """float64 -> E2M1 code (0..15): round to nearest, ties to even, saturate +-6."""
    v = np.asarray(v, dtype=np.float64)
    idx = _encode_grid(v, _E2M1_POS)
    sign = np.signbit(v).astype(np.uint8) << 3
    return (idx | sign).astype(np.uint8)


def ue4m3_encode(v):
    """non-negative float64 -> UE4M3 byte (round to nearest even, saturate 448)."""
    v = np.asarray(v, dtype=np.float64)
    return _encode_grid(v, _E4M3_POS)


def pack_nibbles(codes):
    """[..., 2j] -> low nibble, [..., 2j+1] -> high nibble of byte j."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def bf16_decode(bits):
    """BF16 bit patterns (uint16) -> float64.  A BF16 pattern is the upper half
    of the FP32 pattern with the same value."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def fp16_decode(bits):
    """IEEE binary16 bit patterns (uint16) -> float64, from the fields: sign
    bit 15, exponent bits 10-14 (bias 15), fraction bits 0-9; exponent 0 is
    +-fraction * 2^-24 (zero and subnormals), exponent 31 is Inf (fraction 0)
    or NaN.  (Input dtype of the HALOps "GEMM" page's group_wise_quant.)"""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = sign * (1.0 + f / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = sign * f * 2.0 ** -24
    special = np.where(f == 0, sign * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 31, special, normal))


FP16_MAX = 65504.0


def fp16_round(x):
    """float64 -> IEEE binary16 bits, one rounding (nearest, ties to even):
    11 significant bits for exponents >= -14, a fixed quantum of 2^-24 below
    (subnormals); magnitudes that round above 65504 become Inf; NaN stays NaN
    (the GEMM output dtype of the flashrt/fp4-gemm page's *_fp16 GEMMs)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e = np.frexp(x)
        q = np.maximum(e.astype(np.int64) - 11, -24)
        r = np.ldexp(np.rint(np.ldexp(x, -q)), q)   # np.rint: ties to even
        r = np.where(np.abs(r) > FP16_MAX, np.copysign(np.inf, x), r)
        r = np.where(np.isnan(x), np.nan, r)
        r16 = r.astype(np.float16)                  # exact: r is a binary16 value
    return r16.view(np.uint16)


def bf16_round(x):
    """float64 -> BF16 bits, one rounding (nearest, ties to even).

    BF16 keeps 8 significant bits for exponents >= -126 and a fixed quantum
    of 2^-133 below that (subnormals).  Magnitudes that round above the
    largest finite BF16 become Inf.  NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e = np.frexp(x)                          # |x| = f * 2^e, f in [.5,1)
        q = np.maximum(e.astype(np.int64) - 8, -133)
        r = np.ldexp(np.rint(np.ldexp(x, -q)), q)   # np.rint: ties to even
        r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
        r = np.where(np.isnan(x), np.nan, r)
        r32 = r.astype(np.float32)                  # exact: r is a BF16 value
    return (r32.view(np.uint32) >> 16).astype(np.uint16)
