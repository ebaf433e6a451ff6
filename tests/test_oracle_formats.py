"""Pins for oracle.formats against the published format tables, torch's own
float8/bfloat16 casts (an independent library routine) and exhaustive
enumeration."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


def test_golden_anchor_values():
    for fmt, code, val in _golden("formats.txt"):
        c = int(code, 16)
        want = float(val)
        if fmt == "e4m3":
            got = float(F.e4m3_decode(c))
        elif fmt == "e2m1":
            got = float(F.e2m1_decode(c))
        else:
            got = float(F.ue8m0_decode(c))
        assert _same(got, want), (fmt, code, got, want)


def test_e4m3_table_matches_torch_float8():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.E4M3_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], ours[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(ours[fin]))


def test_e4m3_grid_monotone_and_count():
    pos = F.E4M3_TABLE[:127]
    assert np.all(np.diff(pos) > 0)
    assert pos[-1] == 448.0
    assert np.isnan(F.E4M3_TABLE[127]) and np.isnan(F.E4M3_TABLE[255])
    assert np.array_equal(F.E4M3_TABLE[128:255], -pos)


def test_e2m1_grid():
    assert list(F.E2M1_TABLE[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(F.E2M1_TABLE[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]


def test_e2m1_midpoint_rounding_golden():
    for v, code in _golden("e2m1_midpoints.txt"):
        assert int(F.e2m1_encode(float(v))) == int(code), v


def test_e4m3_encode_matches_torch_in_range():
    # torch's float -> float8_e4m3fn cast rounds to nearest even but does not
    # saturate; inside [-448, 448] (and below the 464 midpoint) it must agree.
    rng = np.random.default_rng(123)
    v = np.concatenate([
        rng.standard_normal(20000) * 50,
        rng.uniform(-448, 448, 20000),
        (rng.standard_normal(5000) * 2.0 ** -8),
        F.E4M3_TABLE[:127], -F.E4M3_TABLE[:127],
        (F.E4M3_TABLE[:126] + F.E4M3_TABLE[1:127]) / 2,   # exact ties
        [0.0, -0.0, 463.99, -463.99, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -10 * 1.0001],
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F.e4m3_encode(v.astype(np.float64))
    assert np.array_equal(ref, ours)


def test_e4m3_encode_saturates():
    for v in [448.0, 449.0, 464.0, 464.0001, 480.0, 1e30]:
        assert F.e4m3_encode(v) == 0x7E
        assert F.e4m3_encode(-v) == 0xFE


def test_e4m3_encode_exhaustive_nearest():
    # Every code's value and both neighbours' midpoints, checked by plain
    # enumeration of distances over all 127 non-negative codes.
    grid = F.E4M3_TABLE[:127]
    probes = np.concatenate([grid, (grid[:-1] + grid[1:]) / 2,
                             grid[1:] * (1 - 2 ** -20), grid[:-1] * (1 + 2 ** -20) + 1e-300])
    for p in probes:
        d = np.abs(grid - p)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert F.e4m3_encode(p) == want, p


def test_ue4m3_roundtrip():
    for c in range(127):
        assert F.ue4m3_encode(F.ue4m3_decode(c)) == c


def test_nibble_pack_order():
    codes = np.array([[1, 2, 3, 4, 0xF, 0]], np.uint8)
    packed = F.pack_nibbles(codes)
    assert packed.tolist() == [[0x21, 0x43, 0x0F]]
    assert np.array_equal(F.unpack_nibbles(packed), codes)


def test_bf16_decode_all_patterns_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = F.bf16_decode(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], ours[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(ours[fin]))


def test_fp16_decode_all_patterns_matches_numpy_and_torch():
    # every binary16 pattern against numpy's and torch's own float16 decoders
    bits = np.arange(65536, dtype=np.uint16)
    ours = F.fp16_decode(bits)
    ref_np = bits.view(np.float16).astype(np.float64)
    ref_t = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    nan = np.isnan(ref_np)
    assert np.array_equal(np.isnan(ours), nan) and np.array_equal(np.isnan(ref_t), nan)
    assert np.array_equal(ours[~nan], ref_np[~nan]) and np.array_equal(ours[~nan], ref_t[~nan])
    # sign of zero, the largest finite value, the smallest subnormal
    assert np.signbit(F.fp16_decode(np.uint16(0x8000))) and F.fp16_decode(np.uint16(0x8000)) == 0
    assert F.fp16_decode(np.uint16(0x7BFF)) == 65504.0 and F.fp16_decode(np.uint16(0x0001)) == 2.0 ** -24


def test_fp16_round_matches_numpy_and_fixes_the_boundaries():
    rng = np.random.default_rng(16)
    # doubles across the whole binary16 range, subnormals and overflow included
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-30, 18, 200000))
    with np.errstate(over="ignore"):          # numpy's cast overflows to Inf on purpose here
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(F.fp16_round(x), ref)
    # every binary16 value maps to itself; midpoints between neighbours go to the even one
    bits = np.arange(0x7C00, dtype=np.uint16)
    vals = F.fp16_decode(bits)
    assert np.array_equal(F.fp16_round(vals), bits)
    mid = (vals[:-1] + vals[1:]) / 2
    want = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:])
    assert np.array_equal(F.fp16_round(mid), want)
    # overflow: 65519.99 -> 65504, 65520 (the midpoint to 2^16) -> Inf; signs kept
    assert F.fp16_round(65519.99) == 0x7BFF and F.fp16_round(65520.0) == 0x7C00
    assert F.fp16_round(-1e9) == 0xFC00 and F.fp16_round(-0.0) == 0x8000
    assert F.fp16_round(2.0 ** -25) == 0 and F.fp16_round(2.0 ** -25 * 1.0001) == 1


def test_bf16_round_identity_and_midpoints():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_decode(bits)
    fin = np.isfinite(vals)
    assert np.array_equal(F.bf16_round(vals[fin]), bits[fin])
    # midpoints between consecutive positive finite BF16 values are exact in
    # FP32, where torch's float32 -> bfloat16 cast (nearest even) is the
    # independent reference; a nudge in float64 must break the tie.
    pos = np.sort(vals[(vals > 0) & np.isfinite(vals)])
    mid = (pos[:-1] + pos[1:]) / 2
    ref = torch.from_numpy(mid.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_round(mid), ref)
    up = F.bf16_round(mid + (pos[1:] - pos[:-1]) * 2 ** -30)
    dn = F.bf16_round(mid - (pos[1:] - pos[:-1]) * 2 ** -30)
    assert np.array_equal(F.bf16_decode(up), pos[1:])
    assert np.array_equal(F.bf16_decode(dn), pos[:-1])


def test_bf16_round_overflow_and_signs():
    assert F.bf16_round(F.BF16_MAX) == 0x7F7F
    assert F.bf16_round((2 - 2 ** -8) * 2.0 ** 127) == 0x7F80     # tie -> even -> Inf
    assert F.bf16_round(-1e39) == 0xFF80
    assert F.bf16_round(-0.0) == 0x8000
    assert F.bf16_round(2.0 ** -134) == 0x0000                     # tie to even zero
    assert F.bf16_round(2.0 ** -134 * 1.5) == 0x0001
