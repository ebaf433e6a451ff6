// Device-side element-format helpers for gfx950: BF16 unpacking, the MX
// (UE8M0) scale rule, E4M3 / E2M1 round-to-nearest-even encoders with
// saturation, and lane-group reductions.
//
// Formats are the ones named on the HALOps "GEMM" page (group_wise_quant
// section): E4M3 "fn" codes, E2M1 nibbles, UE8M0 and UE4M3 scale bytes; their
// bit layouts are those of the OCP MX v1.0 element definitions.  Every
// encoder works on the IEEE FP32 bit pattern with integer arithmetic only, so
// its result does not depend on a hardware conversion mode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal: the data is read once).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// BF16 halves of a packed dword -> FP32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// FP32 -> BF16 bits, round to nearest even (finite inputs; Inf stays Inf).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The shared exponent of an MX block.  amax_bits is the FP32 pattern of the
// block's largest magnitude.  For a normal amax with biased exponent E,
// floor(log2 amax) = E - 127 and the scale s = floor(log2 amax) - EMAX is
// clamped to [-127, 127]; the stored byte is s + 127 = max(E - EMAX, 0).  A
// zero or subnormal amax has floor(log2) <= -127, which clamps to byte 0.
// (E <= 254 for finite inputs, so the upper clamp is never reached.)
template <int EMAX>
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
  int e = (int)(amax_bits >> 23) - EMAX;
  return e < 0 ? 0u : (uint32_t)e;
}

// |v| (FP32) -> E4M3 magnitude code with round-to-nearest-even, saturating
// at 448 (code 0x7E).  Normal results keep 3 of FP32's 23 mantissa bits (add
// 0x7FFFF plus the kept LSB, truncate); results below 2^-6 sit on the fixed
// subnormal grid of step 2^-9, reached by adding 2^14 (whose FP32 ulp is
// 2^-9) and reading off the integer difference.
__device__ __forceinline__ uint32_t e4m3_mag(uint32_t a /* |v| bits */) {
  a = a < 0x43E00000u ? a : 0x43E00000u;                      // min(|v|, 448)
  uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  uint32_t cn = (r >> 20) - (120u << 3);                       // rebias 127 -> 7
  uint32_t cs = __float_as_uint(__uint_as_float(a) + 16384.0f) - 0x46800000u;
  return a < 0x3C800000u ? cs : cn;                            // 2^-6
}

__device__ __forceinline__ uint32_t e4m3_code(float v) {
  uint32_t u = __float_as_uint(v);
  return e4m3_mag(u & 0x7fffffffu) | ((u >> 24) & 0x80u);
}

// |v| -> E2M1 magnitude code, nearest even, saturating at 6 (code 7).
// Normal results (>= 1) keep 1 mantissa bit; below 1 the grid step is 0.5,
// reached by adding 2^22 (FP32 ulp 0.5).
__device__ __forceinline__ uint32_t e2m1_mag(uint32_t a) {
  a = a < 0x40C00000u ? a : 0x40C00000u;                      // min(|v|, 6)
  uint32_t r = a + 0x1FFFFFu + ((a >> 22) & 1u);
  uint32_t cn = (r >> 22) - (126u << 1);                       // rebias 127 -> 1
  uint32_t cs = __float_as_uint(__uint_as_float(a) + 4194304.0f) - 0x4A800000u;
  return a < 0x3F800000u ? cs : cn;                            // 1.0
}

__device__ __forceinline__ uint32_t e2m1_code(float v) {
  uint32_t u = __float_as_uint(v);
  return e2m1_mag(u & 0x7fffffffu) | ((u >> 28) & 0x8u);
}

// Eight FP32 values of one MX block -> E4M3 codes (two dwords, element i in
// byte i) or E2M1 nibbles (one dword, element i in nibble i), each value
// divided by the block scale 2^(byte - 127), round to nearest even,
// saturating -- with the gfx950 scaled conversions (two values per
// instruction).  These use only the exponent of their scale operand and, for
// power-of-two scales, give exactly e4m3_code / e2m1_code of x * 2^-(byte-127)
// (checked on the device over every finite BF16 input and a range of scale
// exponents), except that FP8 results beyond 448 become NaN rather than
// saturate, hence the clamp to +-448 * scale first.  Blocks with byte < 64
// (|x| < 2^-55) are first multiplied by 2^64, exactly, and converted with
// byte + 64, so the scale operand stays a normal float.
__device__ __forceinline__ float mx_hw_scale(uint32_t byte, float (&f)[8]) {
  if (byte < 64u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] *= 18446744073709551616.0f;   // 2^64
    byte += 64u;
  }
  return __uint_as_float(byte << 23);
}

__device__ __forceinline__ uint2 mx_fp8x8(const float (&x)[8], uint32_t byte) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = x[i];
  const float sc = mx_hw_scale(byte, f);
  const float lim = 448.0f * sc;
  typedef short v2s __attribute__((ext_vector_type(2)));
  v2s lo = {0, 0}, hi = {0, 0};
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, __builtin_amdgcn_fmed3f(f[0], -lim, lim),
                                                __builtin_amdgcn_fmed3f(f[1], -lim, lim), sc, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, __builtin_amdgcn_fmed3f(f[2], -lim, lim),
                                                __builtin_amdgcn_fmed3f(f[3], -lim, lim), sc, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, __builtin_amdgcn_fmed3f(f[4], -lim, lim),
                                                __builtin_amdgcn_fmed3f(f[5], -lim, lim), sc, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, __builtin_amdgcn_fmed3f(f[6], -lim, lim),
                                                __builtin_amdgcn_fmed3f(f[7], -lim, lim), sc, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ __forceinline__ uint32_t mx_fp4x8(const float (&x)[8], uint32_t byte) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = x[i];
  const float sc = mx_hw_scale(byte, f);
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[0], f[1], sc, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2], f[3], sc, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4], f[5], sc, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6], f[7], sc, 3);
  return w;
}

// Eight FP32 values -> E2M1 nibbles (element i in nibble i) of the correctly
// rounded FP32 quotients x / s, for an NVFP4 block's effective scale s >= 0
// (its UE4M3 scale times the global scale, not a power of two); s == 0 gives
// signed zeros.  The hardware conversion with a unit scale operand rounds an
// FP32 value to E2M1 exactly as e2m1_code (nearest even, saturating; checked
// on the device over all 2^32 FP32 patterns).  For s in [2^-56, 2^56] the
// quotients are formed with one shared reciprocal: r = 1/s from the hardware
// reciprocal and one Newton-Raphson step, then per value q = x r and two
// FMA residual corrections q += (x - s q) r -- Markstein's correction scheme
// for correctly rounded division (P. Markstein, "IA-64 and Elementary
// Functions", 2000), which is also what AMD's open FP32 division expansion
// does once its operand-scaling steps leave both operands unscaled.  That
// holds whenever the quotient can round to anything but a zero or a
// saturated code (checked on the device against x / s over every BF16 x and
// random FP32 x, for 2052 scales).
// The sign is copied from x, as the division gives it (x = -0 included).
__device__ __forceinline__ uint32_t nv_fp4x8(const float (&x)[8], float s) {
  float q[8];
  if (s >= 0x1p-56f && s <= 0x1p56f) {
    float r = __builtin_amdgcn_rcpf(s);
    r = __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float t = x[i] * r;
      t = __builtin_fmaf(__builtin_fmaf(-s, t, x[i]), r, t);
      t = __builtin_fmaf(__builtin_fmaf(-s, t, x[i]), r, t);
      q[i] = __builtin_copysignf(t, x[i]);
    }
  } else if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = x[i] / s;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_copysignf(0.0f, x[i]);
  }
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
  return w;
}

// E4M3 / UE4M3 code -> FP32 value (exact).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e == 0 ? (float)m * 0.001953125f                       // m/8 * 2^-6
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// SwiGLU of one element, y = up * gate * sigmoid(gate) in FP32 (HALOps "GEMM"
// page, fused_swiglu_quant section): exp(-gate) through the hardware exp2,
// 1/(1+e) through the hardware reciprocal.  Large negative gates give
// e = +Inf and y = 0.  Shared by the SwiGLU kernel and the GEMM's SwiGLU
// epilogue, so both produce the same y bits from the same BF16 gate/up.
__device__ __forceinline__ float silu_mul(float gate, float up) {
  float e = __builtin_amdgcn_exp2f(-gate * 1.4426950408889634f);
  return up * gate * __builtin_amdgcn_rcpf(1.0f + e);
}

// Max over the 4 lanes of a DPP quad (lanes 4j..4j+3), on non-negative FP32
// bit patterns (integer order == float order).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);           // [2,3,0,1]
  return v > t ? v : t;
}

// Max over lane pairs (2j, 2j+1).
__device__ __forceinline__ uint32_t pair_max_u32(uint32_t v) {
  uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  return v > t ? v : t;
}

// Max over a whole wave (64 lanes); every lane receives the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t t = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > t ? v : t;
  }
  return v;
}

}  // namespace hq
