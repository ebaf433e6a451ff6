// Pieces shared by the GEMM kernels: the scaled-MFMA wrapper, the tile space
// of a grouped problem, and the BF16 epilogue store.
//
// GEMM definition: HALOps "GEMM" page, dense_gemm section (output = input @
// weight^T + bias, BF16 output); the grouped forms follow the batch_gemm,
// group_contiguous_gemm and group_masked_gemm sections and cuDNN FE "Grouped
// GEMM + dGLU (SM100)" Step 1 (sum over k of dequantize(A) * dequantize(B)).
//
// Matrix-core contract used here (gfx950 V_MFMA_SCALE_F32_16X16X128_F8F6F4):
// operand src0 is a 16 x 128 tile, src1 a 128 x 16 tile; lane l supplies row
// (l % 16) of src0 / column (l % 16) of src1, and lane group q = l / 16
// supplies the E8M0 scale of K block [32q, 32q + 32) of that row.  Which
// elements a lane's data registers hold depends on the element width (all
// established on the device with integer-coded and one-hot probes):
//   FP4 (4 dwords): elements [32q, 32q + 32), two per byte, low nibble first;
//   FP8 (8 dwords): elements [16q, 16q + 16) in dwords 0-3 and
//                   [64 + 16q, 64 + 16q + 16) in dwords 4-7.
// The 16 x 16 FP32 result lands as D[4 * (l / 16) + r][l % 16] in
// accumulator register r.  We feed the
// weights as src0 and the activations as src1, so lane l holds
// out[m = l % 16][n = 4 * (l / 16) + r]: four consecutive output columns,
// one 8-byte BF16 store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fmt.hpp"
#include "hq_internal.hpp"
#include "sched.hpp"

namespace hq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// FMT: 0 = FP8 E4M3 operands, 4 = FP4 E2M1 operands (the instruction's
// cbsz / blgp format codes).
template <int FMT>
__device__ __forceinline__ v4f mfma_scaled(v8i w, v8i x, v4f acc, int sw, int sx) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, acc, FMT, FMT, 0, sw, 0, sx);
}

// 8 nibbles times one UE4M3 scale -> 8 FP16 (exact: a product has at most
// 6 significant bits and lies in [2^-10, 2688], inside FP16's normal range).
// Nibbles decode to FP16 with the hardware FP4 conversion (scale 1) and take
// the scale with packed FP16 multiplies, two values per instruction each.
__device__ __forceinline__ v8h decode8(uint32_t w, _Float16 sc) {
  const h2 s2 = {sc, sc};
  const h2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const h2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const h2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const h2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return v8h{f0[0], f0[1], f1[0], f1[1], f2[0], f2[1], f3[0], f3[1]};
}

// Rows owned by group g and the tile space (group m-tiles x n-tiles).
struct GroupRows {
  int64_t start;
  int64_t count;
};

// LDS tables for grouped forms: per group start row, row count and the
// inclusive prefix of m-tiles.  Uniform forms need no table.
struct TileTable {
  int start[kMaxGroups];
  int count[kMaxGroups];
  int mt_prefix[kMaxGroups];
};

// Fills the table (all threads must call) and returns the total number of
// group m-tiles.  Rows are clamped as documented for device-side values.
template <int NT>
__device__ inline int build_tile_table(const GemmArgs& p, int TM, TileTable& t) {
  const int G = p.num_groups;
  if (p.form == kContiguous) {
    load_clamped_ends<NT>(t.mt_prefix, p.group_end, G, p.m_rows);   // reuse as scratch
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
      int e = t.mt_prefix[g];
      int s = g > 0 ? t.mt_prefix[g - 1] : 0;
      t.start[g] = s;
      t.count[g] = e - s;
    }
  } else {
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
      int64_t c = p.slot_rows;
      if (p.form == kMasked) {
        int64_t v = p.counts[g];
        c = v < 0 ? 0 : (v > p.slot_rows ? p.slot_rows : v);
      }
      t.start[g] = (int)(g * p.slot_rows);
      t.count[g] = (int)c;
    }
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x) t.mt_prefix[g] = (t.count[g] + TM - 1) / TM;
  __syncthreads();
  return block_scan_1024<NT>(t.mt_prefix, G, OpAdd(), 0);
}

// Group owning linear group-m-tile index gm (prefix is inclusive).
__device__ inline int tile_group(const TileTable& t, int G, int gm) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (t.mt_prefix[mid] > gm) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Four consecutive FP32 results of one output row -> BF16 (nearest even),
// with the optional bias, written as one 8-byte store.
// Four FP32 results (+ BF16 bias) -> four BF16 (or, with f16, binary16)
// values, each rounded to nearest even once.
__device__ __forceinline__ void store_bf16x4(uint16_t* dst, v4f v, const uint16_t* bias4, bool f16 = false) {
  float f[4] = {v[0], v[1], v[2], v[3]};
  if (bias4 != nullptr) {
    uint2 bb = *reinterpret_cast<const uint2*>(bias4);
    f[0] += bf16_lo(bb.x);
    f[1] += bf16_hi(bb.x);
    f[2] += bf16_lo(bb.y);
    f[3] += bf16_hi(bb.y);
  }
  uint2 o;
  if (f16) {
    auto h = [](float x) -> uint32_t { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x); };
    o.x = h(f[0]) | (h(f[1]) << 16);
    o.y = h(f[2]) | (h(f[3]) << 16);
  } else {
    o.x = f32_to_bf16(f[0]) | (f32_to_bf16(f[1]) << 16);
    o.y = f32_to_bf16(f[2]) | (f32_to_bf16(f[3]) << 16);
  }
  *reinterpret_cast<uint2*>(dst) = o;
}

}  // namespace hq
