// Direct-load scaled GEMMs: every lane fetches its own MFMA operand slice
// straight from global memory (no LDS staging), four waves split the K loop
// and their partial tiles are summed through LDS.
//
// This path serves
//   * skinny M (the decode / small-batch tier of the flashrt/fp4-gemm page's
//     M-tiered dispatch): the weights stream from HBM once, the tiny A tile is
//     re-read from cache, and the K split keeps enough waves busy;
//   * any K with k % 32 == 0 (a lane's K slice is exactly one 32-group, so a
//     ragged K tail is a per-lane predicate: zero codes, unit scale);
//   * NVFP4 in those shapes (UE4M3 scales per 16 cannot be folded into the
//     E8M0-scaled instruction, so codes are decoded to FP16 -- exactly: an
//     E2M1 value times a UE4M3 value has at most 6 significant bits and lies
//     in FP16's normal range -- and multiplied on the FP16 matrix cores;
//     alpha = g_A * g_B is applied in FP32).
#include <mutex>
#include <vector>

#include "gemm_common.hpp"

namespace hq {
namespace {

constexpr int kThreads = 256;   // 4 waves = 4-way K split (NVFP4 and multi-fragment tiles)

typedef short v8s __attribute__((ext_vector_type(8)));

// Resolves linear group-m-tile gm to (group, first row, row end).
struct TileRows {
  int g;
  int64_t row0, row_end;
};

__device__ __forceinline__ TileRows resolve_tile(const GemmArgs& p, const TileTable& tt, int TM,
                                                 int mt_per_uniform, int gm) {
  TileRows t;
  if (p.form == kUniform) {
    t.g = gm / mt_per_uniform;
    int mt = gm - t.g * mt_per_uniform;
    int64_t gs = (int64_t)t.g * p.slot_rows;
    t.row0 = gs + (int64_t)mt * TM;
    int64_t ge = gs + p.slot_rows;
    t.row_end = t.row0 + TM < ge ? t.row0 + TM : ge;
  } else {
    t.g = tile_group(tt, p.num_groups, gm);
    int mt = gm - (t.g > 0 ? tt.mt_prefix[t.g - 1] : 0);
    t.row0 = (int64_t)tt.start[t.g] + (int64_t)mt * TM;
    int64_t ge = (int64_t)tt.start[t.g] + tt.count[t.g];
    t.row_end = t.row0 + TM < ge ? t.row0 + TM : ge;
  }
  return t;
}

// One lane's operand slice for K step t (128 elements) and its scale byte.
// FP4: lane group q holds the 32 codes of block 4t + q (16 bytes, dwords
// 0-3).  FP8: the instruction reads the 32 bytes of lane group q as elements
// [16q, 16q + 16) (dwords 0-3) and [64 + 16q, 64 + 16q + 16) (dwords 4-7) of
// the step, while the scale register of lane group q belongs to block
// [32q, 32q + 32).  Blocks at or past K contribute zero codes (scale 2^0).
template <int FMT>
__device__ __forceinline__ void load_slice(const uint8_t* row_codes, const uint8_t* row_sf,
                                           int t, int q, int kgroups, v8i& frag, int& sc) {
  const int kg = t * 4 + q;
  if (FMT == 0) {
    const uint8_t* base = row_codes + (int64_t)t * 128 + 16 * q;
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (t * 4 + (q >> 1) < kgroups) lo = *reinterpret_cast<const uint4*>(base);
    if (t * 4 + 2 + (q >> 1) < kgroups) hi = *reinterpret_cast<const uint4*>(base + 64);
    frag = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  } else {
    uint4 lo = make_uint4(0, 0, 0, 0);
    if (kg < kgroups) lo = *reinterpret_cast<const uint4*>(row_codes + (int64_t)kg * 16);
    frag = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
  }
  sc = kg < kgroups ? (int)row_sf[kg] : 127;
}

// Codes only of the same slice (zeros when !in); the scale bytes come from
// one 8-byte load per K-step pair instead.
template <int FMT>
__device__ __forceinline__ v8i load_codes(const uint8_t* row_codes, int t, int q, bool in) {
  if (FMT == 0) {
    const uint8_t* base = row_codes + (int64_t)t * 128 + 16 * q;
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (in) {
      lo = *reinterpret_cast<const uint4*>(base);
      hi = *reinterpret_cast<const uint4*>(base + 64);
    }
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  uint4 lo = make_uint4(0, 0, 0, 0);
  if (in) lo = *reinterpret_cast<const uint4*>(row_codes + (int64_t)(t * 4 + q) * 16);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
}

// The block's NW = blockDim.x / 64 waves (at most NWMAX; at least 4 for the
// grouped forms, whose tile table takes 256 threads) split K: wave w takes K
// steps w, w + NW, ..., U steps per trip so that U loads per operand are in
// flight per wave; the NW partial tiles are summed through LDS.
// SP > 1 (K % (128 SP) == 0, scale rows 4 SP-byte aligned): the K steps go to
// the waves in groups of SP (group j = steps SP j .. SP j + SP - 1, wave w
// takes groups w, w + NW, ...) and a lane reads the 4 SP scale bytes of a
// group in one 8- or 16-byte load (its lane group's bytes are q, 4 + q, ...)
// instead of one byte per step: one memory transaction per row for SP steps.
template <int SP>
__device__ __forceinline__ void scale_words(const uint8_t* p, bool in, uint32_t (&w)[SP]) {
  if constexpr (SP == 2) {
    const uint2 v = in ? *reinterpret_cast<const uint2*>(p) : make_uint2(0u, 0u);
    w[0] = v.x;
    w[1] = v.y;
  } else {
    static_assert(SP == 4, "groups of 2 or 4 K steps");
    const uint4 v = in ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  }
}

// PA: the weights of group g sit at the addresses b_ptrs[g] / sfb_ptrs[g]
// (discrete expert tensors) instead of at g * stride from one base; a
// separate instantiation, so the packed-weights kernels carry no select.
template <int FMT, int FM, int FN, int NWMAX, int U, int SP = 1, bool PA = false>
__global__ __launch_bounds__(NWMAX * 64) void mx_gemm_direct(GemmArgs p) {
  constexpr int TM = 16 * FM, TN = 16 * FN;
  __shared__ TileTable tt;
  __shared__ v4f red[NWMAX - 1][FM * FN][64];
  const int NW = (int)(blockDim.x >> 6);

  const int G = p.num_groups;
  const int NT = (int)((p.n + TN - 1) / TN);
  const int mt_per = (int)((p.slot_rows + TM - 1) / TM);
  int total_gm;
  if (p.form == kUniform) total_gm = G * mt_per;
  else total_gm = build_tile_table<256>(p, TM, tt);
  const int total = total_gm * NT;

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane >> 4, r16 = lane & 15;
  const int kgroups = (int)(p.k / 32);
  const int ksteps = (kgroups + 3) / 4;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int gm = tile / NT, nt = tile - (tile / NT) * NT;
    const TileRows tr = resolve_tile(p, tt, TM, mt_per, gm);
    const int64_t n0 = (int64_t)nt * TN;

    const uint8_t* arow[FM];
    const uint8_t* asf[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      int64_t r = tr.row0 + fm * 16 + r16;
      r = r < tr.row_end ? r : tr.row_end - 1;     // rows past the tile end re-read a valid row
      arow[fm] = p.a + r * p.lda;
      asf[fm] = p.sfa + r * p.ldsf;
    }
    const uint8_t* bg = PA ? reinterpret_cast<const uint8_t*>(p.b_ptrs[tr.g]) : p.b + (int64_t)tr.g * p.b_stride;
    const uint8_t* bsg = PA ? reinterpret_cast<const uint8_t*>(p.sfb_ptrs[tr.g]) : p.sfb + (int64_t)tr.g * p.sfb_stride;
    const uint8_t* brow[FN];
    const uint8_t* bsf[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      int64_t r = n0 + fn * 16 + r16;
      r = r < p.n ? r : p.n - 1;
      brow[fn] = bg + r * p.lda;
      bsf[fn] = bsg + r * p.ldsf;
    }

    v4f acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = v4f{0.f, 0.f, 0.f, 0.f};

    if constexpr (SP > 1) {
      static_assert(U % SP == 0, "whole scale groups per trip");
      const int ngroups = ksteps / SP;
      for (int p0 = w; p0 < ngroups; p0 += NW * (U / SP)) {
        v8i af[U][FM], bf[U][FN];
        int sa[U][FM], sb[U][FN];
#pragma unroll
        for (int v = 0; v < U / SP; ++v) {
          const int pp = p0 + NW * v;
          const bool in = pp < ngroups;
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            uint32_t sw[SP];
            scale_words<SP>(asf[fm] + 4 * SP * (int64_t)pp, in, sw);
#pragma unroll
            for (int e = 0; e < SP; ++e) {
              af[SP * v + e][fm] = load_codes<FMT>(arow[fm], SP * pp + e, q, in);
              sa[SP * v + e][fm] = (int)((sw[e] >> (8 * q)) & 0xFFu);
            }
          }
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            uint32_t sw[SP];
            scale_words<SP>(bsf[fn] + 4 * SP * (int64_t)pp, in, sw);
#pragma unroll
            for (int e = 0; e < SP; ++e) {
              bf[SP * v + e][fn] = load_codes<FMT>(brow[fn], SP * pp + e, q, in);
              sb[SP * v + e][fn] = (int)((sw[e] >> (8 * q)) & 0xFFu);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              acc[fm][fn] = mfma_scaled<FMT>(bf[u][fn], af[u][fm], acc[fm][fn], sb[u][fn], sa[u][fm]);
      }
    } else {
      for (int t = w; t < ksteps; t += NW * U) {
        v8i af[U][FM], bf[U][FN];
        int sa[U][FM], sb[U][FN];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) load_slice<FMT>(arow[fm], asf[fm], t + NW * u, q, kgroups, af[u][fm], sa[u][fm]);
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) load_slice<FMT>(brow[fn], bsf[fn], t + NW * u, q, kgroups, bf[u][fn], sb[u][fn]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              acc[fm][fn] = mfma_scaled<FMT>(bf[u][fn], af[u][fm], acc[fm][fn], sb[u][fn], sa[u][fm]);
      }
    }

    if (w > 0) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) red[w - 1][fm * FN + fn][lane] = acc[fm][fn];
    }
    __syncthreads();
    if (w == 0) {
      const uint16_t* bias = p.bias ? p.bias + (int64_t)tr.g * p.n : nullptr;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int64_t m = tr.row0 + fm * 16 + r16;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          v4f v = acc[fm][fn];
          for (int i = 0; i < NW - 1; ++i) v += red[i][fm * FN + fn][lane];
          const int64_t n = n0 + fn * 16 + 4 * q;
          if (m < tr.row_end && n < p.n)
            store_bf16x4(p.out + m * p.n + n, v, bias ? bias + n : nullptr, p.out_f16 != 0);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- NVFP4
// Lane slice for NVFP4: 32 elements [32 kb, 32 kb + 32) of a row (16 bytes)
// and the two UE4M3 scales of its 16-groups.  The four FP16 MFMAs of one K
// step consume its elements 8s..8s+7 (s = 0..3); the same K permutation is
// applied to both operands, so the dot products are unchanged.
struct NvSlice {
  uint4 codes;
  _Float16 s0, s1;       // the two UE4M3 scales (exact in FP16)
};

__device__ __forceinline__ NvSlice nv_load(const uint8_t* row_codes, const uint8_t* row_sf, int kb,
                                           bool kin) {
  NvSlice s;
  if (kin) {
    s.codes = *reinterpret_cast<const uint4*>(row_codes + (int64_t)kb * 16);
    s.s0 = (_Float16)e4m3_value(row_sf[(int64_t)kb * 2] & 0x7Fu);
    s.s1 = (_Float16)e4m3_value(row_sf[(int64_t)kb * 2 + 1] & 0x7Fu);
  } else {
    s.codes = make_uint4(0, 0, 0, 0);
    s.s0 = s.s1 = (_Float16)0.0f;
  }
  return s;
}

// SC16 (K % 256 == 0, scale rows 16-byte aligned): K steps in pairs as for
// mx_gemm_direct; a lane reads the 16 scale bytes of a pair in one load and
// decodes its two UE4M3 bytes per step with the hardware FP8 conversion.
// PA as for mx_gemm_direct.  One-fragment tiles are held to 128 VGPRs (4
// waves per SIMD), so that two 512-thread blocks share a CU: left alone the
// compiler takes 129 and the skinny launch runs one block per CU.
template <int FM, int FN, int NWMAX, int U, bool SC16 = false, bool PA = false>
__global__ __launch_bounds__(NWMAX * 64, FM == 1 ? 4 : 1) void nv_gemm_direct(GemmArgs p) {
  constexpr int TM = 16 * FM, TN = 16 * FN;
  __shared__ TileTable tt;
  __shared__ v4f red[NWMAX - 1][FM * FN][64];
  const int NW = (int)(blockDim.x >> 6);       // as for mx_gemm_direct

  const int G = p.num_groups;
  const int NT = (int)((p.n + TN - 1) / TN);
  const int mt_per = (int)((p.slot_rows + TM - 1) / TM);
  int total_gm;
  if (p.form == kUniform) total_gm = G * mt_per;
  else total_gm = build_tile_table<256>(p, TM, tt);
  const int total = total_gm * NT;

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane >> 4, r16 = lane & 15;
  const int kblocks = (int)(p.k / 32);
  const int ksteps = (kblocks + 3) / 4;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int gm = tile / NT, nt = tile - (tile / NT) * NT;
    const TileRows tr = resolve_tile(p, tt, TM, mt_per, gm);
    const int64_t n0 = (int64_t)nt * TN;
    const uint8_t* arow[FM];
    const uint8_t* asf[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      int64_t r = tr.row0 + fm * 16 + r16;
      r = r < tr.row_end ? r : tr.row_end - 1;
      arow[fm] = p.a + r * p.lda;
      asf[fm] = p.sfa + r * p.ldsf;
    }
    const uint8_t* bg = PA ? reinterpret_cast<const uint8_t*>(p.b_ptrs[tr.g]) : p.b + (int64_t)tr.g * p.b_stride;
    const uint8_t* bsg = PA ? reinterpret_cast<const uint8_t*>(p.sfb_ptrs[tr.g]) : p.sfb + (int64_t)tr.g * p.sfb_stride;
    const uint8_t* brow[FN];
    const uint8_t* bsf[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      int64_t r = n0 + fn * 16 + r16;
      r = r < p.n ? r : p.n - 1;
      brow[fn] = bg + r * p.lda;
      bsf[fn] = bsg + r * p.ldsf;
    }
    v4f acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = v4f{0.f, 0.f, 0.f, 0.f};

    // trips: U steps each; with SC16 the steps of a trip are U / 2 pairs
    const int trip_stride = SC16 ? NW * (U / 2) : NW * U;
    const int trips_end = SC16 ? (ksteps >> 1) : ksteps;
    for (int t0 = w; t0 < trips_end; t0 += trip_stride) {
      NvSlice as[U][FM], bs[U][FN];
      if constexpr (SC16) {
        static_assert(U % 2 == 0, "whole pairs per trip");
        typedef float v2f __attribute__((ext_vector_type(2)));
        auto pair_slices = [&](const uint8_t* rc, const uint8_t* rs, int pp, bool in, NvSlice* out2) {
          const uint4 s16 = in ? *reinterpret_cast<const uint4*>(rs + 16 * (int64_t)pp) : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int kb = (2 * pp + e) * 4 + q;
            out2[e].codes = in ? *reinterpret_cast<const uint4*>(rc + (int64_t)kb * 16) : make_uint4(0, 0, 0, 0);
            // bytes 8e + 2q and 8e + 2q + 1 of the pair: dword 2e + q/2, half q & 1
            const uint32_t d = e == 0 ? (q < 2 ? s16.x : s16.y) : (q < 2 ? s16.z : s16.w);
            const h2 f = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((d >> (16 * (q & 1))) & 0x7F7Fu, 1.0f, false);
            out2[e].s0 = f[0];
            out2[e].s1 = f[1];
          }
        };
#pragma unroll
        for (int v = 0; v < U / 2; ++v) {
          const int pp = t0 + NW * v;
          const bool in = pp < (ksteps >> 1);
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            NvSlice two[2];
            pair_slices(arow[fm], asf[fm], pp, in, two);
            as[2 * v][fm] = two[0];
            as[2 * v + 1][fm] = two[1];
          }
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            NvSlice two[2];
            pair_slices(brow[fn], bsf[fn], pp, in, two);
            bs[2 * v][fn] = two[0];
            bs[2 * v + 1][fn] = two[1];
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int kb = (t0 + NW * u) * 4 + q;
          const bool kin = kb < kblocks;
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) as[u][fm] = nv_load(arow[fm], asf[fm], kb, kin);
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) bs[u][fn] = nv_load(brow[fn], bsf[fn], kb, kin);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v8h ad[FM], bd[FN];
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            const uint4 c = as[u][fm].codes;
            const uint32_t wd = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
            ad[fm] = decode8(wd, s < 2 ? as[u][fm].s0 : as[u][fm].s1);
          }
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const uint4 c = bs[u][fn].codes;
            const uint32_t wd = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
            bd[fn] = decode8(wd, s < 2 ? bs[u][fn].s0 : bs[u][fn].s1);
          }
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bd[fn], ad[fm], acc[fm][fn], 0, 0, 0);
        }
      }
    }

    if (w > 0) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) red[w - 1][fm * FN + fn][lane] = acc[fm][fn];
    }
    __syncthreads();
    if (w == 0) {
      const float alpha = p.alpha ? p.alpha[tr.g] : 1.0f;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int64_t m = tr.row0 + fm * 16 + r16;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          v4f v = acc[fm][fn];
          for (int i = 0; i < NW - 1; ++i) v += red[i][fm * FN + fn][lane];
          v = v * alpha;
          const int64_t n = n0 + fn * 16 + 4 * q;
          if (m < tr.row_end && n < p.n) store_bf16x4(p.out + m * p.n + n, v, nullptr, p.out_f16 != 0);
        }
      }
    }
    __syncthreads();
  }
}

// Resident blocks per CU of `fn` at `threads` threads (the runtime's
// occupancy calculator, cached per kernel and block size).
int blocks_per_cu(const void* fn, int threads) {
  struct Entry {
    const void* fn;
    int threads, blocks;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : cache)
    if (e.fn == fn && e.threads == threads) return e.blocks;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, 0) != hipSuccess || nb < 1) nb = 1;
  cache.push_back(Entry{fn, threads, nb});
  return nb;
}

int64_t tile_count(const GemmArgs& p, int TM, int TN) {
  const int64_t NT = (p.n + TN - 1) / TN;
  int64_t gm_upper;
  if (p.form == kContiguous) gm_upper = (p.m_rows + TM - 1) / TM + p.num_groups;
  else gm_upper = (int64_t)p.num_groups * ((p.slot_rows + TM - 1) / TM);
  return gm_upper * NT;
}

// Waves per block for a skinny (one-fragment) tile, whose weights stream
// once: the most waves, up to NWMAX and the K steps, for which every tile
// has a resident block at once (a second, partial round of blocks would
// nearly double the time).  Grouped forms need at least 4 waves.
template <class K>
int skinny_waves(K kernel, int nwmax, const GemmArgs& p, int TM, int TN, const DeviceInfo& dev, int sp = 1) {
  const int64_t tiles = tile_count(p, TM, TN);
  int cus = dev.num_cus;
  if (p.cu_limit > 0 && p.cu_limit < cus) cus = p.cu_limit;
  const int64_t ksteps = (p.k / 32 + 3) / 4 / sp;      // units of work dealt to the waves
  const int lo = p.form == kUniform ? 1 : 4;
  int hi = nwmax;
  if (ksteps < hi) hi = ksteps > lo ? (int)ksteps : lo;
  for (int nw = hi; nw > lo; --nw)
    if ((int64_t)blocks_per_cu((const void*)kernel, nw * 64) * cus >= tiles) return nw;
  return lo;
}

template <class K>
hipError_t launch_direct(hipStream_t s, K kernel, const GemmArgs& p, int TM, int TN,
                         const DeviceInfo& dev, int threads = kThreads) {
  const int64_t tiles = tile_count(p, TM, TN);
  int cus = dev.num_cus;
  if (p.cu_limit > 0 && p.cu_limit < cus) cus = p.cu_limit;
  int64_t grid = (int64_t)cus * 8;
  if (tiles < grid) grid = tiles;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, s, p);
  return hipGetLastError();
}

// Picks the tile shape from the rows per group and N.
template <bool PA>
hipError_t launch_direct_pa(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  const int64_t rows_hint = p.form == kContiguous ? p.m_rows : p.slot_rows;
  const int fm = rows_hint <= 16 ? 1 : (rows_hint <= 32 ? 2 : 4);
  // one 16-row fragment (skinny M): for MX the wave count follows the tile
  // count; NVFP4's decode keeps more registers live, so it keeps 8 waves
  // (512-thread bounds) unless there are fewer tiles than CUs (measured)
  if (p.mode == kNVFP4) {
    if (fm == 1) {
      int cus = dev.num_cus;
      if (p.cu_limit > 0 && p.cu_limit < cus) cus = p.cu_limit;
      const bool few = tile_count(p, 16, 32) < cus && p.k >= 16 * 128;
      const bool sc16 = p.k % 256 == 0 &&
                        ((reinterpret_cast<uintptr_t>(p.sfa) | reinterpret_cast<uintptr_t>(p.sfb)) & 15) == 0;
      if (sc16) {
        if (few) return launch_direct(s, nv_gemm_direct<1, 2, 16, 2, true, PA>, p, 16, 32, dev, 1024);
        return launch_direct(s, nv_gemm_direct<1, 2, 8, 2, true, PA>, p, 16, 32, dev, 512);
      }
      if (few) return launch_direct(s, nv_gemm_direct<1, 2, 16, 2, false, PA>, p, 16, 32, dev, 1024);
      return launch_direct(s, nv_gemm_direct<1, 2, 8, 2, false, PA>, p, 16, 32, dev, 512);
    }
    if (fm == 2) return launch_direct(s, nv_gemm_direct<2, 2, 4, 1, false, PA>, p, 32, 32, dev);
    return launch_direct(s, nv_gemm_direct<4, 2, 4, 1, false, PA>, p, 64, 32, dev);
  }
  // scale rows in whole, aligned groups of 2 or 4 K steps (8 or 16 bytes)
  const uintptr_t sfal = reinterpret_cast<uintptr_t>(p.sfa) | reinterpret_cast<uintptr_t>(p.sfb);
  const bool sc8 = p.k % 256 == 0 && (sfal & 7) == 0;
  const bool sc16 = p.k % 512 == 0 && (sfal & 15) == 0;
  if (p.mode == kMXFP8) {
    if (fm == 1) {
      if (sc16) {
        auto k = mx_gemm_direct<0, 1, 1, 16, 4, 4, PA>;
        return launch_direct(s, k, p, 16, 16, dev, 64 * skinny_waves(k, 16, p, 16, 16, dev, 4));
      }
      if (sc8) {
        auto k = mx_gemm_direct<0, 1, 1, 16, 4, 2, PA>;
        return launch_direct(s, k, p, 16, 16, dev, 64 * skinny_waves(k, 16, p, 16, 16, dev));
      }
      auto k = mx_gemm_direct<0, 1, 1, 16, 4, 1, PA>;
      return launch_direct(s, k, p, 16, 16, dev, 64 * skinny_waves(k, 16, p, 16, 16, dev));
    }
    if (fm == 2) return launch_direct(s, mx_gemm_direct<0, 2, 2, 4, 2, 1, PA>, p, 32, 32, dev);
    return launch_direct(s, mx_gemm_direct<0, 4, 4, 4, 2, 1, PA>, p, 64, 64, dev);
  }
  if (fm == 1) {
    if (sc16) {
      auto k = mx_gemm_direct<4, 1, 1, 16, 4, 4, PA>;
      return launch_direct(s, k, p, 16, 16, dev, 64 * skinny_waves(k, 16, p, 16, 16, dev, 4));
    }
    if (sc8) {
      auto k = mx_gemm_direct<4, 1, 1, 16, 4, 2, PA>;
      return launch_direct(s, k, p, 16, 16, dev, 64 * skinny_waves(k, 16, p, 16, 16, dev));
    }
    auto k = mx_gemm_direct<4, 1, 1, 16, 4, 1, PA>;
    return launch_direct(s, k, p, 16, 16, dev, 64 * skinny_waves(k, 16, p, 16, 16, dev));
  }
  if (fm == 2) return launch_direct(s, mx_gemm_direct<4, 2, 2, 4, 2, 1, PA>, p, 32, 32, dev);
  return launch_direct(s, mx_gemm_direct<4, 4, 4, 4, 2, 1, PA>, p, 64, 64, dev);
}

}  // namespace

// Direct path entry.
hipError_t launch_gemm_direct(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  return p.b_ptrs ? launch_direct_pa<true>(s, p, dev) : launch_direct_pa<false>(s, p, dev);
}

}  // namespace hq
