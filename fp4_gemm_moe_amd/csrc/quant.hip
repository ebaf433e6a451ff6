// Group-wise quantisation of BF16 rows (HALOps "GEMM" page, group_wise_quant
// section; plain row-major scale layout).
//
// Memory-bound: 2 bytes in, 1 (FP8) or 0.5 (FP4) bytes out per element plus
// one scale byte per group.  Work layout: the tensor is cut into blocks of
// kUnroll x 256 consecutive 16-byte chunks of 8 BF16 values, one block per
// workgroup (thread t takes chunks t, t + 256, ...), so neighbouring
// workgroups stream neighbouring memory (measured 14 % faster than a
// grid-stride loop over a capped grid).  Because k % 32 == 0, groups never
// straddle rows, so the [m, k] tensor is processed as one flat array: chunk c covers
// elements 8c..8c+7, its 32-group is c/4 (MX) or its 16-group is c/2
// (NVFP4), which is also the flat index of the scale byte.  The lanes of one
// group are consecutive lanes of a wave, so the group's amax is a DPP
// reduction over a lane quad (MX) or pair (NVFP4) with no LDS traffic.
#include "fmt.hpp"
#include "hq_internal.hpp"

namespace hq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 2;       // chunks in flight per thread (quantisation)

struct Chunk8 {
  float f[8];
};

// Eight 16-bit inputs -> FP32 (exact): BF16 (F16 = false) or IEEE binary16
// (F16 = true, the hardware half -> float conversion).
__device__ __forceinline__ float f16_bits(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <bool F16>
__device__ __forceinline__ Chunk8 unpack(uint4 v) {
  Chunk8 c;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c.f[2 * i] = F16 ? f16_bits(w[i] & 0xFFFFu) : bf16_lo(w[i]);
    c.f[2 * i + 1] = F16 ? f16_bits(w[i] >> 16) : bf16_hi(w[i]);
  }
  return c;
}

__device__ __forceinline__ uint32_t abs_max_bits(const Chunk8& c) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t a = __float_as_uint(c.f[i]) & 0x7fffffffu;
    m = a > m ? a : m;
  }
  return m;
}

// MX quantisation of one chunk whose group amax (all 4 lanes) is known.
// Writes 8 E4M3 bytes or 4 bytes of E2M1 nibbles for chunk index c.
template <int MODE>
__device__ __forceinline__ void mx_emit(const Chunk8& c, uint32_t amax, int64_t ci,
                                        uint8_t* __restrict__ q, uint8_t* __restrict__ sf) {
  constexpr int EMAX = MODE == kMXFP8 ? 8 : 2;
  uint32_t sb = mx_scale_byte<EMAX>(amax);
  if (MODE == kMXFP8) {
    reinterpret_cast<uint2*>(q)[ci] = mx_fp8x8(c.f, sb);
  } else {
    reinterpret_cast<uint32_t*>(q)[ci] = mx_fp4x8(c.f, sb);
  }
  if ((ci & 3) == 0) sf[ci >> 2] = (uint8_t)sb;
}

template <int MODE, bool F16>
__global__ __launch_bounds__(kThreads) void mx_quant_kernel(const uint4* __restrict__ x,
                                                            int64_t nchunks,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ sf) {
  constexpr int64_t kBlock = (int64_t)kUnroll * kThreads;
  for (int64_t base = (int64_t)blockIdx.x * kBlock + threadIdx.x; base < nchunks;
       base += (int64_t)gridDim.x * kBlock) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int64_t ci = base + u * kThreads;
      if (ci < nchunks) v[u] = load_nt(&x[ci]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int64_t ci = base + u * kThreads;
      // nchunks % 4 == 0 and quads start at multiples of 4: a lane quad is
      // all in or all out.
      if (ci < nchunks) {
        Chunk8 c = unpack<F16>(v[u]);
        uint32_t amax = quad_max_u32(abs_max_bits(c));
        mx_emit<MODE>(c, amax, ci, q, sf);
      }
    }
  }
}

// ---------------------------------------------------------------- NVFP4
// Global scale g = amax / 2688 (FP32), in two launches in stream order: every
// workgroup of the first writes the |x| maximum of its block of chunks to a
// slot of its own (the slots sit in q, whose codes are written only by the
// quantisation that follows); one workgroup then folds the slots and writes g.
constexpr int kAmaxUnroll = 4;   // chunks per thread (NVFP4 amax pass)

template <bool F16>
__global__ __launch_bounds__(kThreads) void nv_amax_kernel(const uint4* __restrict__ x,
                                                           int64_t nchunks,
                                                           uint32_t* __restrict__ slots) {
  __shared__ uint32_t wmax[kThreads / 64];
  constexpr int64_t kBlock = (int64_t)kAmaxUnroll * kThreads;
  uint32_t m = 0;
  for (int64_t base = (int64_t)blockIdx.x * kBlock + threadIdx.x; base < nchunks;
       base += (int64_t)gridDim.x * kBlock) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t ci = base + u * kThreads;
      v[u] = ci < nchunks ? x[ci] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const uint32_t a = abs_max_bits(unpack<F16>(v[u]));
      m = a > m ? a : m;
    }
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) b = wmax[i] > b ? wmax[i] : b;
    slots[blockIdx.x] = b;
  }
}

constexpr int kFoldThreads = 1024;

__global__ __launch_bounds__(kFoldThreads) void nv_gs_fold(const uint32_t* __restrict__ slots,
                                                           int64_t nslots, float* __restrict__ gs) {
  __shared__ uint32_t wmax[kFoldThreads / 64];
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < nslots; i += kFoldThreads) m = slots[i] > m ? slots[i] : m;
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = 0;
#pragma unroll
    for (int i = 0; i < kFoldThreads / 64; ++i) b = wmax[i] > b ? wmax[i] : b;
    const float a = __uint_as_float(b);
    *gs = a == 0.0f ? 1.0f : a / 2688.0f;
  }
}

// NVFP4: per 16-group (two lanes of 8), sf = UE4M3(amax_b / (6 g)),
// s_eff = decode(sf) * g, code = E2M1(x / s_eff) with correctly rounded FP32
// quotients.
__device__ __forceinline__ void nv_emit(const Chunk8& c, uint32_t amax_bits, float g, float d,
                                        int64_t ci, uint8_t* __restrict__ q,
                                        uint8_t* __restrict__ sf) {
  float ratio = __uint_as_float(amax_bits) / d;
  uint32_t sb = e4m3_mag(__float_as_uint(ratio) & 0x7fffffffu);
  float s_eff = e4m3_value(sb) * g;
  const uint32_t w = nv_fp4x8(c.f, s_eff);
  // non-temporal: 6 % faster at [4096, 17408] (the MX kernels measured no change)
  __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(q) + ci);
  if ((ci & 1) == 0) sf[ci >> 1] = (uint8_t)sb;
}

template <bool F16>
__global__ __launch_bounds__(kThreads) void nv_quant_kernel(const uint4* __restrict__ x,
                                                            int64_t nchunks,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ sf,
                                                            const float* __restrict__ gs) {
  const float g = *gs;
  const float d = 6.0f * g;
  constexpr int64_t kBlock = (int64_t)kUnroll * kThreads;
  for (int64_t base = (int64_t)blockIdx.x * kBlock + threadIdx.x; base < nchunks;
       base += (int64_t)gridDim.x * kBlock) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int64_t ci = base + u * kThreads;
      if (ci < nchunks) v[u] = load_nt(&x[ci]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int64_t ci = base + u * kThreads;
      if (ci < nchunks) {
        Chunk8 c = unpack<F16>(v[u]);
        uint32_t amax = pair_max_u32(abs_max_bits(c));
        nv_emit(c, amax, g, d, ci, q, sf);
      }
    }
  }
}

// One workgroup per block of kUnroll x 256 chunks (the loop in the kernels
// only runs more than once past 2^30 blocks).
int grid_for(int64_t nchunks, int per_thread) {
  int64_t blocks = (nchunks + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  if (blocks > (1ll << 30)) blocks = 1ll << 30;
  return blocks < 1 ? 1 : (int)blocks;
}

}  // namespace

namespace {
template <bool F16>
hipError_t launch_quant_t(hipStream_t s, int mode, const uint16_t* x, int64_t m, int64_t k,
                          uint8_t* q, uint8_t* sf, float* gs, bool gs_input) {
  const int64_t nchunks = m * k / 8;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int grid = grid_for(nchunks, kUnroll);
  if (mode == kMXFP8) {
    hipLaunchKernelGGL((mx_quant_kernel<kMXFP8, F16>), dim3(grid), dim3(kThreads), 0, s, xv, nchunks, q, sf);
  } else if (mode == kMXFP4) {
    hipLaunchKernelGGL((mx_quant_kernel<kMXFP4, F16>), dim3(grid), dim3(kThreads), 0, s, xv, nchunks, q, sf);
  } else {
    if (!gs_input) {
      // one slot per amax workgroup, in q (4 bytes per chunk of codes)
      const int ablocks = grid_for(nchunks, kAmaxUnroll);
      uint32_t* slots = reinterpret_cast<uint32_t*>(q);
      hipLaunchKernelGGL(nv_amax_kernel<F16>, dim3(ablocks), dim3(kThreads), 0, s, xv, nchunks, slots);
      hipLaunchKernelGGL(nv_gs_fold, dim3(1), dim3(kFoldThreads), 0, s, (const uint32_t*)slots,
                         (int64_t)ablocks, gs);
    }
    hipLaunchKernelGGL(nv_quant_kernel<F16>, dim3(grid), dim3(kThreads), 0, s, xv, nchunks, q, sf,
                       (const float*)gs);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_quant(hipStream_t s, int mode, const uint16_t* x, int64_t m, int64_t k,
                        uint8_t* q, uint8_t* sf, float* gs, bool gs_input, bool fp16) {
  return fp16 ? launch_quant_t<true>(s, mode, x, m, k, q, sf, gs, gs_input)
              : launch_quant_t<false>(s, mode, x, m, k, q, sf, gs, gs_input);
}

}  // namespace hq
