// Token permute into the masked-GEMM layout (HALOps "GEMM" page,
// prefill_permute_to_masked_gemm section): each (token, slot) pair of the
// top-k routing with expert id e in [0, E) sends the token's row to the next
// free row of expert e's slot [e * max_tokens, (e + 1) * max_tokens), writes
// that expert-local row to the map, and re-lays the token's scale factors
// out at one byte per 32 elements.
//
// Three launches on the stream:
//   1. clear the E counters (a fill kernel, safe to capture in a graph);
//   2. one wave per token: lane j claims a row for slot j with an atomic add
//      on its expert's counter (rows past max_tokens are dropped: map -1),
//      then the wave reads the token's row once, 16 bytes per lane, and
//      stores it to every claimed row; the scale row likewise;
//   3. clamp the counters to max_tokens (the number of rows written).
// The order of the rows inside an expert follows the atomics, so it is not
// fixed from run to run; the set of rows, their contents and the counts are.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hq_internal.hpp"

namespace hq {
namespace {

constexpr int kThreads = 256;     // 4 waves = 4 tokens per block

__global__ __launch_bounds__(kThreads) void permute_clear(int32_t* counts, int32_t E) {
  for (int e = blockIdx.x * kThreads + threadIdx.x; e < E; e += gridDim.x * kThreads) counts[e] = 0;
}

__global__ __launch_bounds__(kThreads) void permute_clamp(int32_t* counts, int32_t E, int32_t max_tokens) {
  for (int e = blockIdx.x * kThreads + threadIdx.x; e < E; e += gridDim.x * kThreads) {
    const int32_t c = counts[e];
    counts[e] = c < max_tokens ? c : max_tokens;
  }
}

// PermuteArgs: see launch_permute.
struct PermuteArgs {
  const uint8_t* x;
  const void* scale;
  const int64_t* ids;
  uint8_t* out_x;
  uint8_t* out_scale;
  int32_t* map;
  int32_t* counts;
  int64_t tokens, row_bytes, hidden, max_tokens;
  int32_t topk, experts, scale_mode;
};

__global__ __launch_bounds__(kThreads) void permute_scatter(PermuteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= a.tokens) return;                       // whole waves leave together

  // lane j < topk: claim a row for slot j
  int32_t row = -1, expert = -1;
  if (lane < a.topk) {
    const int64_t id = a.ids[t * a.topk + lane];
    if (id >= 0 && id < a.experts) {
      const int32_t r = atomicAdd(a.counts + id, 1);
      if (r < a.max_tokens) {
        row = r;
        expert = (int32_t)id;
      }
    }
    a.map[t * a.topk + lane] = row;
  }

  // the token's row, 16 bytes per lane per pass, to every claimed row
  const int64_t chunks = a.row_bytes / 16;
  const uint4* src = reinterpret_cast<const uint4*>(a.x + t * a.row_bytes);
  for (int64_t c = lane; c < chunks; c += 64) {
    const uint4 v = src[c];
    for (int j = 0; j < a.topk; ++j) {
      const int32_t r = __shfl(row, j, 64);
      const int32_t e = __shfl(expert, j, 64);
      if (r >= 0) {
        uint4* dst = reinterpret_cast<uint4*>(a.out_x + ((int64_t)e * a.max_tokens + r) * a.row_bytes);
        dst[c] = v;
      }
    }
  }

  // scales: hidden / 32 output bytes per row, written as dwords.  Broadcast:
  // source byte g128 (little-endian within int32 words) -> output dword g128
  // (its four 32-groups); direct: source dword d -> output dword d.
  const int64_t dwords = a.hidden / 128;           // output dwords per row
  const uint32_t* ssrc = reinterpret_cast<const uint32_t*>(a.scale);
  for (int64_t d = lane; d < dwords; d += 64) {
    uint32_t v;
    if (a.scale_mode == 0) {
      const uint32_t word = ssrc[t * (a.hidden / 512) + d / 4];
      v = ((word >> (8 * (d % 4))) & 0xFFu) * 0x01010101u;
    } else {
      v = ssrc[t * dwords + d];
    }
    for (int j = 0; j < a.topk; ++j) {
      const int32_t r = __shfl(row, j, 64);
      const int32_t e = __shfl(expert, j, 64);
      if (r >= 0)
        reinterpret_cast<uint32_t*>(a.out_scale + ((int64_t)e * a.max_tokens + r) * (a.hidden / 32))[d] = v;
    }
  }
}

}  // namespace

hipError_t launch_permute(hipStream_t s, const uint8_t* x, int64_t tokens, int64_t row_bytes,
                          int64_t hidden, const void* scale, int32_t scale_mode, const int64_t* ids,
                          int32_t topk, int32_t experts, int64_t max_tokens, uint8_t* out_x,
                          uint8_t* out_scale, int32_t* map, int32_t* counts) {
  const int eblocks = (experts + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(permute_clear, dim3(eblocks), dim3(kThreads), 0, s, counts, experts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (tokens > 0) {
    PermuteArgs a{x, scale, ids, out_x, out_scale, map, counts, tokens, row_bytes, hidden, max_tokens,
                  topk, experts, scale_mode};
    const int64_t blocks = (tokens + kThreads / 64 - 1) / (kThreads / 64);
    hipLaunchKernelGGL(permute_scatter, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(permute_clamp, dim3(eblocks), dim3(kThreads), 0, s, counts, experts,
                     (int32_t)max_tokens);
  return hipGetLastError();
}

}  // namespace hq
