// Token permute into the masked-GEMM layout (HALOps "GEMM" page,
// prefill_permute_to_masked_gemm section): each (token, slot) pair of the
// top-k routing with expert id e in [0, E) sends the token's row to the next
// free row of expert e's slot [e * max_tokens, (e + 1) * max_tokens), writes
// that expert-local row to the map, and re-lays the token's scale factors
// out at one byte per 32 elements.
//
// Three launches on the stream:
//   1. clear the E counters (a fill kernel, safe to capture in a graph);
//   2. a block per run of up to 64 tokens (fewer when there are few tokens,
//      so that there are about two blocks per CU): its pairs take block-local ranks per expert
//      with LDS atomics, the block reserves each expert's run of rows with
//      one global atomic add per expert it touches, and every pair's row is
//      base + local rank (rows past max_tokens are dropped: map -1); then
//      each wave copies whole tokens, reading a row once, 16 bytes per lane,
//      and storing it to every row its pairs claimed; the scale row likewise;
//   3. clamp the counters to max_tokens (the number of rows written).
// The order of the rows inside an expert follows the atomics, so it is not
// fixed from run to run; the set of rows, their contents and the counts are.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hq_internal.hpp"

namespace hq {
namespace {

constexpr int kThreads = 256;     // 4 waves

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
  int32_t tpb;                    // tokens per block, at most kMaxTokens
};

constexpr int kMaxTokens = 64;

// Dynamic LDS: one int per expert (the block's pair count, then the first
// row of its run), then per pair of the block its expert and its row
// (2 * tpb * topk ints; at most 36 KB).
__global__ __launch_bounds__(kThreads) void permute_scatter(PermuteArgs a) {
  extern __shared__ int32_t sh[];
  int32_t* cnt = sh;                               // [E]: pairs per expert, then base row
  int32_t* pex = sh + a.experts;                   // [pairs]: expert or -1
  int32_t* prow = pex + a.tpb * a.topk;            // [pairs]: local rank, then row or -1
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * a.tpb;
  const int ntok = a.tokens - t0 < a.tpb ? (int)(a.tokens - t0) : a.tpb;
  const int npairs = ntok * a.topk;

  for (int e = tid; e < a.experts; e += kThreads) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < npairs; i += kThreads) {
    const int64_t id = a.ids[t0 * a.topk + i];
    const bool ok = id >= 0 && id < a.experts;
    pex[i] = ok ? (int32_t)id : -1;
    prow[i] = ok ? atomicAdd(cnt + id, 1) : -1;    // block-local rank
  }
  __syncthreads();
  for (int e = tid; e < a.experts; e += kThreads) {
    const int32_t c = cnt[e];
    cnt[e] = c > 0 ? atomicAdd(a.counts + e, c) : 0;   // first row of the block's run
  }
  __syncthreads();
  for (int i = tid; i < npairs; i += kThreads) {
    const int32_t e = pex[i];
    int32_t r = -1;
    if (e >= 0) {
      r = cnt[e] + prow[i];
      if (r >= a.max_tokens) r = -1;              // the slot is full: dropped
    }
    prow[i] = r;
    a.map[t0 * a.topk + i] = r;
  }
  __syncthreads();

  // copies: wave w takes the block's tokens w, w + 4, ...
  const int64_t chunks = a.row_bytes / 16;
  const int64_t dwords = a.hidden / 128;           // output scale dwords per row
  const uint32_t* ssrc = reinterpret_cast<const uint32_t*>(a.scale);
  for (int tl = w; tl < ntok; tl += kThreads / 64) {
    const int64_t t = t0 + tl;
    const int32_t* rows = prow + tl * a.topk;
    const int32_t* exps = pex + tl * a.topk;
    const uint4* src = reinterpret_cast<const uint4*>(a.x + t * a.row_bytes);
    // the row is read once and each copy written once: both with the
    // non-temporal policy (16384 BF16 tokens of 2048, top-8: 8 % faster)
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u* vsrc = reinterpret_cast<const v4u*>(src);
    for (int64_t c = lane; c < chunks; c += 64) {
      const v4u v = __builtin_nontemporal_load(vsrc + c);
      for (int j = 0; j < a.topk; ++j) {
        const int32_t r = rows[j];
        if (r >= 0)
          __builtin_nontemporal_store(
              v, reinterpret_cast<v4u*>(a.out_x + ((int64_t)exps[j] * a.max_tokens + r) * a.row_bytes) + c);
      }
    }
    // broadcast: source byte g128 (little-endian in int32 words) -> output
    // dword g128, its four 32-groups; direct: source dword -> output dword
    for (int64_t d = lane; d < dwords; d += 64) {
      uint32_t v;
      if (a.scale_mode == 0) {
        const uint32_t word = ssrc[t * (a.hidden / 512) + d / 4];
        v = ((word >> (8 * (d % 4))) & 0xFFu) * 0x01010101u;
      } else {
        v = ssrc[t * dwords + d];
      }
      for (int j = 0; j < a.topk; ++j) {
        const int32_t r = rows[j];
        if (r >= 0)
          reinterpret_cast<uint32_t*>(a.out_scale + ((int64_t)exps[j] * a.max_tokens + r) * (a.hidden / 32))[d] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_permute(hipStream_t s, const uint8_t* x, int64_t tokens, int64_t row_bytes,
                          int64_t hidden, const void* scale, int32_t scale_mode, const int64_t* ids,
                          int32_t topk, int32_t experts, int64_t max_tokens, uint8_t* out_x,
                          uint8_t* out_scale, int32_t* map, int32_t* counts, int num_cus) {
  const int eblocks = (experts + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(permute_clear, dim3(eblocks), dim3(kThreads), 0, s, counts, experts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (tokens > 0) {
    int64_t tpb = tokens / (2 * (int64_t)(num_cus > 0 ? num_cus : 256));
    tpb = tpb < 4 ? 4 : (tpb > kMaxTokens ? kMaxTokens : tpb);
    PermuteArgs a{x, scale, ids, out_x, out_scale, map, counts, tokens, row_bytes, hidden, max_tokens,
                  topk, experts, scale_mode, (int32_t)tpb};
    const int64_t blocks = (tokens + tpb - 1) / tpb;
    const size_t lds = sizeof(int32_t) * ((size_t)experts + 2 * (size_t)tpb * topk);
    hipLaunchKernelGGL(permute_scatter, dim3((unsigned)blocks), dim3(kThreads), lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(permute_clamp, dim3(eblocks), dim3(kThreads), 0, s, counts, experts,
                     (int32_t)max_tokens);
  return hipGetLastError();
}

}  // namespace hq
