// Group/row bookkeeping shared by the grouped GEMM and the fused SwiGLU
// kernels: a block-wide inclusive scan over at most 1024 per-group values,
// and the clamped interpretation of device-side group ends / counts.
//
// Grouped-contiguous rows follow HALOps "GEMM" page, group_contiguous_gemm
// section, with cumulative ends as in cuDNN FE "Grouped GEMM + dGLU (SM100)"
// Step 1; grouped-masked slots follow the group_masked_gemm section.  Device
// values cannot be validated by the host, so ends are clamped to
// [previous end, rows] and counts to [0, slot_rows].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

constexpr int kMaxGroups = 1024;

struct OpAdd {
  __device__ int operator()(int a, int b) const { return a + b; }
};
struct OpMax {
  __device__ int operator()(int a, int b) const { return a > b ? a : b; }
};

// In-place inclusive scan of s[0, n) (n <= 1024) by the first NT threads of
// the block (NT a multiple of 64, at most 1024); threads past NT only meet
// the barriers.  Each scanning thread takes 1024 / NT consecutive entries,
// waves scan their thread totals with lane shuffles, and the wave totals are
// combined through LDS.  `op` must be associative with `identity` neutral.
// Returns the scan's last value to every thread.  Must be reached by all
// threads.
template <int NT, class Op>
__device__ int block_scan_1024(int* s, int n, Op op, int identity) {
  static_assert(NT % 64 == 0 && NT >= 64 && NT <= 1024, "block of whole waves, at most 1024 threads");
  constexpr int PER = 1024 / NT, NW = NT / 64;
  __shared__ int wsum[NW];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = t * PER + i;
    v[i] = idx < n ? s[idx] : identity;
    if (i > 0) v[i] = op(v[i - 1], v[i]);
  }
  int x = v[PER - 1];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x = op(x, y);
  }
  if (lane == 63 && w < NW) wsum[w] = x;     // threads past NT hold no entries
  __syncthreads();
  int prefix = identity, total = identity;
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    if (j < w) prefix = op(prefix, wsum[j]);
    total = op(total, wsum[j]);
  }
  int excl = __shfl_up(x, 1, 64);
  if (lane == 0) excl = identity;
  excl = op(prefix, excl);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = t * PER + i;
    if (idx < n) s[idx] = op(excl, v[i]);
  }
  __syncthreads();
  return total;
}

// Loads group ends into s[0, G) as clamped, non-decreasing ends:
// e'_g = min(max(e_0 .. e_g, 0), rows).
template <int NT>
__device__ inline void load_clamped_ends(int* s, const int32_t* group_end, int G, int64_t rows) {
  for (int i = threadIdx.x; i < G; i += blockDim.x) {
    int e = group_end[i];
    s[i] = e > 0 ? e : 0;
  }
  __syncthreads();
  block_scan_1024<NT>(s, G, OpMax(), 0);
  for (int i = threadIdx.x; i < G; i += blockDim.x) {
    int64_t e = s[i];
    s[i] = (int)(e < rows ? e : rows);
  }
  __syncthreads();
}

// First group whose clamped end exceeds row r (G if none).
__device__ inline int find_group(const int* ends, int G, int r) {
  int lo = 0, hi = G;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (ends[mid] > r) hi = mid; else lo = mid + 1;
  }
  return lo;
}

}  // namespace hq
