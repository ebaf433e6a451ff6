// Internal interfaces between the C-ABI layer (hq_api.cpp) and the kernel
// translation units.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

enum Mode : int32_t { kMXFP8 = 0, kMXFP4 = 1, kNVFP4 = 2 };

// How the rows of a grouped problem are described.
enum GroupForm : int32_t {
  kUniform = 0,    // group g owns rows [g*slot_rows, (g+1)*slot_rows)    (dense, batch)
  kContiguous = 1, // group g owns rows [end[g-1], end[g]), ends clamped  (grouped-contiguous)
  kMasked = 2,     // group g owns rows g*slot_rows + [0, min(cnt[g], slot_rows))
};

// One launch of any GEMM form.  Pointers are device pointers; strides are in
// bytes (codes / scales) or elements (out, bias).
struct GemmArgs {
  const uint8_t* a;
  const uint8_t* sfa;
  const uint8_t* b;
  const uint8_t* sfb;
  const uint16_t* bias;   // [G, n] or nullptr (MXFP8 only)
  const float* alpha;     // [G] or nullptr (NVFP4 only)
  uint16_t* out;
  const int32_t* group_end;  // kContiguous
  const int32_t* counts;     // kMasked
  int64_t m_rows;       // rows of a / out (all groups)
  int64_t slot_rows;    // kUniform / kMasked: rows per group slot
  int64_t n;
  int64_t k;            // logical K (elements)
  int64_t lda;          // bytes per row of a and b (K for FP8, K/2 for FP4)
  int64_t ldsf;         // scale bytes per row (K/32 or K/16)
  int64_t b_stride;     // bytes between consecutive groups' weights (n * lda)
  int64_t sfb_stride;   // n * ldsf
  int32_t num_groups;
  int32_t form;
  int32_t mode;
  int32_t cu_limit;
  // K split (tiled kernel, uniform form only): ksplit > 1 slices the K steps
  // of every tile into ksplit contiguous ranges; each range's FP32 partial
  // tile goes to partial[slice][row][col] and a second kernel sums the slices
  // in order and writes the BF16 output.  Set by the tiled launcher.
  int32_t ksplit;
  float* partial;
  int64_t ldo;          // output row stride in elements (0: n); the K-split reduce only
  int32_t tile_limit;   // tiled kernel: process only the first tile_limit tiles (0: all)
  // h > 0: gate|up GEMM whose epilogue applies SwiGLU and the MXFP8 re-quant
  // (tiled kernel, grouped-contiguous form): the weights hold n = 2h rows
  // [gate | up]; y = up * silu(gate) of the first valid[g] rows of each group
  // goes to q_out [m_rows, h] / sf_out [m_rows, h/32] (and y_debug
  // [m_rows, h] FP32 when given); out is not written.
  int64_t h;
  uint8_t* q_out;
  uint8_t* sf_out;
  float* y_debug;
  const int32_t* valid;
  // Discrete expert weights (grouped forms): b_ptrs[g] / sfb_ptrs[g] are the
  // device addresses of group g's [n, K'] codes and [n, k/gs] scales; b / sfb
  // and the strides are then unused.  nullptr: one [groups, n, K'] tensor.
  const uint64_t* b_ptrs;
  const uint64_t* sfb_ptrs;
  int32_t out_f16;      // out holds IEEE binary16 instead of BF16 (round to nearest even)
  // Caller-owned FP32 workspace of a K-split dense / batch call (nullptr: the
  // call runs unsplit).  The launcher splits only when workspace_bytes holds
  // the plan's bytes (plan_split).
  void* workspace;
  uint64_t workspace_bytes;
  // Backward GEMM with the dSwiGLU epilogue (kContiguous, tiled kernel): R =
  // alpha[g]^2 A B^T combined with the forward activations c_in [m_rows, 2n]
  // BF16 (32-column input / gate blocks), scaled by beta[g], and prob
  // [m_rows]; writes d_out [m_rows, 2n] BF16 and adds row sums to dprob.
  const uint16_t* c_in;
  const float* beta;
  const float* prob;
  float* dprob;
  uint16_t* d_out;
  // Stream-K form of a dense call (tiled kernel, set by the launcher): the
  // K steps of all tiles form sk_upt units of sk_unit steps per tile, dealt
  // out in equal runs to the workgroups.  sk_flags: one 64-bit flag per
  // workgroup at the start of the workspace; sk_tag: this call's flag value.
  int32_t sk_upt;
  int32_t sk_unit;
  uint32_t sk_tag;
  uint64_t* sk_flags;
};

// Bytes at the start of a split workspace that hold the stream-K flags (one
// 64-bit word per workgroup, the last one the spin-timeout word); the FP32
// partial tiles of every split form follow them.
constexpr uint64_t kWsHeader = 16384;
constexpr int kSkMaxGrid = 1023;

// How a dense or batch call on the tiled kernel splits K (plan_split).
enum SplitKind : int32_t {
  kSplitNone = 0,
  kSplitAll = 1,    // every tile's K steps in S slices
  kSplitTail = 2,   // the last round's tiles (a rectangle at r0, c0) in S slices
  kSplitStream = 3, // stream-K: equal runs of every tile's K units per workgroup
};
struct SplitPlan {
  int32_t kind;
  int64_t S;
  uint64_t bytes;        // FP32 workspace the split needs
  int64_t r0, c0;        // kSplitTail: the rectangle's first row and column
  int64_t rect_tiles;    // kSplitTail: its tiles
  int64_t grid;          // kSplitStream: workgroups
  int32_t upt, unit;     // kSplitStream: K units per tile, K steps per unit
};

struct DeviceInfo {
  int device;
  int num_cus;
  int max_smem;  // bytes of LDS per workgroup
};

// Returns hipSuccess or the error of the launch.
// x: BF16 bit patterns, or IEEE binary16 ones when fp16.
hipError_t launch_quant(hipStream_t s, int mode, const uint16_t* x, int64_t m, int64_t k,
                        uint8_t* q, uint8_t* sf, float* gs, bool gs_input, bool fp16);
hipError_t launch_swiglu_quant(hipStream_t s, int mode, const uint16_t* x, int64_t rows,
                               int64_t h, int32_t num_groups, const int32_t* group_end,
                               int64_t slot_rows, const int32_t* valid, uint8_t* q,
                               uint8_t* sf, const float* gs, float* y_debug);
hipError_t launch_gemm(hipStream_t s, const GemmArgs& args, const DeviceInfo& dev);
// The split plan of a tiled dense / batch launch, and the workspace bytes a
// call of this shape uses (0 when it never splits: other forms, the direct
// kernel).
SplitPlan plan_split(const GemmArgs& args, const DeviceInfo& dev);
// *stream_k (optional): whether that plan is the stream-K one.
uint64_t gemm_workspace_bytes(const GemmArgs& args, const DeviceInfo& dev, bool* stream_k = nullptr);
// The gate|up GEMM with the SwiGLU + re-quant epilogue (args.h > 0); false
// when the tiled kernel cannot take the shape (K, alignment).
bool gemm_swiglu_supported(const GemmArgs& args);
// The backward grouped GEMM with the dSwiGLU epilogue (args.c_in / d_out);
// false when the tiled kernel cannot take the shape.
bool gemm_dswiglu_supported(const GemmArgs& args);
hipError_t launch_gemm_dswiglu(hipStream_t s, const GemmArgs& args, const DeviceInfo& dev);
hipError_t launch_gemm_swiglu(hipStream_t s, const GemmArgs& args, const DeviceInfo& dev);
hipError_t launch_permute(hipStream_t s, const uint8_t* x, int64_t tokens, int64_t row_bytes,
                          int64_t hidden, const void* scale, int32_t scale_mode, const int64_t* ids,
                          int32_t topk, int32_t experts, int64_t max_tokens, uint8_t* out_x,
                          uint8_t* out_scale, int32_t* map, int32_t* counts, int num_cus);

}  // namespace hq
