// GEMM dispatch by mode, form and shape (the M-tiered dispatch of the
// flashrt/fp4-gemm page, re-chosen for gfx950):
//   * more than 16 rows per group and K a multiple of the K step (128 for
//     MXFP8, 256 for MXFP4 and NVFP4) of at least two steps: the LDS-tiled
//     persistent kernel;
//   * skinny M (<= 16 rows per group) and any other K: the direct kernel.
#include "gemm_common.hpp"

namespace hq {

hipError_t launch_gemm_direct(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev);
hipError_t launch_gemm_tiled(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev);
bool tiled_supported(const GemmArgs& p);

namespace {
bool use_tiled(const GemmArgs& p) {
  const int64_t rows_hint = p.form == kContiguous ? p.m_rows : p.slot_rows;
  return rows_hint > 16 && tiled_supported(p);
}
}  // namespace

hipError_t launch_gemm(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  if (use_tiled(p)) return launch_gemm_tiled(s, p, dev);
  return launch_gemm_direct(s, p, dev);
}

uint64_t gemm_workspace_bytes(const GemmArgs& p, const DeviceInfo& dev, bool* stream_k) {
  if (stream_k != nullptr) *stream_k = false;
  if (!use_tiled(p)) return 0;
  const SplitPlan sp = plan_split(p, dev);
  if (stream_k != nullptr) *stream_k = sp.kind == kSplitStream;
  return sp.kind == kSplitNone ? 0 : sp.bytes;
}

}  // namespace hq
