// C-ABI layer: argument validation (host only, before any device work),
// device checks and dispatch to the kernel launchers.
//
// Error convention: flashrt/fp4-gemm page, Notes -- unsupported calls fail
// before launch and an output is never left silently undefined.  Every check
// here runs before the first HIP call, so a rejected call touches neither the
// device nor any output buffer.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "hq.h"
#include "hq_internal.hpp"

namespace {

thread_local char g_err[512] = "";

hq_status fail(hq_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

hq_status ok() {
  g_err[0] = '\0';
  return HQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kI32 = 2147483647LL;

const char* mode_name(int32_t mode) {
  return mode == HQ_MXFP8 ? "MXFP8" : mode == HQ_MXFP4 ? "MXFP4" : mode == HQ_NVFP4 ? "NVFP4" : "?";
}

// ---------------------------------------------------------------- device
struct DevCache {
  bool probed = false;
  bool ok = false;
  hq::DeviceInfo info{};
};
std::mutex g_dev_mu;
DevCache g_dev[64];

hq_status current_device(hq::DeviceInfo* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64)
    return fail(HQ_ERR_DEVICE, "no usable HIP device (%s)", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevCache& c = g_dev[dev];
  if (!c.probed) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(HQ_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    c.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    c.info.device = dev;
    c.info.num_cus = prop.multiProcessorCount;
    c.info.max_smem = (int)prop.sharedMemPerBlock;
    c.probed = true;
    if (!c.ok) {
      c.probed = true;
      return fail(HQ_ERR_DEVICE, "device %d is %s; this library is built for gfx950", dev,
                  prop.gcnArchName);
    }
  }
  if (!c.ok) return fail(HQ_ERR_DEVICE, "device %d is not gfx950", dev);
  *out = c.info;
  return HQ_OK;
}

hq_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(HQ_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------- scratch
// The K-split workspace of hq_dense_gemm_scratch: a fixed device array of
// HQ_SCRATCH_BYTES, one copy per GPU, held until the process ends.  In host
// code `scratch` only names the symbol: its device address on the current
// GPU comes from hipGetSymbolAddress, once per device, and only that address
// is handed to kernels.  Every call on a GPU shares its copy (calls that
// overlap on one GPU race); nothing in it has to start at zero, since a
// K-split launch writes every partial value before its reduce reads it.
static __device__ __align__(256) uint8_t scratch[HQ_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// The current device's scratch address (dev.device current); nullptr and a
// message when the symbol cannot be resolved.
void* scratch_address(const hq::DeviceInfo& dev) {
  if (dev.device < 0 || dev.device >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev.device] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      fail(HQ_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev.device, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev.device] = ptr;
  }
  return g_scratch_ptr[dev.device];
}

// ---------------------------------------------------------------- GEMM checks
struct GemmCheck {
  int32_t mode;
  const void *a, *sfa, *b, *sfb, *bias, *alpha, *out;
  int64_t rows, n, k;
  int64_t groups;
  const char* what;
};

// Shape and mode checks common to the GEMM forms.  Returns HQ_OK and sets
// *noop when there is nothing to compute.
hq_status check_gemm(const GemmCheck& c, bool* noop) {
  *noop = false;
  if (c.mode < HQ_MXFP8 || c.mode > HQ_NVFP4) return fail(HQ_ERR_MODE, "%s: unknown mode %d", c.what, c.mode);
  if (c.k <= 0 || c.k % 32 != 0) return fail(HQ_ERR_SHAPE, "%s: k=%lld must be a positive multiple of 32", c.what, (long long)c.k);
  if (c.n < 0 || c.n % 8 != 0) return fail(HQ_ERR_SHAPE, "%s: n=%lld must be a non-negative multiple of 8", c.what, (long long)c.n);
  if (c.rows < 0) return fail(HQ_ERR_SHAPE, "%s: negative row count", c.what);
  if (c.rows > kI32 || c.n > kI32 || c.k > kI32)
    return fail(HQ_ERR_SHAPE, "%s: dimensions must be below 2^31", c.what);
  // tile ids are 32-bit: (rows/16 + groups) * (n/16) must stay below 2^31
  if ((c.rows / 16 + c.groups + 1) * (c.n / 16 + 1) > kI32)
    return fail(HQ_ERR_SHAPE, "%s: problem too large (tile count exceeds 2^31)", c.what);
  if (c.bias != nullptr && c.mode != HQ_MXFP8)
    return fail(HQ_ERR_MODE, "%s: bias is only supported in MXFP8 mode (got %s)", c.what, mode_name(c.mode));
  if (c.mode == HQ_NVFP4 && c.alpha == nullptr && c.rows > 0 && c.n > 0)
    return fail(HQ_ERR_MODE, "%s: alpha is required in NVFP4 mode", c.what);
  if (c.mode != HQ_NVFP4 && c.alpha != nullptr)
    return fail(HQ_ERR_MODE, "%s: alpha is only accepted in NVFP4 mode (got %s)", c.what, mode_name(c.mode));
  if (c.rows == 0 || c.n == 0) {
    *noop = true;
    return HQ_OK;
  }
  if (!c.a || !c.sfa || !c.b || !c.sfb || !c.out) return fail(HQ_ERR_NULL, "%s: a, sfa, b, sfb and out are required", c.what);
  if (!aligned16(c.a) || !aligned16(c.b) || !aligned16(c.out))
    return fail(HQ_ERR_ALIGN, "%s: a, b and out must be 16-byte aligned", c.what);
  return HQ_OK;
}

hq::GemmArgs make_args(int32_t mode, const uint8_t* a, const uint8_t* sfa, const uint8_t* b,
                       const uint8_t* sfb, const uint16_t* bias, const float* alpha,
                       uint16_t* out, int64_t n, int64_t k, int32_t cu_limit) {
  hq::GemmArgs p{};
  p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.bias = bias; p.alpha = alpha; p.out = out;
  p.n = n; p.k = k;
  p.lda = mode == HQ_MXFP8 ? k : k / 2;
  p.ldsf = mode == HQ_NVFP4 ? k / 16 : k / 32;
  p.b_stride = n * p.lda;
  p.sfb_stride = n * p.ldsf;
  p.mode = mode;
  p.cu_limit = cu_limit;
  return p;
}

}  // namespace

extern "C" {

const char* hq_last_error(void) { return g_err; }

hq_status hq_group_wise_quant(void* stream, int32_t mode, const uint16_t* x, int64_t m, int64_t k,
                              uint8_t* q, uint8_t* sf, float* global_scale, uint32_t flags) {
  const char* what = "hq_group_wise_quant";
  if (mode < HQ_MXFP8 || mode > HQ_NVFP4) return fail(HQ_ERR_MODE, "%s: unknown mode %d", what, mode);
  if (k <= 0 || k % 32 != 0) return fail(HQ_ERR_SHAPE, "%s: k=%lld must be a positive multiple of 32", what, (long long)k);
  if (m < 0 || m > kI32 || k > kI32) return fail(HQ_ERR_SHAPE, "%s: m=%lld out of range", what, (long long)m);
  if (mode != HQ_NVFP4) {
    if (global_scale != nullptr) return fail(HQ_ERR_MODE, "%s: global_scale is NVFP4 only", what);
    if ((flags & ~HQ_IN_FP16) != 0) return fail(HQ_ERR_MODE, "%s: flags 0x%x: only HQ_IN_FP16 applies to MX modes", what, flags);
  } else {
    if ((flags & ~(HQ_GS_INPUT | HQ_IN_FP16)) != 0) return fail(HQ_ERR_MODE, "%s: unknown flags 0x%x", what, flags);
    if (global_scale == nullptr) return fail(HQ_ERR_NULL, "%s: NVFP4 needs global_scale", what);
  }
  if (m == 0) return ok();
  if (!x || !q || !sf) return fail(HQ_ERR_NULL, "%s: x, q and sf are required", what);
  if (!aligned16(x) || !aligned16(q)) return fail(HQ_ERR_ALIGN, "%s: x and q must be 16-byte aligned", what);
  hq::DeviceInfo dev;
  hq_status st = current_device(&dev);
  if (st != HQ_OK) return st;
  return launched(hq::launch_quant((hipStream_t)stream, mode, x, m, k, q, sf, global_scale,
                                   (flags & HQ_GS_INPUT) != 0, (flags & HQ_IN_FP16) != 0),
                  what);
}

// A caller workspace: null with 0 bytes (unsplit), else 16-byte aligned.
static hq_status check_workspace(const void* ws, uint64_t bytes, const char* what) {
  if (bytes > 0 && ws == nullptr) return fail(HQ_ERR_NULL, "%s: workspace is NULL but workspace_bytes > 0", what);
  if (ws != nullptr && !aligned16(ws)) return fail(HQ_ERR_ALIGN, "%s: workspace must be 16-byte aligned", what);
  return HQ_OK;
}

hq_status hq_dense_gemm_ws(void* stream, int32_t mode, const uint8_t* a, const uint8_t* sfa,
                           const uint8_t* b, const uint8_t* sfb, const uint16_t* bias,
                           const float* alpha, uint16_t* out, int64_t m, int64_t n, int64_t k,
                           int32_t cu_limit, void* workspace, uint64_t workspace_bytes) {
  const bool out_f16 = (mode & HQ_OUT_FP16) != 0;   // binary16 output
  mode &= ~(int32_t)HQ_OUT_FP16;
  GemmCheck c{mode, a, sfa, b, sfb, bias, alpha, out, m, n, k, 1, "hq_dense_gemm"};
  bool noop;
  hq_status st = check_gemm(c, &noop);
  if (st != HQ_OK) return st;
  if ((st = check_workspace(workspace, workspace_bytes, c.what)) != HQ_OK) return st;
  if (noop) return ok();
  hq::DeviceInfo dev;
  if ((st = current_device(&dev)) != HQ_OK) return st;
  hq::GemmArgs p = make_args(mode, a, sfa, b, sfb, bias, alpha, out, n, k, cu_limit);
  p.out_f16 = out_f16 ? 1 : 0;
  p.form = hq::kUniform;
  p.num_groups = 1;
  p.m_rows = m;
  p.slot_rows = m;
  p.workspace = workspace;
  p.workspace_bytes = workspace_bytes;
  return launched(hq::launch_gemm((hipStream_t)stream, p, dev), c.what);
}

hq_status hq_dense_gemm(void* stream, int32_t mode, const uint8_t* a, const uint8_t* sfa,
                        const uint8_t* b, const uint8_t* sfb, const uint16_t* bias,
                        const float* alpha, uint16_t* out, int64_t m, int64_t n, int64_t k,
                        int32_t cu_limit) {
  return hq_dense_gemm_ws(stream, mode, a, sfa, b, sfb, bias, alpha, out, m, n, k, cu_limit, nullptr, 0);
}

hq_status hq_dense_gemm_scratch(void* stream, int32_t mode, const uint8_t* a, const uint8_t* sfa,
                                const uint8_t* b, const uint8_t* sfb, const uint16_t* bias,
                                const float* alpha, uint16_t* out, int64_t m, int64_t n, int64_t k,
                                int32_t cu_limit) {
  const bool out_f16 = (mode & HQ_OUT_FP16) != 0;   // binary16 output
  mode &= ~(int32_t)HQ_OUT_FP16;
  GemmCheck c{mode, a, sfa, b, sfb, bias, alpha, out, m, n, k, 1, "hq_dense_gemm_scratch"};
  bool noop;
  hq_status st = check_gemm(c, &noop);
  if (st != HQ_OK) return st;
  if (noop) return ok();
  hq::DeviceInfo dev;
  if ((st = current_device(&dev)) != HQ_OK) return st;
  hq::GemmArgs p = make_args(mode, a, sfa, b, sfb, bias, alpha, out, n, k, cu_limit);
  p.out_f16 = out_f16 ? 1 : 0;
  p.form = hq::kUniform;
  p.num_groups = 1;
  p.m_rows = m;
  p.slot_rows = m;
  bool stream_k = false;
  uint64_t need = hq::gemm_workspace_bytes(p, dev, &stream_k);
  // a stream-K plan that does not fit the scratch is not taken: the call
  // runs unsplit, as hq_dense_gemm_ws does with a workspace of that size
  if (stream_k && need > (uint64_t)HQ_SCRATCH_BYTES) need = 0;
  if (need > (uint64_t)HQ_SCRATCH_BYTES)
    return fail(HQ_ERR_SHAPE, "%s: this shape's K split needs %llu bytes of workspace, more than the %llu "
                "of the library's scratch (use hq_dense_gemm_ws with a workspace of that size, or hq_dense_gemm)",
                c.what, (unsigned long long)need, (unsigned long long)HQ_SCRATCH_BYTES);
  if (need > 0) {
    void* ptr = scratch_address(dev);
    if (ptr == nullptr) return HQ_ERR_DEVICE;
    p.workspace = ptr;
    p.workspace_bytes = (uint64_t)HQ_SCRATCH_BYTES;
  }
  return launched(hq::launch_gemm((hipStream_t)stream, p, dev), c.what);
}

hq_status hq_batch_gemm_ws(void* stream, int32_t mode, const uint8_t* a, const uint8_t* sfa,
                           const uint8_t* b, const uint8_t* sfb, const uint16_t* bias,
                           const float* alpha, uint16_t* out, int64_t batch, int64_t m, int64_t n,
                           int64_t k, int32_t cu_limit, void* workspace, uint64_t workspace_bytes) {
  const bool out_f16 = (mode & HQ_OUT_FP16) != 0;   // binary16 output
  mode &= ~(int32_t)HQ_OUT_FP16;
  const char* what = "hq_batch_gemm";
  if (batch < 0 || batch > kI32) return fail(HQ_ERR_SHAPE, "%s: batch=%lld out of range", what, (long long)batch);
  if (m < 0 || (batch > 0 && m > kI32 / (batch > 0 ? batch : 1)))
    return fail(HQ_ERR_SHAPE, "%s: batch * m must be below 2^31", what);
  GemmCheck c{mode, a, sfa, b, sfb, bias, alpha, out, batch * m, n, k, batch, what};
  bool noop;
  hq_status st = check_gemm(c, &noop);
  if (st != HQ_OK) return st;
  if ((st = check_workspace(workspace, workspace_bytes, what)) != HQ_OK) return st;
  if (noop) return ok();
  hq::DeviceInfo dev;
  if ((st = current_device(&dev)) != HQ_OK) return st;
  hq::GemmArgs p = make_args(mode, a, sfa, b, sfb, bias, alpha, out, n, k, cu_limit);
  p.out_f16 = out_f16 ? 1 : 0;
  p.form = hq::kUniform;
  p.num_groups = (int32_t)batch;
  p.m_rows = batch * m;
  p.slot_rows = m;
  p.workspace = workspace;
  p.workspace_bytes = workspace_bytes;
  return launched(hq::launch_gemm((hipStream_t)stream, p, dev), what);
}

hq_status hq_batch_gemm(void* stream, int32_t mode, const uint8_t* a, const uint8_t* sfa,
                        const uint8_t* b, const uint8_t* sfb, const uint16_t* bias,
                        const float* alpha, uint16_t* out, int64_t batch, int64_t m, int64_t n,
                        int64_t k, int32_t cu_limit) {
  return hq_batch_gemm_ws(stream, mode, a, sfa, b, sfb, bias, alpha, out, batch, m, n, k, cu_limit,
                          nullptr, 0);
}

hq_status hq_gemm_workspace_size(int32_t mode, int64_t batch, int64_t m, int64_t n, int64_t k,
                                 int32_t cu_limit, uint64_t* bytes) {
  const char* what = "hq_gemm_workspace_size";
  if (!bytes) return fail(HQ_ERR_NULL, "%s: bytes is required", what);
  *bytes = 0;
  mode &= ~(int32_t)HQ_OUT_FP16;
  if (batch < 1 || batch > kI32) return fail(HQ_ERR_SHAPE, "%s: batch=%lld must be in [1, 2^31)", what, (long long)batch);
  if (m < 0 || m > kI32 / batch) return fail(HQ_ERR_SHAPE, "%s: batch * m must be below 2^31", what);
  // shape and mode checks of the GEMM calls (no pointers: bias / alpha as the mode wants)
  static const uint8_t kAny[16] = {};
  const float* alpha = mode == HQ_NVFP4 ? reinterpret_cast<const float*>(kAny) : nullptr;
  GemmCheck c{mode, kAny, kAny, kAny, kAny, nullptr, alpha, kAny, batch * m, n, k, batch, what};
  bool noop;
  hq_status st = check_gemm(c, &noop);
  if (st != HQ_OK) return st;
  if (noop) return ok();
  hq::DeviceInfo dev;
  if ((st = current_device(&dev)) != HQ_OK) return st;
  hq::GemmArgs p = make_args(mode, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, n, k, cu_limit);
  p.form = hq::kUniform;
  p.num_groups = (int32_t)batch;
  p.m_rows = batch * m;
  p.slot_rows = m;
  *bytes = hq::gemm_workspace_bytes(p, dev);
  return ok();
}

hq_status hq_group_contiguous_gemm(void* stream, int32_t mode, const uint8_t* a,
                                   const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                                   const int32_t* group_end, int32_t num_groups,
                                   const uint16_t* bias, const float* alpha, uint16_t* out,
                                   int64_t m_total, int64_t n, int64_t k, int32_t cu_limit) {
  const bool out_f16 = (mode & HQ_OUT_FP16) != 0;   // binary16 output
  mode &= ~(int32_t)HQ_OUT_FP16;
  const char* what = "hq_group_contiguous_gemm";
  if (num_groups < 1 || num_groups > 1024)
    return fail(HQ_ERR_SHAPE, "%s: num_groups=%d must be in [1, 1024]", what, num_groups);
  GemmCheck c{mode, a, sfa, b, sfb, bias, alpha, out, m_total, n, k, num_groups, what};
  bool noop;
  hq_status st = check_gemm(c, &noop);
  if (st != HQ_OK) return st;
  if (noop) return ok();
  if (!group_end) return fail(HQ_ERR_NULL, "%s: group_end is required", what);
  hq::DeviceInfo dev;
  if ((st = current_device(&dev)) != HQ_OK) return st;
  hq::GemmArgs p = make_args(mode, a, sfa, b, sfb, bias, alpha, out, n, k, cu_limit);
  p.out_f16 = out_f16 ? 1 : 0;
  p.form = hq::kContiguous;
  p.group_end = group_end;
  p.num_groups = num_groups;
  p.m_rows = m_total;
  p.slot_rows = 0;
  return launched(hq::launch_gemm((hipStream_t)stream, p, dev), what);
}

hq_status hq_group_contiguous_gemm_ptr_array(void* stream, int32_t mode, const uint8_t* a,
                                             const uint8_t* sfa, const uint64_t* b_ptrs,
                                             const uint64_t* sfb_ptrs, const int32_t* group_end,
                                             int32_t num_groups, const uint16_t* bias,
                                             const float* alpha, uint16_t* out, int64_t m_total,
                                             int64_t n, int64_t k, int32_t cu_limit) {
  const bool out_f16 = (mode & HQ_OUT_FP16) != 0;   // binary16 output
  mode &= ~(int32_t)HQ_OUT_FP16;
  const char* what = "hq_group_contiguous_gemm_ptr_array";
  if (num_groups < 1 || num_groups > 1024)
    return fail(HQ_ERR_SHAPE, "%s: num_groups=%d must be in [1, 1024]", what, num_groups);
  // b / sfb stand in for the pointer arrays in the common checks (their
  // elements' alignment is the caller's contract: the arrays are device data)
  GemmCheck c{mode, a, sfa, b_ptrs, sfb_ptrs, bias, alpha, out, m_total, n, k, num_groups, what};
  bool noop;
  hq_status st = check_gemm(c, &noop);
  if (st != HQ_OK) return st;
  if (noop) return ok();
  if (!group_end) return fail(HQ_ERR_NULL, "%s: group_end is required", what);
  hq::DeviceInfo dev;
  if ((st = current_device(&dev)) != HQ_OK) return st;
  hq::GemmArgs p = make_args(mode, a, sfa, nullptr, nullptr, bias, alpha, out, n, k, cu_limit);
  p.out_f16 = out_f16 ? 1 : 0;
  p.form = hq::kContiguous;
  p.group_end = group_end;
  p.num_groups = num_groups;
  p.m_rows = m_total;
  p.slot_rows = 0;
  p.b_ptrs = b_ptrs;
  p.sfb_ptrs = sfb_ptrs;
  return launched(hq::launch_gemm((hipStream_t)stream, p, dev), what);
}

hq_status hq_group_contiguous_gemm_swiglu_quant(void* stream, int32_t mode, const uint8_t* a,
                                                const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                                                const int32_t* group_end, int32_t num_groups,
                                                const int32_t* valid, const uint16_t* bias, uint8_t* q,
                                                uint8_t* sf, float* y_debug, int64_t m_total, int64_t h,
                                                int64_t k, int32_t cu_limit) {
  const char* what = "hq_group_contiguous_gemm_swiglu_quant";
  if (mode != HQ_MXFP8) return fail(HQ_ERR_MODE, "%s: only MXFP8 is supported (got %d)", what, mode);
  if (num_groups < 1 || num_groups > 1024)
    return fail(HQ_ERR_SHAPE, "%s: num_groups=%d must be in [1, 1024]", what, num_groups);
  if (h <= 0 || h % 128 != 0 || h > (1 << 20))
    return fail(HQ_ERR_SHAPE, "%s: h=%lld must be a positive multiple of 128, at most 2^20", what, (long long)h);
  GemmCheck c{mode, a, sfa, b, sfb, bias, nullptr, q, m_total, 2 * h, k, num_groups, what};
  bool noop;
  hq_status st = check_gemm(c, &noop);
  if (st != HQ_OK) return st;
  // a tile's up rows lie h + 127 rows past its first gate row: their byte
  // offsets from the tile's base must stay 32-bit
  if ((h + 256) * k >= ((int64_t)1 << 31))
    return fail(HQ_ERR_SHAPE, "%s: (h + 256) * k = %lld must be below 2^31", what, (long long)((h + 256) * k));
  if (noop) return ok();
  if (!group_end || !sf) return fail(HQ_ERR_NULL, "%s: group_end and sf are required", what);
  if (y_debug && !aligned16(y_debug)) return fail(HQ_ERR_ALIGN, "%s: y_debug must be 16-byte aligned", what);
  hq::GemmArgs p = make_args(mode, a, sfa, b, sfb, bias, nullptr, nullptr, 2 * h, k, cu_limit);
  p.form = hq::kContiguous;
  p.group_end = group_end;
  p.num_groups = num_groups;
  p.m_rows = m_total;
  p.slot_rows = 0;
  p.h = h;
  p.q_out = q;
  p.sf_out = sf;
  p.y_debug = y_debug;
  p.valid = valid;
  if (!hq::gemm_swiglu_supported(p)) {
    if ((reinterpret_cast<uintptr_t>(sfa) | reinterpret_cast<uintptr_t>(sfb)) & 3)
      return fail(HQ_ERR_ALIGN, "%s: sfa and sfb must be 4-byte aligned", what);
    return fail(HQ_ERR_SHAPE, "%s: k=%lld must be a multiple of 128 of at least 256", what, (long long)k);
  }
  hq::DeviceInfo dev;
  if ((st = current_device(&dev)) != HQ_OK) return st;
  return launched(hq::launch_gemm_swiglu((hipStream_t)stream, p, dev), what);
}

// Shared by the BF16 and the row-quantised dSwiGLU calls (exactly one of d
// and dq is set).
static hq_status dswiglu_call(const char* what, void* stream, int32_t mode, const uint8_t* a, const uint8_t* sfa,
                       const uint8_t* b, const uint8_t* sfb, const int32_t* group_end, int32_t num_groups,
                       const uint16_t* c, const float* alpha, const float* beta, const float* prob, float* dprob,
                       uint16_t* d, uint8_t* dq, uint8_t* dsf, int64_t m_total, int64_t n, int64_t k,
                       int32_t cu_limit) {
  if (mode != HQ_MXFP8 && mode != HQ_MXFP4)
    return fail(HQ_ERR_MODE, "%s: MXFP8 or MXFP4 codes only (got %d)", what, mode);
  if (num_groups < 1 || num_groups > 1024)
    return fail(HQ_ERR_SHAPE, "%s: num_groups=%d must be in [1, 1024]", what, num_groups);
  if (n % 32 != 0) return fail(HQ_ERR_SHAPE, "%s: n=%lld must be a multiple of 32", what, (long long)n);
  if (n > 0 && n * 1024 >= ((int64_t)1 << 31))
    return fail(HQ_ERR_SHAPE, "%s: n=%lld too large (n * 1024 must be below 2^31)", what, (long long)n);
  // alpha here is the per-group GEMM scale (entering squared), not the NVFP4
  // alpha; the output check takes whichever output the call has
  const void* out = dq != nullptr ? static_cast<const void*>(dq) : static_cast<const void*>(d);
  GemmCheck cc{mode, a, sfa, b, sfb, nullptr, nullptr, static_cast<const uint16_t*>(out), m_total, n, k,
               num_groups, what};
  bool noop;
  hq_status st = check_gemm(cc, &noop);
  if (st != HQ_OK) return st;
  if (noop) return ok();
  if (!group_end || !c || !prob || !dprob) return fail(HQ_ERR_NULL, "%s: group_end, c, prob and dprob are required", what);
  if (dq != nullptr && dsf == nullptr) return fail(HQ_ERR_NULL, "%s: dsf is required", what);
  if (!aligned16(c)) return fail(HQ_ERR_ALIGN, "%s: c must be 16-byte aligned", what);
  if ((reinterpret_cast<uintptr_t>(prob) | reinterpret_cast<uintptr_t>(dprob)) & 3u)
    return fail(HQ_ERR_ALIGN, "%s: prob and dprob must be 4-byte aligned", what);
  hq::GemmArgs p = make_args(mode, a, sfa, b, sfb, nullptr, alpha, nullptr, n, k, cu_limit);
  p.form = hq::kContiguous;
  p.group_end = group_end;
  p.num_groups = num_groups;
  p.m_rows = m_total;
  p.slot_rows = 0;
  p.c_in = c;
  p.beta = beta;
  p.prob = prob;
  p.dprob = dprob;
  p.d_out = d;
  p.q_out = dq;
  p.sf_out = dsf;
  if (!hq::gemm_dswiglu_supported(p)) {
    if ((reinterpret_cast<uintptr_t>(sfa) | reinterpret_cast<uintptr_t>(sfb)) & 3)
      return fail(HQ_ERR_ALIGN, "%s: sfa and sfb must be 4-byte aligned", what);
    return fail(HQ_ERR_SHAPE, "%s: k=%lld must be a multiple of the K step (128 MXFP8, 256 MXFP4) of at least "
                "two steps", what, (long long)k);
  }
  hq::DeviceInfo dev;
  if ((st = current_device(&dev)) != HQ_OK) return st;
  return launched(hq::launch_gemm_dswiglu((hipStream_t)stream, p, dev), what);
}

hq_status hq_group_contiguous_gemm_dswiglu(void* stream, int32_t mode, const uint8_t* a,
                                           const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                                           const int32_t* group_end, int32_t num_groups,
                                           const uint16_t* c, const float* alpha, const float* beta,
                                           const float* prob, float* dprob, uint16_t* d,
                                           int64_t m_total, int64_t n, int64_t k, int32_t cu_limit) {
  return dswiglu_call("hq_group_contiguous_gemm_dswiglu", stream, mode, a, sfa, b, sfb, group_end, num_groups, c,
                      alpha, beta, prob, dprob, d, nullptr, nullptr, m_total, n, k, cu_limit);
}

hq_status hq_group_contiguous_gemm_dswiglu_quant(void* stream, int32_t mode, const uint8_t* a,
                                                 const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                                                 const int32_t* group_end, int32_t num_groups,
                                                 const uint16_t* c, const float* alpha, const float* beta,
                                                 const float* prob, float* dprob, uint8_t* dq, uint8_t* dsf,
                                                 int64_t m_total, int64_t n, int64_t k, int32_t cu_limit) {
  const char* what = "hq_group_contiguous_gemm_dswiglu_quant";
  if (dq == nullptr && m_total > 0 && n > 0) return fail(HQ_ERR_NULL, "%s: dq is required", what);
  return dswiglu_call(what, stream, mode, a, sfa, b, sfb, group_end, num_groups, c, alpha, beta, prob, dprob,
                      nullptr, dq, dsf, m_total, n, k, cu_limit);
}

hq_status hq_group_masked_gemm(void* stream, int32_t mode, const uint8_t* a, const uint8_t* sfa,
                               const uint8_t* b, const uint8_t* sfb, const int32_t* masked_m,
                               int32_t num_groups, int64_t max_m_per_group, const uint16_t* bias,
                               const float* alpha, uint16_t* out, int64_t n, int64_t k,
                               int32_t cu_limit) {
  const bool out_f16 = (mode & HQ_OUT_FP16) != 0;   // binary16 output
  mode &= ~(int32_t)HQ_OUT_FP16;
  const char* what = "hq_group_masked_gemm";
  if (num_groups < 1 || num_groups > 1024)
    return fail(HQ_ERR_SHAPE, "%s: num_groups=%d must be in [1, 1024]", what, num_groups);
  if (max_m_per_group <= 0 || max_m_per_group > kI32 / num_groups)
    return fail(HQ_ERR_SHAPE, "%s: max_m_per_group=%lld must be > 0 and num_groups * max_m below 2^31",
                what, (long long)max_m_per_group);
  GemmCheck c{mode, a, sfa, b, sfb, bias, alpha, out, num_groups * max_m_per_group, n, k, num_groups, what};
  bool noop;
  hq_status st = check_gemm(c, &noop);
  if (st != HQ_OK) return st;
  if (noop) return ok();
  if (!masked_m) return fail(HQ_ERR_NULL, "%s: masked_m is required", what);
  hq::DeviceInfo dev;
  if ((st = current_device(&dev)) != HQ_OK) return st;
  hq::GemmArgs p = make_args(mode, a, sfa, b, sfb, bias, alpha, out, n, k, cu_limit);
  p.out_f16 = out_f16 ? 1 : 0;
  p.form = hq::kMasked;
  p.counts = masked_m;
  p.num_groups = num_groups;
  p.m_rows = num_groups * max_m_per_group;
  p.slot_rows = max_m_per_group;
  return launched(hq::launch_gemm((hipStream_t)stream, p, dev), what);
}

hq_status hq_fused_swiglu_quant(void* stream, int32_t mode, const uint16_t* x, int64_t rows,
                                int64_t h, int32_t num_groups, const int32_t* group_end,
                                int64_t slot_rows, const int32_t* valid, uint8_t* q, uint8_t* sf,
                                const float* global_scale, float* y_debug) {
  const char* what = "hq_fused_swiglu_quant";
  if (mode < HQ_MXFP8 || mode > HQ_NVFP4) return fail(HQ_ERR_MODE, "%s: unknown mode %d", what, mode);
  if (h <= 0 || h % 32 != 0 || h > kI32) return fail(HQ_ERR_SHAPE, "%s: h=%lld must be a positive multiple of 32", what, (long long)h);
  if (rows < 0 || rows > kI32) return fail(HQ_ERR_SHAPE, "%s: rows=%lld out of range", what, (long long)rows);
  if (num_groups < 1 || num_groups > 1024)
    return fail(HQ_ERR_SHAPE, "%s: num_groups=%d must be in [1, 1024]", what, num_groups);
  if (group_end == nullptr && slot_rows <= 0)
    return fail(HQ_ERR_SHAPE, "%s: slot_rows must be > 0 without group_end", what);
  if (mode == HQ_NVFP4 && global_scale == nullptr) return fail(HQ_ERR_NULL, "%s: NVFP4 needs global_scale", what);
  if (mode != HQ_NVFP4 && global_scale != nullptr) return fail(HQ_ERR_MODE, "%s: global_scale is NVFP4 only", what);
  if (rows == 0) return ok();
  if (!x || !q || !sf) return fail(HQ_ERR_NULL, "%s: x, q and sf are required", what);
  if (!aligned16(x) || !aligned16(q) || (y_debug && !aligned16(y_debug)))
    return fail(HQ_ERR_ALIGN, "%s: x, q and y_debug must be 16-byte aligned", what);
  hq::DeviceInfo dev;
  hq_status st = current_device(&dev);
  if (st != HQ_OK) return st;
  return launched(hq::launch_swiglu_quant((hipStream_t)stream, mode, x, rows, h, num_groups,
                                          group_end, slot_rows, valid, q, sf, global_scale, y_debug),
                  what);
}

hq_status hq_prefill_permute_to_masked_gemm(void* stream, const uint8_t* x, int64_t num_tokens,
                                            int64_t row_bytes, int64_t hidden, const void* scale,
                                            int32_t scale_mode, const int64_t* topk_ids,
                                            int32_t topk, int32_t num_experts,
                                            int64_t max_token_num, uint8_t* permute_x,
                                            uint8_t* out_scale, int32_t* indice_map,
                                            int32_t* token_nums) {
  const char* what = "hq_prefill_permute_to_masked_gemm";
  if (scale_mode != HQ_SCALE_BROADCAST && scale_mode != HQ_SCALE_DIRECT)
    return fail(HQ_ERR_MODE, "%s: unknown scale mode %d", what, scale_mode);
  if (num_tokens < 0) return fail(HQ_ERR_SHAPE, "%s: num_tokens=%lld < 0", what, (long long)num_tokens);
  if (topk < 1 || topk > 64) return fail(HQ_ERR_SHAPE, "%s: topk=%d must be in [1, 64]", what, topk);
  if (num_tokens * topk > kI32)
    return fail(HQ_ERR_SHAPE, "%s: num_tokens * topk must be < 2^31", what);
  if (num_experts < 1 || num_experts > 1024)
    return fail(HQ_ERR_SHAPE, "%s: num_experts=%d must be in [1, 1024]", what, num_experts);
  if (max_token_num < 128 || max_token_num % 128 != 0 || max_token_num > kI32)
    return fail(HQ_ERR_SHAPE, "%s: max_token_num=%lld must be a positive multiple of 128", what,
                (long long)max_token_num);
  if (num_experts * max_token_num > kI32)
    return fail(HQ_ERR_SHAPE, "%s: num_experts * max_token_num must be < 2^31", what);
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(HQ_ERR_SHAPE, "%s: row_bytes=%lld must be a positive multiple of 16", what, (long long)row_bytes);
  const int64_t hstep = scale_mode == HQ_SCALE_BROADCAST ? 512 : 128;
  if (hidden <= 0 || hidden % hstep != 0)
    return fail(HQ_ERR_SHAPE, "%s: hidden=%lld must be a positive multiple of %lld in this scale mode", what,
                (long long)hidden, (long long)hstep);
  if (!token_nums) return fail(HQ_ERR_NULL, "%s: token_nums is required", what);
  if (num_tokens > 0 && (!x || !scale || !topk_ids || !permute_x || !out_scale || !indice_map))
    return fail(HQ_ERR_NULL, "%s: x, scale, topk_ids, permute_x, out_scale and indice_map are required", what);
  if (!aligned16(x) || !aligned16(permute_x))
    return fail(HQ_ERR_ALIGN, "%s: x and permute_x must be 16-byte aligned", what);
  if ((reinterpret_cast<uintptr_t>(scale) | reinterpret_cast<uintptr_t>(out_scale)) & 3u)
    return fail(HQ_ERR_ALIGN, "%s: scale and out_scale must be 4-byte aligned", what);
  hq::DeviceInfo dev;
  hq_status st = current_device(&dev);
  if (st != HQ_OK) return st;
  return launched(hq::launch_permute((hipStream_t)stream, x, num_tokens, row_bytes, hidden, scale, scale_mode,
                                     topk_ids, topk, num_experts, max_token_num, permute_x, out_scale,
                                     indice_map, token_nums, dev.num_cus),
                  what);
}

}  // extern "C"
