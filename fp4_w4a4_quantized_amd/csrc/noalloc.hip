// noalloc.hip -- fp4q_quantize_noalloc: fp4q_quantize for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  The quantizer's
// workspace (the small-tensor NVFP4 exchange state, the partial maxima of
// the large path, the per-group amax words) is a file-scope device array
// instead of a caller buffer.  Each GPU the library runs on holds its own
// copy until the process ends; it is zero at module load, which is the
// state the exchange needs before its first use, and every call on a GPU
// shares it (overlapping calls on one GPU race).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fp4q_internal.h"

namespace {

constexpr size_t kScratchBytes = 32768;   // 512-byte exchange state + 8064 amax words
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.  In host code the
// array's name is a host-side stand-in, not a device address, so it is
// looked up once per device with that device current and kept.
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int fp4q_quantize_noalloc(fp4q_format_t fmt, fp4q_layout_t layout, const uint16_t* x,
                                     int64_t rows, int64_t cols, int64_t ldx,
                                     const int32_t* group_offsets, int32_t num_groups,
                                     const int32_t* chan_idx, int32_t n_chan, uint8_t* q,
                                     uint8_t* scales, float* tensor_scale, uint16_t* resid,
                                     void* stream) {
  // every argument check before the first HIP call, as for fp4q_quantize
  const int rc = fp4q::quantize_checks(fmt, layout, x, rows, cols, ldx, group_offsets, num_groups,
                                       chan_idx, n_chan, q, scales, tensor_scale, resid);
  if (rc != FP4Q_OK) return rc;
  if (fp4q_quantize_workspace_bytes(fmt, rows, cols, num_groups) > kScratchBytes)
    return FP4Q_ERR_UNSUPPORTED;   // more groups than the static scratch holds
  void* ptr = nullptr;
  const hipError_t e = scratch_on_current_device(&ptr);
  if (e != hipSuccess) {
    fp4q::set_last_hip_error((int)e);
    return FP4Q_ERR_HIP;
  }
  return fp4q_quantize(fmt, layout, x, rows, cols, ldx, group_offsets, num_groups, chan_idx,
                       n_chan, q, scales, tensor_scale, resid, ptr, kScratchBytes, stream);
}
