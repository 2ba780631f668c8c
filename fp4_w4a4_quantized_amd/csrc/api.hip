// api.hip -- the C ABI of libfp4q (declared in include/fp4q.h): host-side
// argument validation, workspace queries and kernel launches.  Every check
// runs before the first HIP call, so invalid calls fail without touching
// the device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "fp4q_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

// FP4Q_HOOK_FAIL_NEXT_LAUNCH: a hipError_t that the next call which would
// launch reports instead of launching (0: none).
std::atomic<int> g_fail_next{0};

// True (and the hook consumed) when a test asked the launch path to fail.
inline bool injected_failure() {
  const int e = g_fail_next.exchange(0);
  if (e == 0) return false;
  g_last_hip_error = e;
  return true;
}

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

inline int blk_of(int fmt) { return fmt == FP4Q_NVFP4 ? 16 : 32; }

inline bool fmt_ok(int fmt) { return fmt == FP4Q_NVFP4 || fmt == FP4Q_MXFP4; }

inline bool layout_ok(int layout) {
  return layout == FP4Q_LAYOUT_ROWMAJOR || layout == FP4Q_LAYOUT_TILED;
}

// Clear any stale error state before a launch, so that check_launch() sees
// only what this call's launches produced.
inline void clear_error() { (void)hipGetLastError(); }

// Report launch errors from the calls just made on this thread.
inline int check_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FP4Q_ERR_HIP;
  }
  return FP4Q_OK;
}

constexpr int MAX_GROUPS = 2048;  // grouped GEMM scans 8 groups per thread of 256

}  // namespace

extern "C" {

const char* fp4q_status_str(int status) {
  switch (status) {
    case FP4Q_OK: return "ok";
    case FP4Q_ERR_INVALID: return "invalid argument";
    case FP4Q_ERR_UNSUPPORTED: return "unsupported shape";
    case FP4Q_ERR_WORKSPACE: return "workspace missing or too small";
    case FP4Q_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int fp4q_last_hip_error(void) { return g_last_hip_error; }

int fp4q_packed_bytes(fp4q_format_t fmt, fp4q_layout_t layout, int64_t rows, int64_t cols,
                      size_t* code_bytes, size_t* scale_bytes) {
  if (!fmt_ok(fmt) || !layout_ok(layout) || rows < 0 || cols <= 0) return FP4Q_ERR_INVALID;
  const int blk = blk_of(fmt);
  if (cols % blk != 0) return FP4Q_ERR_INVALID;
  int64_t rc = rows, rs = rows;
  if (layout == FP4Q_LAYOUT_TILED) {
    if (cols % 128 != 0) return FP4Q_ERR_INVALID;
    rc = (rows + 15) / 16 * 16;
    rs = (rows + 63) / 64 * 64;
  }
  if (code_bytes) *code_bytes = (size_t)(rc * (cols / 2));
  if (scale_bytes) *scale_bytes = (size_t)(rs * (cols / blk));
  return FP4Q_OK;
}

size_t fp4q_quantize_workspace_bytes(fp4q_format_t fmt, int64_t rows, int64_t cols,
                                     int32_t num_groups) {
  (void)rows;
  (void)cols;
  return fp4q::quantize_workspace_bytes(fmt, num_groups > 0 ? num_groups : 1);
}

}  // extern "C"

namespace fp4q {

void set_last_hip_error(int e) { g_last_hip_error = e; }

// fp4q_quantize's argument checks other than the workspace (host only).
int quantize_checks(int fmt, int layout, const uint16_t* x, int64_t rows, int64_t cols,
                    int64_t ldx, const int32_t* group_offsets, int32_t num_groups,
                    const int32_t* chan_idx, int32_t n_chan, const uint8_t* q,
                    const uint8_t* scales, const float* tensor_scale, const uint16_t* resid) {
  if (!fmt_ok(fmt) || !layout_ok(layout)) return FP4Q_ERR_INVALID;
  const int blk = blk_of(fmt);
  if (rows < 0 || cols <= 0 || cols % blk != 0 || ldx < cols || ldx % 8 != 0)
    return FP4Q_ERR_INVALID;
  if (layout == FP4Q_LAYOUT_TILED && cols % 128 != 0) return FP4Q_ERR_INVALID;
  if (num_groups < 1 || (num_groups > 1 && !group_offsets)) return FP4Q_ERR_INVALID;
  if (n_chan < 0 || n_chan > cols) return FP4Q_ERR_INVALID;
  if ((n_chan > 0) != (chan_idx != nullptr) || (n_chan > 0) != (resid != nullptr))
    return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_NVFP4 && !tensor_scale) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_MXFP4 && tensor_scale) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!x || !q || !scales)) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4)))
    return FP4Q_ERR_INVALID;
  const int64_t prow = layout == FP4Q_LAYOUT_TILED ? (rows + 15) / 16 * 16 : rows;
  if (prow * (cols / 8) >= ((int64_t)1 << 31)) return FP4Q_ERR_UNSUPPORTED;  // 32-bit chunk index
  return FP4Q_OK;
}

}  // namespace fp4q

extern "C" {

int fp4q_quantize(fp4q_format_t fmt, fp4q_layout_t layout, const uint16_t* x, int64_t rows,
                  int64_t cols, int64_t ldx, const int32_t* group_offsets, int32_t num_groups,
                  const int32_t* chan_idx, int32_t n_chan, uint8_t* q, uint8_t* scales,
                  float* tensor_scale, uint16_t* resid, void* workspace, size_t workspace_bytes,
                  void* stream) {
  const int rc = fp4q::quantize_checks(fmt, layout, x, rows, cols, ldx, group_offsets, num_groups,
                                       chan_idx, n_chan, q, scales, tensor_scale, resid);
  if (rc != FP4Q_OK) return rc;
  const size_t need = fp4q_quantize_workspace_bytes(fmt, rows, cols, num_groups);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 8)))
    return FP4Q_ERR_WORKSPACE;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_quantize(fmt, layout == FP4Q_LAYOUT_TILED, x, rows, cols, ldx, group_offsets,
                        num_groups, chan_idx, n_chan, q, scales, tensor_scale, resid, workspace,
                        static_cast<hipStream_t>(stream));
  return check_launch();
}

size_t fp4q_qdq_fallback_workspace_bytes(fp4q_format_t fmt, int64_t rows, int64_t cols) {
  (void)rows;
  (void)cols;
  return fp4q::quantize_workspace_bytes(fmt, 1);
}

int fp4q_qdq_fallback(fp4q_format_t fmt, const uint16_t* x, int64_t rows, int64_t cols,
                      int64_t ldx, float* y, int64_t ldy, int64_t* n_fallback, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!fmt_ok(fmt)) return FP4Q_ERR_INVALID;
  if (rows < 0 || cols <= 0 || cols % blk_of(fmt) != 0 || ldx < cols || ldx % 8 != 0)
    return FP4Q_ERR_INVALID;
  if (ldy < cols || ldy % 4 != 0) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!x || !y || !aligned(x, 16) || !aligned(y, 16))) return FP4Q_ERR_INVALID;
  if (n_fallback && !aligned(n_fallback, 8)) return FP4Q_ERR_INVALID;
  if (rows * (cols / 8) >= ((int64_t)1 << 31)) return FP4Q_ERR_UNSUPPORTED;
  const size_t need = fp4q_qdq_fallback_workspace_bytes(fmt, rows, cols);
  if (need > 0 && rows > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 8)))
    return FP4Q_ERR_WORKSPACE;
  if (rows == 0 && !n_fallback) return FP4Q_OK;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_qdq_fallback(fmt, x, rows, cols, ldx, y, ldy, n_fallback, workspace,
                            static_cast<hipStream_t>(stream));
  return check_launch();
}

int fp4q_quantize_status(const void* workspace, size_t workspace_bytes, int32_t* status,
                         void* stream) {
  if (!status) return FP4Q_ERR_INVALID;
  if (!workspace || !aligned(workspace, 8) ||
      workspace_bytes < fp4q_quantize_workspace_bytes(FP4Q_NVFP4, 0, 16, 1))
    return FP4Q_ERR_WORKSPACE;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  uint32_t v = 0;
  if (fp4q::quantize_status(workspace, static_cast<hipStream_t>(stream), &v) != 0) {
    const hipError_t e = hipGetLastError();
    g_last_hip_error = e != hipSuccess ? (int)e : (int)hipErrorUnknown;
    return FP4Q_ERR_HIP;
  }
  *status = (int32_t)v;
  return FP4Q_OK;
}

int fp4q_test_hook(int32_t hook, int64_t value) {
  switch (hook) {
    case FP4Q_HOOK_RESET:
      g_fail_next.store(0);
      fp4q::set_grid_hooks(0, -1);
      return FP4Q_OK;
    case FP4Q_HOOK_FAIL_NEXT_LAUNCH:
      if (value <= 0 || value > INT32_MAX) return FP4Q_ERR_INVALID;
      g_fail_next.store((int)value);
      return FP4Q_OK;
    case FP4Q_HOOK_GRID_SPIN_LIMIT:
      if (value < 0 || value > UINT32_MAX) return FP4Q_ERR_INVALID;
      fp4q::set_grid_hooks((uint32_t)value, fp4q::grid_hook_skip());
      return FP4Q_OK;
    case FP4Q_HOOK_GRID_SKIP_SLOT:
      if (value < -1 || value > 1 << 20) return FP4Q_ERR_INVALID;
      fp4q::set_grid_hooks(fp4q::grid_hook_spin(), (int)value);
      return FP4Q_OK;
    default:
      return FP4Q_ERR_INVALID;
  }
}

static int validate_gemm_common(int fmt, int64_t N, int64_t K, const uint8_t* a_q,
                                const uint8_t* a_s, const float* a_ts, const uint8_t* b_q,
                                const uint8_t* b_s, const float* b_ts, const int32_t* chan_idx,
                                int32_t n_chan, const uint16_t* resid, const void* y,
                                int y_dtype, int64_t rows) {
  if (!fmt_ok(fmt)) return FP4Q_ERR_INVALID;
  if (y_dtype != FP4Q_OUT_F32 && y_dtype != FP4Q_OUT_BF16) return FP4Q_ERR_INVALID;
  if (rows < 0 || N < 0 || K <= 0 || K % blk_of(fmt) != 0) return FP4Q_ERR_INVALID;
  if (n_chan < 0 || n_chan > K) return FP4Q_ERR_INVALID;
  if ((n_chan > 0) != (chan_idx != nullptr) || (n_chan > 0) != (resid != nullptr))
    return FP4Q_ERR_INVALID;
  if (n_chan > 0 && !aligned(resid, 16)) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_NVFP4 && (!a_ts || !b_ts)) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_MXFP4 && (a_ts || b_ts)) return FP4Q_ERR_INVALID;
  if (rows > 0 && N > 0) {
    if (!a_q || !a_s || !b_q || !b_s || !y) return FP4Q_ERR_INVALID;
    if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_s, 8) || !aligned(b_s, 8))
      return FP4Q_ERR_INVALID;
  }
  if (K % 128 != 0) return FP4Q_ERR_UNSUPPORTED;
  return FP4Q_OK;
}

// The experts' weight layout of a grouped GEMM: row-major everywhere; tiled
// where the 128 x 512 NVFP4 grouped kernel serves the shape (its tokens'
// codes below 4 GiB when gathered).
static int validate_w_layout(int fmt, int w_layout, int64_t N, int64_t K, int32_t n_chan,
                             int64_t gather_bytes = 0) {
  if (!layout_ok(w_layout)) return FP4Q_ERR_INVALID;
  if (w_layout != FP4Q_LAYOUT_TILED) return FP4Q_OK;
  if (K % 128 != 0) return FP4Q_ERR_INVALID;
  if (!fp4q::grouped_tiled_ok(fmt, N, K, n_chan) || gather_bytes > (int64_t)UINT32_MAX)
    return FP4Q_ERR_UNSUPPORTED;
  return FP4Q_OK;
}

size_t fp4q_gemm_workspace_bytes(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M, int64_t N,
                                 int64_t K, int32_t n_chan) {
  (void)fmt;
  (void)layout;
  if (M <= 0 || N <= 0 || K <= 0 || n_chan <= 0) return 0;
  return fp4q::gemm_workspace_bytes(M, N, K, n_chan);
}

int fp4q_gemm(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M, int64_t N, int64_t K,
              const uint8_t* a_q, const uint8_t* a_s, const float* a_ts, const uint8_t* b_q,
              const uint8_t* b_s, const float* b_ts, const int32_t* chan_idx, int32_t n_chan,
              const uint16_t* resid, void* y, fp4q_dtype_t y_dtype, int64_t ldy, void* workspace,
              size_t workspace_bytes, void* stream) {
  if (!layout_ok(layout)) return FP4Q_ERR_INVALID;
  int rc = validate_gemm_common(fmt, N, K, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan,
                                resid, y, y_dtype, M);
  if (rc != FP4Q_OK) return rc;
  if (ldy < N) return FP4Q_ERR_INVALID;
  if ((M + 127) / 128 > (int64_t)UINT32_MAX || (N + 31) / 32 > 65535) return FP4Q_ERR_UNSUPPORTED;
  const size_t need = fp4q_gemm_workspace_bytes(fmt, layout, M, N, K, n_chan);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
    return FP4Q_ERR_WORKSPACE;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_gemm(fmt, layout == FP4Q_LAYOUT_TILED, M, N, K, nullptr, 1, a_q, a_s, a_ts, b_q,
                    b_s, b_ts, chan_idx, n_chan, resid, nullptr, y, y_dtype == FP4Q_OUT_BF16, ldy,
                    workspace, static_cast<hipStream_t>(stream));
  return check_launch();
}

size_t fp4q_comp_weights_bytes(fp4q_format_t fmt, fp4q_layout_t layout, int64_t N, int64_t K,
                               int32_t n_chan) {
  (void)fmt;
  (void)layout;
  (void)K;
  return fp4q::comp_weights_bytes(N, n_chan);
}

int fp4q_comp_weights(fp4q_format_t fmt, fp4q_layout_t layout, int64_t N, int64_t K,
                      const uint8_t* b_q, const uint8_t* b_s, const int32_t* chan_idx,
                      int32_t n_chan, uint8_t* out, size_t out_bytes, void* stream) {
  if (!layout_ok(layout) || !fmt_ok(fmt)) return FP4Q_ERR_INVALID;
  if (N < 0 || K < 0 || n_chan < 0) return FP4Q_ERR_INVALID;
  if ((n_chan > 0) != (chan_idx != nullptr)) return FP4Q_ERR_INVALID;
  if (N == 0 || n_chan == 0) return FP4Q_OK;
  if (!b_q || !b_s || !out || !aligned(out, 16)) return FP4Q_ERR_INVALID;
  if (K % 128 != 0) return FP4Q_ERR_UNSUPPORTED;
  if (out_bytes < fp4q_comp_weights_bytes(fmt, layout, N, K, n_chan)) return FP4Q_ERR_WORKSPACE;
  if (((N + 15) / 16) * ((n_chan + 31) / 32) / 4 >= (int64_t)UINT32_MAX)
    return FP4Q_ERR_UNSUPPORTED;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_comp_weights(fmt, layout == FP4Q_LAYOUT_TILED, b_q, b_s, N, K, chan_idx, n_chan, 1,
                            out, static_cast<hipStream_t>(stream));
  return check_launch();
}

int fp4q_gemm_prepared(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M, int64_t N, int64_t K,
                       const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                       const uint8_t* b_q, const uint8_t* b_s, const float* b_ts,
                       const int32_t* chan_idx, int32_t n_chan, const uint16_t* resid,
                       const uint8_t* comp_w, size_t comp_w_bytes, void* y,
                       fp4q_dtype_t y_dtype, int64_t ldy, void* stream) {
  if (!layout_ok(layout)) return FP4Q_ERR_INVALID;
  int rc = validate_gemm_common(fmt, N, K, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan,
                                resid, y, y_dtype, M);
  if (rc != FP4Q_OK) return rc;
  if (ldy < N) return FP4Q_ERR_INVALID;
  if ((M + 127) / 128 > (int64_t)UINT32_MAX || (N + 31) / 32 > 65535) return FP4Q_ERR_UNSUPPORTED;
  const bool work = M > 0 && N > 0 && n_chan > 0;
  if (work && (!comp_w || !aligned(comp_w, 16) ||
               comp_w_bytes < fp4q_comp_weights_bytes(fmt, layout, N, K, n_chan)))
    return FP4Q_ERR_WORKSPACE;
  // shapes whose kernels stream no compensation weights take the term from
  // chan_idx as fp4q_gemm does (they need no workspace)
  if (fp4q::gemm_path(M, N, K, n_chan) == fp4q::PATH_GENERIC) comp_w = nullptr;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_gemm(fmt, layout == FP4Q_LAYOUT_TILED, M, N, K, nullptr, 1, a_q, a_s, a_ts, b_q,
                    b_s, b_ts, chan_idx, n_chan, resid, nullptr, y, y_dtype == FP4Q_OUT_BF16, ldy,
                    nullptr, static_cast<hipStream_t>(stream), work ? comp_w : nullptr);
  return check_launch();
}

int fp4q_gemm_decode_fused(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M, int64_t N,
                           int64_t K, const uint16_t* x, int64_t ldx, const uint8_t* b_q,
                           const uint8_t* b_s, const float* b_ts, const int32_t* chan_idx,
                           int32_t n_chan, const uint8_t* comp_w, size_t comp_w_bytes, void* y,
                           fp4q_dtype_t y_dtype, int64_t ldy, uint8_t* a_q_out,
                           uint8_t* a_s_out, float* a_ts_out, uint16_t* resid_out,
                           void* stream) {
  if (!fmt_ok(fmt) || !layout_ok(layout)) return FP4Q_ERR_INVALID;
  if (y_dtype != FP4Q_OUT_F32 && y_dtype != FP4Q_OUT_BF16) return FP4Q_ERR_INVALID;
  if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || ldx < K || ldx % 8 != 0 || ldy < N)
    return FP4Q_ERR_INVALID;
  if (n_chan < 0 || n_chan > K || (n_chan > 0) != (chan_idx != nullptr)) return FP4Q_ERR_INVALID;
  if (!b_ts) return FP4Q_ERR_INVALID;
  const bool outs = a_q_out != nullptr;
  if (outs != (a_s_out != nullptr) || outs != (a_ts_out != nullptr) ||
      (outs && n_chan > 0) != (resid_out != nullptr))
    return FP4Q_ERR_INVALID;
  if (M > 0 && N > 0) {
    if (!x || !b_q || !b_s || !y) return FP4Q_ERR_INVALID;
    if (!aligned(x, 16) || !aligned(b_q, 16) || !aligned(b_s, 8)) return FP4Q_ERR_INVALID;
    if (outs && (!aligned(a_q_out, 16) || !aligned(a_s_out, 2))) return FP4Q_ERR_INVALID;
  }
  if (fmt != FP4Q_NVFP4 || K % 128 != 0 || !fp4q::decode_fused_eligible(M > 0 ? M : 1, K, n_chan))
    return FP4Q_ERR_UNSUPPORTED;
  if ((N + 47) / 48 > (int64_t)INT32_MAX) return FP4Q_ERR_UNSUPPORTED;
  const bool work = M > 0 && N > 0;
  if (work && n_chan > 0 &&
      (!comp_w || !aligned(comp_w, 16) ||
       comp_w_bytes < fp4q_comp_weights_bytes(fmt, layout, N, K, n_chan)))
    return FP4Q_ERR_WORKSPACE;
  if (!work) return FP4Q_OK;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_gemm_decode_fused(layout == FP4Q_LAYOUT_TILED, M, N, K, x, ldx, b_q, b_s, b_ts,
                                 chan_idx, n_chan, n_chan > 0 ? comp_w : nullptr, y,
                                 y_dtype == FP4Q_OUT_BF16, ldy, a_q_out, a_s_out, a_ts_out,
                                 resid_out, static_cast<hipStream_t>(stream));
  return check_launch();
}

static size_t deq_resid_bytes(int64_t M, int32_t n_chan) {
  return (size_t)((M * n_chan * 2 + 255) / 256 * 256);
}

size_t fp4q_gemm_residual_fp4_workspace_bytes(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M,
                                              int64_t N, int64_t K, int32_t n_chan) {
  if (M <= 0 || N <= 0 || K <= 0 || n_chan <= 0) return 0;
  return deq_resid_bytes(M, n_chan) + fp4q_gemm_workspace_bytes(fmt, layout, M, N, K, n_chan);
}

int fp4q_gemm_residual_fp4(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M, int64_t N,
                           int64_t K, const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                           const uint8_t* b_q, const uint8_t* b_s, const float* b_ts,
                           const int32_t* chan_idx, int32_t n_chan, const uint8_t* r_q,
                           const uint8_t* r_s, const float* r_ts, void* y, fp4q_dtype_t y_dtype,
                           int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  if (!layout_ok(layout) || !fmt_ok(fmt)) return FP4Q_ERR_INVALID;
  if (n_chan < 0 || (n_chan > 0) != (r_q != nullptr) || (n_chan > 0) != (r_s != nullptr))
    return FP4Q_ERR_INVALID;
  if (n_chan % blk_of(fmt) != 0) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_NVFP4 && (n_chan > 0) != (r_ts != nullptr)) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_MXFP4 && r_ts) return FP4Q_ERR_INVALID;
  const bool work = M > 0 && N > 0 && n_chan > 0;
  const size_t need = work ? fp4q_gemm_residual_fp4_workspace_bytes(fmt, layout, M, N, K, n_chan)
                           : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
    return FP4Q_ERR_WORKSPACE;
  // the decoded residual goes to the front of the workspace; it stands in
  // for fp4q_gemm's resid in the shared validation (an empty product only
  // needs a non-null stand-in, never read)
  alignas(16) static const uint16_t kNoRows[8] = {};
  uint16_t* rdeq = work ? static_cast<uint16_t*>(workspace) : nullptr;
  const uint16_t* rval = work ? rdeq : (n_chan > 0 ? kNoRows : nullptr);
  int rc = validate_gemm_common(fmt, N, K, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan,
                                rval, y, y_dtype, M);
  if (rc != FP4Q_OK) return rc;
  if (ldy < N) return FP4Q_ERR_INVALID;
  if ((M + 127) / 128 > (int64_t)UINT32_MAX || (N + 31) / 32 > 65535) return FP4Q_ERR_UNSUPPORTED;
  if (M * (int64_t)n_chan / 8 >= ((int64_t)1 << 31)) return FP4Q_ERR_UNSUPPORTED;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  void* gws = work ? static_cast<uint8_t*>(workspace) + deq_resid_bytes(M, n_chan) : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (work) fp4q::launch_deq_resid(fmt, M, n_chan, r_q, r_s, rdeq, st);
  fp4q::launch_gemm(fmt, layout == FP4Q_LAYOUT_TILED, M, N, K, nullptr, 1, a_q, a_s, a_ts, b_q,
                    b_s, b_ts, chan_idx, n_chan, rval, r_ts, y, y_dtype == FP4Q_OUT_BF16, ldy, gws,
                    st);
  return check_launch();
}

size_t fp4q_grouped_gemm_workspace_bytes(fp4q_format_t fmt, fp4q_layout_t w_layout,
                                         int64_t total_rows, int64_t N, int64_t K,
                                         int32_t num_groups, int32_t n_chan) {
  (void)fmt;
  (void)w_layout;
  if (total_rows <= 0 || N <= 0 || K <= 0 || n_chan <= 0 || num_groups < 1) return 0;
  return fp4q::grouped_workspace_bytes(N, K, num_groups, n_chan);
}

int fp4q_grouped_gemm(fp4q_format_t fmt, fp4q_layout_t w_layout, int64_t total_rows, int64_t N,
                      int64_t K, const int32_t* group_offsets, int32_t num_groups,
                      const uint8_t* a_q,
                      const uint8_t* a_s, const float* a_ts, const uint8_t* b_q,
                      const uint8_t* b_s, const float* b_ts, const int32_t* chan_idx,
                      int32_t n_chan, const uint16_t* resid, void* y, fp4q_dtype_t y_dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_gemm_common(fmt, N, K, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan,
                                resid, y, y_dtype, total_rows);
  if (rc != FP4Q_OK) return rc;
  if ((rc = validate_w_layout(fmt, w_layout, N, K, n_chan)) != FP4Q_OK) return rc;
  if (num_groups < 1 || !group_offsets) return FP4Q_ERR_INVALID;
  if (num_groups > MAX_GROUPS) return FP4Q_ERR_UNSUPPORTED;
  if ((N + 127) / 128 > 65535) return FP4Q_ERR_UNSUPPORTED;
  const size_t need =
      fp4q_grouped_gemm_workspace_bytes(fmt, w_layout, total_rows, N, K, num_groups, n_chan);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
    return FP4Q_ERR_WORKSPACE;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_gemm(fmt, w_layout == FP4Q_LAYOUT_TILED, total_rows, N, K, group_offsets,
                    num_groups, a_q, a_s, a_ts, b_q,
                    b_s, b_ts, chan_idx, n_chan, resid, nullptr, y, y_dtype == FP4Q_OUT_BF16, N,
                    workspace, static_cast<hipStream_t>(stream));
  return check_launch();
}

size_t fp4q_grouped_gemm_residual_fp4_workspace_bytes(fp4q_format_t fmt,
                                                      fp4q_layout_t w_layout,
                                                      int64_t total_rows, int64_t N, int64_t K,
                                                      int32_t num_groups, int32_t n_chan) {
  if (total_rows <= 0 || N <= 0 || K <= 0 || n_chan <= 0 || num_groups < 1) return 0;
  return deq_resid_bytes(total_rows, n_chan) +
         fp4q_grouped_gemm_workspace_bytes(fmt, w_layout, total_rows, N, K, num_groups, n_chan);
}

int fp4q_grouped_gemm_residual_fp4(fp4q_format_t fmt, fp4q_layout_t w_layout,
                                   int64_t total_rows, int64_t N, int64_t K,
                                   const int32_t* group_offsets, int32_t num_groups,
                                   const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                                   const uint8_t* b_q, const uint8_t* b_s, const float* b_ts,
                                   const int32_t* chan_idx, int32_t n_chan, const uint8_t* r_q,
                                   const uint8_t* r_s, const float* r_ts, void* y,
                                   fp4q_dtype_t y_dtype, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!fmt_ok(fmt)) return FP4Q_ERR_INVALID;
  if (n_chan < 0 || (n_chan > 0) != (r_q != nullptr) || (n_chan > 0) != (r_s != nullptr))
    return FP4Q_ERR_INVALID;
  if (n_chan % blk_of(fmt) != 0) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_NVFP4 && (n_chan > 0) != (r_ts != nullptr)) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_MXFP4 && r_ts) return FP4Q_ERR_INVALID;
  if (num_groups < 1 || !group_offsets) return FP4Q_ERR_INVALID;
  if (num_groups > MAX_GROUPS) return FP4Q_ERR_UNSUPPORTED;
  const bool work = total_rows > 0 && N > 0 && n_chan > 0;
  const size_t need = work ? fp4q_grouped_gemm_residual_fp4_workspace_bytes(
                                 fmt, w_layout, total_rows, N, K, num_groups, n_chan)
                           : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
    return FP4Q_ERR_WORKSPACE;
  // the decoded residual goes to the front of the workspace and stands in
  // for fp4q_grouped_gemm's resid (an empty product only needs a non-null
  // stand-in, never read)
  alignas(16) static const uint16_t kNoRows[8] = {};
  uint16_t* rdeq = work ? static_cast<uint16_t*>(workspace) : nullptr;
  const uint16_t* rval = work ? rdeq : (n_chan > 0 ? kNoRows : nullptr);
  int rc = validate_gemm_common(fmt, N, K, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan,
                                rval, y, y_dtype, total_rows);
  if (rc != FP4Q_OK) return rc;
  if ((rc = validate_w_layout(fmt, w_layout, N, K, n_chan)) != FP4Q_OK) return rc;
  if ((N + 127) / 128 > 65535) return FP4Q_ERR_UNSUPPORTED;
  if (total_rows * (int64_t)n_chan / 8 >= ((int64_t)1 << 31)) return FP4Q_ERR_UNSUPPORTED;
  if (total_rows == 0 || N == 0) return FP4Q_OK;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  void* gws = work ? static_cast<uint8_t*>(workspace) + deq_resid_bytes(total_rows, n_chan)
                   : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (work) fp4q::launch_deq_resid(fmt, total_rows, n_chan, r_q, r_s, rdeq, st);
  fp4q::launch_gemm(fmt, w_layout == FP4Q_LAYOUT_TILED, total_rows, N, K, group_offsets,
                    num_groups, a_q, a_s, a_ts, b_q,
                    b_s, b_ts, chan_idx, n_chan, rval, r_ts, y, y_dtype == FP4Q_OUT_BF16, N, gws,
                    st);
  return check_launch();
}

size_t fp4q_grouped_comp_weights_bytes(fp4q_format_t fmt, int64_t N, int64_t K,
                                       int32_t num_groups, int32_t n_chan) {
  (void)fmt;
  (void)K;
  if (num_groups < 1) return 0;
  return (size_t)num_groups * fp4q::comp_weights_bytes(N, n_chan);
}

int fp4q_grouped_comp_weights(fp4q_format_t fmt, fp4q_layout_t w_layout, int64_t N, int64_t K,
                              int32_t num_groups, const uint8_t* b_q, const uint8_t* b_s,
                              const int32_t* chan_idx, int32_t n_chan, uint8_t* out,
                              size_t out_bytes, void* stream) {
  if (!fmt_ok(fmt) || !layout_ok(w_layout)) return FP4Q_ERR_INVALID;
  if (N < 0 || K < 0 || n_chan < 0 || num_groups < 1) return FP4Q_ERR_INVALID;
  if (num_groups > MAX_GROUPS) return FP4Q_ERR_UNSUPPORTED;
  if ((n_chan > 0) != (chan_idx != nullptr)) return FP4Q_ERR_INVALID;
  if (N == 0 || n_chan == 0) return FP4Q_OK;
  if (!b_q || !b_s || !out || !aligned(out, 16)) return FP4Q_ERR_INVALID;
  if (K % 128 != 0) return FP4Q_ERR_UNSUPPORTED;
  if (out_bytes < fp4q_grouped_comp_weights_bytes(fmt, N, K, num_groups, n_chan))
    return FP4Q_ERR_WORKSPACE;
  if ((int64_t)num_groups * ((N + 15) / 16) * ((n_chan + 31) / 32) / 4 >= (int64_t)UINT32_MAX)
    return FP4Q_ERR_UNSUPPORTED;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_comp_weights(fmt, w_layout == FP4Q_LAYOUT_TILED, b_q, b_s, N, K, chan_idx,
                            n_chan, num_groups, out, static_cast<hipStream_t>(stream));
  return check_launch();
}

int fp4q_grouped_gemm_prepared(fp4q_format_t fmt, fp4q_layout_t w_layout, int64_t total_rows,
                               int64_t N, int64_t K, const int32_t* group_offsets,
                               int32_t num_groups,
                               const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                               const uint8_t* b_q, const uint8_t* b_s, const float* b_ts,
                               const int32_t* chan_idx, int32_t n_chan, const uint16_t* resid,
                               const uint8_t* comp_w, size_t comp_w_bytes, void* y,
                               fp4q_dtype_t y_dtype, void* stream) {
  int rc = validate_gemm_common(fmt, N, K, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan,
                                resid, y, y_dtype, total_rows);
  if (rc != FP4Q_OK) return rc;
  if ((rc = validate_w_layout(fmt, w_layout, N, K, n_chan)) != FP4Q_OK) return rc;
  if (num_groups < 1 || !group_offsets) return FP4Q_ERR_INVALID;
  if (num_groups > MAX_GROUPS) return FP4Q_ERR_UNSUPPORTED;
  if ((N + 127) / 128 > 65535) return FP4Q_ERR_UNSUPPORTED;
  const bool work = total_rows > 0 && N > 0 && n_chan > 0;
  if (work && (!comp_w || !aligned(comp_w, 16) ||
               comp_w_bytes < fp4q_grouped_comp_weights_bytes(fmt, N, K, num_groups, n_chan)))
    return FP4Q_ERR_WORKSPACE;
  // shapes served by the general grouped kernel take the term from chan_idx
  if (!fp4q::big_grouped_eligible(N, K, n_chan)) comp_w = nullptr;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_gemm(fmt, w_layout == FP4Q_LAYOUT_TILED, total_rows, N, K, group_offsets,
                    num_groups, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan, resid, nullptr,
                    y, y_dtype == FP4Q_OUT_BF16, N, nullptr, static_cast<hipStream_t>(stream),
                    work ? comp_w : nullptr);
  return check_launch();
}

int fp4q_grouped_gemm_gather(fp4q_format_t fmt, fp4q_layout_t w_layout, int64_t total_rows,
                             int64_t N, int64_t K, const int32_t* group_offsets,
                             int32_t num_groups,
                             const int32_t* row_src, int64_t tokens, const uint8_t* a_q,
                             const uint8_t* a_s, const float* a_ts, const uint8_t* b_q,
                             const uint8_t* b_s, const float* b_ts, const int32_t* chan_idx,
                             int32_t n_chan, const uint16_t* resid, const uint8_t* comp_w,
                             size_t comp_w_bytes, void* y, fp4q_dtype_t y_dtype, void* stream) {
  int rc = validate_gemm_common(fmt, N, K, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan,
                                resid, y, y_dtype, total_rows);
  if (rc != FP4Q_OK) return rc;
  if (num_groups < 1 || !group_offsets) return FP4Q_ERR_INVALID;
  if (tokens < 0 || (total_rows > 0 && (tokens == 0 || !row_src))) return FP4Q_ERR_INVALID;
  if ((rc = validate_w_layout(fmt, w_layout, N, K, n_chan, tokens * (K / 2))) != FP4Q_OK)
    return rc;
  if (num_groups > MAX_GROUPS) return FP4Q_ERR_UNSUPPORTED;
  if ((N + 127) / 128 > 65535 || !fp4q::big_grouped_eligible(N, K, n_chan))
    return FP4Q_ERR_UNSUPPORTED;
  const bool work = total_rows > 0 && N > 0;
  if (work && n_chan > 0 &&
      (!comp_w || !aligned(comp_w, 16) ||
       comp_w_bytes < fp4q_grouped_comp_weights_bytes(fmt, N, K, num_groups, n_chan)))
    return FP4Q_ERR_WORKSPACE;
  if (!work) return FP4Q_OK;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_gemm_big_grouped(fmt, total_rows, N, K, group_offsets, num_groups, a_q, a_s, a_ts,
                                b_q, b_s, b_ts, chan_idx, n_chan, resid, nullptr,
                                n_chan > 0 ? comp_w : nullptr, y, y_dtype == FP4Q_OUT_BF16, nullptr,
                                static_cast<hipStream_t>(stream), w_layout == FP4Q_LAYOUT_TILED,
                                row_src, tokens);
  return check_launch();
}

size_t fp4q_select_channels_workspace_bytes(int64_t rows, int64_t cols) {
  return fp4q::select_workspace_bytes(rows, cols);
}

int fp4q_select_channels(fp4q_format_t fmt, fp4q_layout_t layout, const uint16_t* x,
                         int64_t rows, int64_t cols, int64_t ldx, const uint8_t* q,
                         const uint8_t* scales, const float* tensor_scale, int32_t k,
                         int32_t* chan_out, uint16_t* resid_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!fmt_ok(fmt) || !layout_ok(layout)) return FP4Q_ERR_INVALID;
  if (rows < 0 || cols <= 0 || cols % blk_of(fmt) != 0 || ldx < cols || ldx % 8 != 0)
    return FP4Q_ERR_INVALID;
  if (layout == FP4Q_LAYOUT_TILED && cols % 128 != 0) return FP4Q_ERR_INVALID;
  if (k < 0 || k > cols) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_NVFP4 && !tensor_scale) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_MXFP4 && tensor_scale) return FP4Q_ERR_INVALID;
  if (k > 0 && (!chan_out || !aligned(chan_out, 4))) return FP4Q_ERR_INVALID;
  if (rows > 0 && k > 0 && (!resid_out || !aligned(resid_out, 2))) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!x || !q || !scales)) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!aligned(x, 16) || !aligned(q, 4))) return FP4Q_ERR_INVALID;
  if (cols > INT32_MAX || rows * (int64_t)k >= ((int64_t)1 << 31)) return FP4Q_ERR_UNSUPPORTED;
  if (k == 0) return FP4Q_OK;
  const size_t need = fp4q::select_workspace_bytes(rows, cols);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return FP4Q_ERR_WORKSPACE;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_select(fmt, layout == FP4Q_LAYOUT_TILED, x, rows, cols, ldx, q, scales,
                      tensor_scale, k, chan_out, resid_out, workspace,
                      static_cast<hipStream_t>(stream));
  return check_launch();
}

static size_t round256_sz(size_t b) { return (b + 255) / 256 * 256; }

size_t fp4q_quantize_select_workspace_bytes(fp4q_format_t fmt, fp4q_layout_t layout,
                                            int64_t rows, int64_t cols) {
  if (!fmt_ok(fmt) || !layout_ok(layout) || rows < 0 || cols <= 0) return 0;
  const size_t qb = round256_sz(fp4q_quantize_workspace_bytes(fmt, rows, cols, 1));
  size_t sb = fp4q::select_workspace_bytes(rows, cols);
  if (rows > 0 && cols % 32 == 0) {
    const int64_t bands = fp4q::quantize_score_bands(layout == FP4Q_LAYOUT_TILED, rows, cols);
    sb = std::max(sb, fp4q::select_scored_workspace_bytes(bands, cols));
  }
  return qb + sb;
}

int fp4q_quantize_select(fp4q_format_t fmt, fp4q_layout_t layout, const uint16_t* x,
                         int64_t rows, int64_t cols, int64_t ldx, int32_t k, uint8_t* q,
                         uint8_t* scales, float* tensor_scale, int32_t* chan_out,
                         uint16_t* resid_out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  const int rc = fp4q::quantize_checks(fmt, layout, x, rows, cols, ldx, nullptr, 1, nullptr, 0, q,
                                       scales, tensor_scale, nullptr);
  if (rc != FP4Q_OK) return rc;
  if (k < 0 || k > cols || ldx % 8 != 0) return FP4Q_ERR_INVALID;
  if (k > 0 && (!chan_out || !aligned(chan_out, 4))) return FP4Q_ERR_INVALID;
  if (rows > 0 && k > 0 && (!resid_out || !aligned(resid_out, 2))) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!aligned(x, 16) || !aligned(q, 4))) return FP4Q_ERR_INVALID;
  if (cols > INT32_MAX || rows * (int64_t)k >= ((int64_t)1 << 31)) return FP4Q_ERR_UNSUPPORTED;
  const size_t need = fp4q_quantize_select_workspace_bytes(fmt, layout, rows, cols);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return FP4Q_ERR_WORKSPACE;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  const bool tiled = layout == FP4Q_LAYOUT_TILED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  void* wsq = workspace;
  void* wss = static_cast<char*>(workspace) +
              round256_sz(fp4q_quantize_workspace_bytes(fmt, rows, cols, 1));
  if (k > 0 && rows > 0 && cols % 32 == 0) {
    const int64_t bands = fp4q::launch_quantize_scored(fmt, tiled, x, rows, cols, ldx, q, scales,
                                                       tensor_scale, wsq,
                                                       static_cast<uint16_t*>(wss), st);
    fp4q::launch_select_scored(fmt, tiled, x, rows, cols, ldx, q, scales, tensor_scale, k,
                               chan_out, resid_out, static_cast<const uint16_t*>(wss), bands, wss,
                               st);
  } else {
    fp4q::launch_quantize(fmt, tiled, x, rows, cols, ldx, nullptr, 1, nullptr, 0, q, scales,
                          tensor_scale, nullptr, wsq, st);
    if (k > 0)
      fp4q::launch_select(fmt, tiled, x, rows, cols, ldx, q, scales, tensor_scale, k, chan_out,
                          resid_out, wss, st);
  }
  return check_launch();
}

size_t fp4q_select_channels_grouped_workspace_bytes(int64_t rows, int64_t cols,
                                                    int32_t num_groups) {
  return fp4q::select_grouped_workspace_bytes(rows, cols, num_groups);
}

int fp4q_select_channels_grouped(fp4q_format_t fmt, const uint16_t* x, int64_t rows, int64_t cols,
                                 int64_t ldx, const int32_t* group_offsets, int32_t num_groups,
                                 const uint8_t* q, const uint8_t* scales,
                                 const float* tensor_scale, int32_t k, int32_t* chan_out,
                                 uint16_t* resid_out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!fmt_ok(fmt)) return FP4Q_ERR_INVALID;
  if (rows < 0 || cols <= 0 || cols % blk_of(fmt) != 0 || ldx < cols || ldx % 8 != 0)
    return FP4Q_ERR_INVALID;
  if (k < 0 || k > cols) return FP4Q_ERR_INVALID;
  if (num_groups < 1 || !group_offsets) return FP4Q_ERR_INVALID;
  if (num_groups > MAX_GROUPS) return FP4Q_ERR_UNSUPPORTED;
  if (fmt == FP4Q_NVFP4 && !tensor_scale) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_MXFP4 && tensor_scale) return FP4Q_ERR_INVALID;
  if (k > 0 && (!chan_out || !aligned(chan_out, 4))) return FP4Q_ERR_INVALID;
  if (rows > 0 && k > 0 && (!resid_out || !aligned(resid_out, 2))) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!x || !q || !scales)) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!aligned(x, 16) || !aligned(q, 4))) return FP4Q_ERR_INVALID;
  if (!fp4q::select_grouped_cols_ok(cols)) return FP4Q_ERR_UNSUPPORTED;
  if (rows * (int64_t)k >= ((int64_t)1 << 31)) return FP4Q_ERR_UNSUPPORTED;
  if (k == 0) return FP4Q_OK;
  const size_t need = fp4q::select_grouped_workspace_bytes(rows, cols, num_groups);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return FP4Q_ERR_WORKSPACE;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_select_grouped(fmt, x, rows, cols, ldx, q, scales, tensor_scale, group_offsets,
                              num_groups, k, chan_out, resid_out, workspace,
                              static_cast<hipStream_t>(stream));
  return check_launch();
}

int fp4q_permute_quantized(fp4q_format_t fmt, const uint16_t* x, int64_t tokens, int64_t cols,
                           int64_t ldx, const uint8_t* q, const uint8_t* scales,
                           const float* tensor_scale, const int32_t* row_src, int64_t rows,
                           const int32_t* group_offsets, int32_t num_groups,
                           const int32_t* chan_idx, int32_t n_chan, uint8_t* q_out,
                           uint8_t* scales_out, float* tensor_scale_out, uint16_t* resid_out,
                           void* stream) {
  if (!fmt_ok(fmt)) return FP4Q_ERR_INVALID;
  if (tokens < 0 || rows < 0 || cols <= 0 || cols % blk_of(fmt) != 0) return FP4Q_ERR_INVALID;
  if (rows > 0 && tokens == 0) return FP4Q_ERR_INVALID;
  if (num_groups < 1 || !group_offsets) return FP4Q_ERR_INVALID;
  if (n_chan < 0 || n_chan > cols) return FP4Q_ERR_INVALID;
  if ((n_chan > 0) != (chan_idx != nullptr) || (n_chan > 0) != (resid_out != nullptr))
    return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_NVFP4 && (!tensor_scale || !tensor_scale_out)) return FP4Q_ERR_INVALID;
  if (fmt == FP4Q_MXFP4 && (tensor_scale || tensor_scale_out)) return FP4Q_ERR_INVALID;
  // q_out and scales_out both NULL: the residual (and tensor scales) only,
  // for a grouped GEMM that gathers the codes itself
  if ((q_out == nullptr) != (scales_out == nullptr)) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!row_src || !q || !scales)) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!aligned(q, 8) || !aligned(q_out, 8))) return FP4Q_ERR_INVALID;
  if (rows > 0 && n_chan > 0 && (!x || !aligned(x, 2) || ldx < cols)) return FP4Q_ERR_INVALID;
  if (rows >= ((int64_t)1 << 31) || cols >= ((int64_t)1 << 30) || num_groups > MAX_GROUPS)
    return FP4Q_ERR_UNSUPPORTED;
  if (rows == 0 && fmt == FP4Q_MXFP4) return FP4Q_OK;  // no rows and no tensor scales to copy
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_permute(fmt, x, ldx, tokens, cols, q, scales, tensor_scale, row_src, rows,
                       group_offsets, num_groups, chan_idx, n_chan, q_out, scales_out,
                       tensor_scale_out, resid_out, static_cast<hipStream_t>(stream));
  return check_launch();
}

size_t fp4q_error_decompose_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0) return 0;
  return fp4q::decompose_workspace_bytes(rows, cols);
}

int fp4q_error_decompose(fp4q_format_t fmt, const uint16_t* x, int64_t rows, int64_t cols,
                         int64_t ldx, fp4q_err_stats_t* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!fmt_ok(fmt)) return FP4Q_ERR_INVALID;
  if (rows < 0 || cols <= 0 || cols % blk_of(fmt) != 0 || ldx < cols || ldx % 8 != 0)
    return FP4Q_ERR_INVALID;
  if (!out || !aligned(out, 8)) return FP4Q_ERR_INVALID;
  if (rows > 0 && (!x || !aligned(x, 16))) return FP4Q_ERR_INVALID;
  const size_t need = fp4q::decompose_workspace_bytes(rows, cols);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return FP4Q_ERR_WORKSPACE;
  if (injected_failure()) return FP4Q_ERR_HIP;
  clear_error();
  fp4q::launch_decompose(fmt, x, rows, cols, ldx, out, workspace,
                         static_cast<hipStream_t>(stream));
  return check_launch();
}

}  // extern "C"
