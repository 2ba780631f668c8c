// fp4q_internal.h -- declarations shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp4q.h"

namespace fp4q {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

int launch_quantize(int fmt, bool tiled, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                    const int32_t* off, int G, const int32_t* chan, int nS, uint8_t* q,
                    uint8_t* scales, float* tscale, uint16_t* resid, void* ws,
                    hipStream_t stream);

size_t quantize_workspace_bytes(int fmt, int G);

// Outlier Fallback: quantize-dequantize to FP32 with the deadzone entries
// kept (one group, row-major x); count: device int64 or null.  NVFP4 uses
// the quantize workspace's amax words.
int launch_qdq_fallback(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                        float* y, int64_t ldy, int64_t* count, void* ws, hipStream_t stream);

// fp4q_quantize's argument checks other than the workspace (host only), and
// the calling thread's last HIP error (for entry points outside api.hip).
int quantize_checks(int fmt, int layout, const uint16_t* x, int64_t rows, int64_t cols,
                    int64_t ldx, const int32_t* group_offsets, int32_t num_groups,
                    const int32_t* chan_idx, int32_t n_chan, const uint8_t* q,
                    const uint8_t* scales, const float* tensor_scale, const uint16_t* resid);
void set_last_hip_error(int e);

// Status word of a quantize workspace (bit 0: the small-tensor exchange ran
// out of spins); waits for the stream, then reads and clears it.
int quantize_status(const void* ws, hipStream_t stream, uint32_t* status);

// Test hooks of the small-tensor exchange: spin limit (0: default) and a
// workgroup that skips its slot store (-1: none).
void set_grid_hooks(uint32_t spin, int skip);
uint32_t grid_hook_spin();
int grid_hook_skip();

// Dense GEMM kernel choice (a function of the shape only, so that the
// workspace query and the launch agree).
enum GemmPath { PATH_GENERIC = 0, PATH_SKINNY = 1, PATH_BIG = 2 };
GemmPath gemm_path(int64_t M, int64_t N, int64_t K, int nS);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int nS);

// cts: device tensor scale of the compensation term (NVFP4 second-pass
// residual), or null for 1: y = t_w (t_x main + cts comp); grouped: one per
// group, cts[g].
int launch_gemm(int fmt, bool tiled, int64_t M, int64_t N, int64_t K, const int32_t* off, int G,
                const uint8_t* aq, const uint8_t* as, const float* ats, const uint8_t* bq,
                const uint8_t* bs, const float* bts, const int32_t* chan, int nS,
                const uint16_t* resid, const float* cts, void* y, int y_bf16, int64_t ldy,
                void* ws, hipStream_t stream, const uint8_t* bsel_pre = nullptr);

// Second-pass residual: BF16 e2m1 * block scale (exact; tensor scale
// excluded) of the row-major FP4 residual rq [M, nS/2], rs [M, nS/blk].
void launch_deq_resid(int fmt, int64_t M, int nS, const uint8_t* rq, const uint8_t* rs,
                      uint16_t* out, hipStream_t stream);

bool big_gemm_eligible(int64_t M, int64_t N, int64_t K, int nS);
bool big_grouped_eligible(int64_t N, int64_t K, int nS);
size_t big_gemm_workspace_bytes(int64_t N, int nS);
// The large-tile grouped kernels take the compensation weights from the
// prepared array or gather them into the workspace once per call.  wtiled:
// every expert's weights in the tiled layout (NVFP4 only).
size_t grouped_workspace_bytes(int64_t N, int64_t K, int G, int nS);
bool grouped_tiled_ok(int fmt, int64_t N, int64_t K, int nS);
int launch_gemm_big_grouped(int fmt, int64_t total_rows, int64_t N, int64_t K,
                            const int32_t* off, int G, const uint8_t* aq, const uint8_t* as,
                            const float* ats, const uint8_t* bq, const uint8_t* bs,
                            const float* bts, const int32_t* chan, int nS,
                            const uint16_t* resid, const float* cts, const uint8_t* bsel_pre,
                            void* y, int y_bf16, void* ws, hipStream_t stream, bool wtiled,
                            const int32_t* row_src = nullptr, int64_t src_rows = 0);
int launch_gemm_big(int fmt, bool tiled, int64_t M, int64_t N, int64_t K, const uint8_t* aq,
                    const uint8_t* as, const float* ats, const uint8_t* bq, const uint8_t* bs,
                    const float* bts, const int32_t* chan, int nS, const uint16_t* resid,
                    const float* cts, const uint8_t* bsel_pre, void* y, int y_bf16, int64_t ldy,
                    void* ws, hipStream_t stream);
// Compensation weights B[n, S_j] (BF16, tensor scale excluded) in the tiled
// layout the GEMMs stream: 1 KB per 16 columns and 32 channels.
size_t comp_weights_bytes(int64_t N, int nS);
void launch_comp_weights(int fmt, bool tiled, const uint8_t* bq, const uint8_t* bs, int64_t N,
                         int64_t K, const int32_t* chan, int nS, int G, uint8_t* out,
                         hipStream_t stream);

bool skinny_gemm_eligible(int64_t M, int64_t N, int64_t K, int nS);
int launch_gemm_skinny(int fmt, bool tiled, int64_t M, int64_t N, int64_t K, const uint8_t* aq,
                       const uint8_t* as, const float* ats, const uint8_t* bq, const uint8_t* bs,
                       const float* bts, const int32_t* chan, int nS, const uint16_t* resid,
                       const float* cts, const uint8_t* bsel, void* y, int y_bf16, int64_t ldy,
                       hipStream_t stream);

// Fused decode datapath: the activations quantized (NVFP4) inside the decode
// GEMM.  M <= 64, K <= 2048, nS <= 64; bsel = prepared compensation weights
// (null iff nS == 0); q_out etc. optional (all null or all set).
bool decode_fused_eligible(int64_t M, int64_t K, int nS);
int launch_gemm_decode_fused(bool tiled, int64_t M, int64_t N, int64_t K, const uint16_t* x,
                             int64_t ldx, const uint8_t* bq, const uint8_t* bs, const float* bts,
                             const int32_t* chan, int nS, const uint8_t* bsel, void* y, int y_bf16,
                             int64_t ldy, uint8_t* q_out, uint8_t* s_out, float* ts_out,
                             uint16_t* r_out, hipStream_t stream);

// Online channel selection: scores, top-k pick, residual emission.
size_t select_workspace_bytes(int64_t rows, int64_t cols);
void launch_select(int fmt, bool tiled, const uint16_t* x, int64_t rows, int64_t cols,
                   int64_t ldx, const uint8_t* q, const uint8_t* scales, const float* tscale,
                   int k, int32_t* chan, uint16_t* resid, void* ws, hipStream_t stream);
// The fused form: the tile quantizer's scored pass (rows > 0, cols % 32 ==
// 0; score [bands, cols] BF16 bits; returns bands), then steps 2-4 from its
// partial maxima (workspace: select_scored_workspace_bytes, part first).
int64_t launch_quantize_scored(int fmt, bool tiled, const uint16_t* x, int64_t rows, int64_t cols,
                               int64_t ldx, uint8_t* q, uint8_t* scales, float* tscale, void* ws,
                               uint16_t* score, hipStream_t stream);
int64_t quantize_score_bands(bool tiled, int64_t rows, int64_t cols);
size_t select_scored_workspace_bytes(int64_t bands, int64_t cols);
void launch_select_scored(int fmt, bool tiled, const uint16_t* x, int64_t rows, int64_t cols,
                          int64_t ldx, const uint8_t* q, const uint8_t* scales,
                          const float* tscale, int k, int32_t* chan, uint16_t* resid,
                          const uint16_t* part, int64_t bands, void* ws, hipStream_t stream);
// Grouped selection (row-major operands; cols <= 30720): chan [G, k], each
// group's residual rows on its own list.
size_t select_grouped_workspace_bytes(int64_t rows, int64_t cols, int G);
bool select_grouped_cols_ok(int64_t cols);
void launch_select_grouped(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                           const uint8_t* q, const uint8_t* scales, const float* tscale,
                           const int32_t* off, int G, int k, int32_t* chan, uint16_t* resid,
                           void* ws, hipStream_t stream);

// Quantize-before-permute: token codes to expert order, per-group residual.
void launch_permute(int fmt, const uint16_t* x, int64_t ldx, int64_t tokens, int64_t cols,
                    const uint8_t* q, const uint8_t* scales, const float* tscale,
                    const int32_t* row_src, int64_t rows, const int32_t* off, int G,
                    const int32_t* chan, int nS, uint8_t* q_out, uint8_t* s_out, float* ts_out,
                    uint16_t* r_out, hipStream_t stream);

size_t decompose_workspace_bytes(int64_t rows, int64_t cols);
int launch_decompose(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                     fp4q_err_stats_t* out, void* ws, hipStream_t stream);

}  // namespace fp4q
