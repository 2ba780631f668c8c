/*
 * fp4q.h -- C ABI of libfp4q: block-scaled FP4 (NVFP4 / MXFP4) activation
 * quantization, the W4A4 GEMM with fused sparse residual compensation, its
 * expert-grouped (MoE) form, and the exact three-way MXFP4 error
 * decomposition, on AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages:
 *  - "QUADS: Stabilizing NVFP4 Reinforcement Learning for MoE via
 *    QUantization-error Alignment across Dual Sides", abstract: NVFP4 combines
 *    fine-grained scaling with native W4A4 FP4 GEMMs; activations are
 *    re-quantized online every forward pass; Residual Activation
 *    Compensation corrects high-error activation channels while keeping the
 *    W4A4 GEMM native; weights share one quantize-dequantize path.
 *  - its German explainer (gist.science), section 2.2 B: a residual term on
 *    selected channels is added to the quantized output.
 *  - "FourSight: Stable FP4 RL Post-Training via Sequence Filtering and Sparse
 *    Channel Compensation", abstract: a few top-variance activation channels
 *    are kept in BF16 inside an otherwise NVFP4 GEMM.
 *  - "Decomposing MXFP4 quantization error for LLM reinforcement learning",
 *    abstract: MXFP4 error = scale bias + deadzone truncation + grid noise,
 *    exactly.
 *
 * Formats (the pages name them; block sizes and encodings are the reading
 * this library implements):
 *  - element: E2M1, magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3;
 *    round to nearest, ties to the even mantissa bit, saturating at 6; the
 *    sign bit is the input's sign bit (so -0 gives code 0x8).
 *  - NVFP4: 16-element blocks along the contiguous dimension; block scale
 *    E4M3 (bias 7, largest 448, satfinite, nearest-even) of
 *    (block_amax / 6) / t, where t = tensor_amax / 2688 (FP32; t = 1 when
 *    the amax is 0); element = e2m1(x / (scale * t)).
 *  - MXFP4: 32-element blocks; scale 2^e with the smallest e in [-127, 127]
 *    such that 6 * 2^e >= block_amax, stored as E8M0 code e + 127;
 *    element = e2m1(x * 2^-e).  No tensor scale.
 *  - packing: two codes per byte, even element in the low nibble.
 *
 * Packed operand layouts (codes and block scales; chosen per call):
 *  - FP4Q_LAYOUT_ROWMAJOR: codes u8 [rows, cols/2], scales u8 [rows, cols/blk].
 *  - FP4Q_LAYOUT_TILED (cols % 128 == 0): the GEMM's native layout.  Codes
 *    are 1 KB blocks, one per (16-row group G, 128-column step k), block
 *    (G, k) at byte (G * cols/128 + k) * 1024; inside it the 16 bytes of row
 *    16G + r, step bytes [16c, 16c + 16) (c = 0..3), sit at (c*16 + r)*16.
 *    Scales are blocks per (64-row group H, step k) at
 *    (H * cols/128 + k) * (64 * 128/blk): NVFP4 (512 bytes) holds scale byte
 *    8k + 4d + e of row 64H + r at (d*64 + r)*4 + e; MXFP4 (256 bytes) holds
 *    byte 4k + e of row 64H + r at r*4 + e.  Rows are padded up to a
 *    multiple of 16 (codes) and 64 (scales); fp4q_packed_bytes() gives the
 *    sizes.  A GEMM load of 16 rows x 64 bytes, or of 64 rows' scales, is
 *    then one contiguous span: on MI355X that streams operand tiles about
 *    2.7x faster than rows 2 KB apart.  The contents of padding rows are
 *    never used in a result.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing.  Its host state is a thread-local last error and
 *    the test hooks (fp4q_test_hook).  Its only device state is the static
 *    scratch array of fp4q_quantize_noalloc (32 KiB per device, below).
 *    What a kernel carries from one call to the next otherwise (the
 *    small-tensor NVFP4 quantizer's exchange slots, see fp4q_quantize)
 *    lives in the caller's workspace, so calls with different workspaces
 *    are independent on any streams, and calls sharing a workspace must
 *    not overlap (as for any buffer a call writes).
 *  - Every call is asynchronous on the caller's HIP stream (passed as void*,
 *    NULL = default stream); results are ready when that stream is.
 *  - Unpacked tensors are row-major; FP4 blocks run along the contiguous
 *    (K) dimension.  Weights are passed transposed, W^T [N, K].
 *  - Arguments are validated on the host before any HIP call; device-side
 *    contents are preconditions and are NOT checked (doing so would need a
 *    synchronisation): channel lists ascending, unique and < K; group
 *    offsets non-decreasing with offsets[0] = 0 and offsets[G] = rows;
 *    inputs finite; dequantized products within FP32 range.
 *  - No C++ exception crosses the ABI.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FP4Q_NVFP4 = 0, FP4Q_MXFP4 = 1 } fp4q_format_t;
typedef enum { FP4Q_OUT_F32 = 0, FP4Q_OUT_BF16 = 1 } fp4q_dtype_t;
typedef enum { FP4Q_LAYOUT_ROWMAJOR = 0, FP4Q_LAYOUT_TILED = 1 } fp4q_layout_t;

/* Status codes. */
#define FP4Q_OK 0
#define FP4Q_ERR_INVALID (-1)     /* null pointer with non-zero size, bad enum, bad shape or stride, misaligned pointer */
#define FP4Q_ERR_UNSUPPORTED (-2) /* a valid shape the kernels do not take (e.g. K not a multiple of 128 in a GEMM) */
#define FP4Q_ERR_WORKSPACE (-3)   /* workspace missing or smaller than the *_workspace_bytes query */
#define FP4Q_ERR_HIP (-4)         /* a HIP call failed; fp4q_last_hip_error() returns its hipError_t */

/* Message for a status code (static storage). */
const char* fp4q_status_str(int status);

/* hipError_t of the last FP4Q_ERR_HIP on the calling thread (0 if none). */
int fp4q_last_hip_error(void);

/* Bytes of the packed codes and block scales of a [rows, cols] tensor in a
 * layout (rows padded as the tiled layout requires).  Returns FP4Q_OK, or
 * FP4Q_ERR_INVALID for a bad enum, negative rows, cols not a multiple of the
 * block size, or a tiled layout with cols % 128 != 0. */
int fp4q_packed_bytes(fp4q_format_t fmt, fp4q_layout_t layout, int64_t rows, int64_t cols,
                      size_t* code_bytes, size_t* scale_bytes);

/* ------------------------------------------------------------------------
 * Activation (or weight) quantization.  QUADS abstract: activations are
 * quantized online each forward pass (weights go through the same path once
 * per weight sync, with n_chan = 0); QUADS explainer section 2.2 B /
 * FourSight abstract: the residual of the selected channels is kept.
 *
 *   x             bf16 [rows, cols], row stride ldx elements (ldx >= cols,
 *                 ldx % 8 == 0, x 16-byte aligned)
 *   group_offsets device int32 [num_groups + 1] row ranges, one quantization
 *                 group each (own tensor scale and channel list); NULL with
 *                 num_groups == 1 means one group of all rows
 *   chan_idx      device int32 [num_groups, n_chan]: channels (columns) whose
 *                 residual is emitted, ascending per group; NULL iff n_chan == 0
 *   layout        layout of q and scales (see above); FP4Q_LAYOUT_TILED needs
 *                 cols % 128 == 0 and buffers of fp4q_packed_bytes()
 *   q             out packed codes (16-byte aligned), u8 [rows, cols/2]
 *                 when row-major
 *   scales        out block scale codes (blk 16 / 32; 4-byte aligned),
 *                 u8 [rows, cols/blk] when row-major
 *   tensor_scale  out f32 [num_groups] (NVFP4; must be NULL for MXFP4);
 *                 empty groups get 1.0
 *   resid         out bf16 [rows, n_chan]: bf16_rne(x - deq(code)) at
 *                 column chan_idx[g][j]; deq = (e2m1 * scale) * t in FP32
 *                 (NVFP4) or e2m1 * 2^e (MXFP4); NULL iff n_chan == 0
 *   workspace     device scratch of fp4q_quantize_workspace_bytes() bytes,
 *                 8-byte aligned (NVFP4 only; may be NULL when that is 0).
 *                 Its first 512 bytes hold the small-tensor path's exchange
 *                 state (below): ZERO-FILL the workspace once before its
 *                 first use; the library keeps it consistent from then on,
 *                 so do not write to it between calls.  The rest is scratch
 *                 left undefined.
 *
 * cols must be a multiple of the block size; 0 <= n_chan <= cols.
 * rows * cols / 8 must be below 2^31 (FP4Q_ERR_UNSUPPORTED otherwise: 32 GiB
 * of BF16 per call).
 *
 * Small NVFP4 tensors (one group, at most 131,072 elements, the tiled
 * layout counting its rows padded to 16) take one launch whose workgroups
 * exchange the tensor maximum through slots in the workspace, tagged by a
 * launch counter kept beside them.  The exchange waits a bounded time; a
 * workgroup whose wait runs out (it cannot happen while every workgroup of
 * the launch runs; the test hooks force it) poisons what it writes: block
 * scales 0x7F (E4M3 NaN), residuals BF16 NaN, and a NaN tensor scale when
 * it is workgroup 0, so a GEMM on the result gives NaN, never a silent
 * wrong value; it also sets FP4Q_QSTATUS_GRID_EXPIRED in the workspace's
 * status word, which fp4q_quantize_status() returns.
 * ------------------------------------------------------------------------ */
size_t fp4q_quantize_workspace_bytes(fp4q_format_t fmt, int64_t rows, int64_t cols,
                                     int32_t num_groups);

int fp4q_quantize(fp4q_format_t fmt, fp4q_layout_t layout, const uint16_t* x, int64_t rows,
                  int64_t cols, int64_t ldx, const int32_t* group_offsets, int32_t num_groups,
                  const int32_t* chan_idx, int32_t n_chan, uint8_t* q, uint8_t* scales,
                  float* tensor_scale, uint16_t* resid, void* workspace, size_t workspace_bytes,
                  void* stream);

/* ------------------------------------------------------------------------
 * Outlier Fallback ("Decomposing MXFP4 quantization error ...", abstract:
 * the fallback recovers the deadzone entries).  Reading: the entries the
 * quantizer sends to zero (code magnitude 0: the deadzone set of the
 * three-way split, and exact zeros) keep their own BF16 value; every other
 * entry is dequantized from fp4q_quantize's code and block scale (one
 * group).  The fallback is the element-sparse counterpart of the channel
 * compensation; this call materialises the dequantized tensor with it:
 *
 *   y[r, c] = x[r, c]              where the code magnitude is 0
 *   y[r, c] = (e2m1 * sb) * t      (NVFP4; FP32, the residual's value)
 *   y[r, c] = e2m1 * 2^e           (MXFP4; exact)
 *
 *   x           bf16 [rows, cols], ldx as for fp4q_quantize
 *   y           out f32 [rows, ldy] (16-byte aligned, ldy % 4 == 0)
 *   n_fallback  out device int64 [1] (8-byte aligned) or NULL: the number
 *               of non-zero entries that fell back (the deadzone count)
 *   workspace   device scratch of fp4q_qdq_fallback_workspace_bytes()
 *               bytes (NVFP4 only; 8-byte aligned), left undefined
 * Errors as fp4q_quantize.
 * ------------------------------------------------------------------------ */
size_t fp4q_qdq_fallback_workspace_bytes(fp4q_format_t fmt, int64_t rows, int64_t cols);

int fp4q_qdq_fallback(fp4q_format_t fmt, const uint16_t* x, int64_t rows, int64_t cols,
                      int64_t ldx, float* y, int64_t ldy, int64_t* n_fallback, void* workspace,
                      size_t workspace_bytes, void* stream);

/* fp4q_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, results and errors without the workspace, which is a
 * static device array of the library instead (32 KiB per GPU, held until
 * the process ends, zero at load).  It allocates nothing and calls no
 * allocating routine.  Limits: NVFP4 with at most 8,064 groups
 * (FP4Q_ERR_UNSUPPORTED beyond); MXFP4 needs no scratch.  Every call on a
 * GPU shares that GPU's array, so calls that overlap on one GPU (other
 * streams, parallel graph branches) race; calls on one stream are fine.
 * FP4Q_ERR_HIP also when the array's device address cannot be found. */
int fp4q_quantize_noalloc(fp4q_format_t fmt, fp4q_layout_t layout, const uint16_t* x,
                          int64_t rows, int64_t cols, int64_t ldx, const int32_t* group_offsets,
                          int32_t num_groups, const int32_t* chan_idx, int32_t n_chan, uint8_t* q,
                          uint8_t* scales, float* tensor_scale, uint16_t* resid, void* stream);

/* Status of the quantize calls that used an NVFP4 workspace since the last
 * query: waits for `stream` (the caller's stream of those calls), reads the
 * workspace's status word into *status and clears it.  Bits:
 * FP4Q_QSTATUS_GRID_EXPIRED (the small-tensor exchange ran out of time; the
 * outputs of that call are NaN-poisoned).  0 means every such call found
 * its tensor maximum.  Errors: FP4Q_ERR_INVALID (status NULL),
 * FP4Q_ERR_WORKSPACE (workspace NULL, misaligned or smaller than an NVFP4
 * workspace), FP4Q_ERR_HIP. */
#define FP4Q_QSTATUS_GRID_EXPIRED 1
int fp4q_quantize_status(const void* workspace, size_t workspace_bytes, int32_t* status,
                         void* stream);

/* Test hooks (failure injection for the error paths; not for production
 * use, and not synchronised with calls running on other threads):
 *   FP4Q_HOOK_RESET              all hooks off (value ignored)
 *   FP4Q_HOOK_FAIL_NEXT_LAUNCH   the next entry point that passes its
 *                                argument checks returns FP4Q_ERR_HIP
 *                                WITHOUT launching anything, with
 *                                fp4q_last_hip_error() = value (> 0)
 *   FP4Q_HOOK_GRID_SPIN_LIMIT    spin limit of the small-tensor NVFP4
 *                                exchange (0 = the default 2^22 loads)
 *   FP4Q_HOOK_GRID_SKIP_SLOT     that workgroup of the small-tensor NVFP4
 *                                launches skips its slot store (-1 = none),
 *                                so the others' waits run out
 * Returns FP4Q_OK, or FP4Q_ERR_INVALID for an unknown hook or value. */
#define FP4Q_HOOK_RESET 0
#define FP4Q_HOOK_FAIL_NEXT_LAUNCH 1
#define FP4Q_HOOK_GRID_SPIN_LIMIT 2
#define FP4Q_HOOK_GRID_SKIP_SLOT 3
int fp4q_test_hook(int32_t hook, int64_t value);

/* ------------------------------------------------------------------------
 * Compensated W4A4 GEMM.  QUADS abstract (native W4A4 FP4 GEMM plus
 * Residual Activation Compensation on high-error channels), explainer
 * section 2.2 B (residual term added to the quantized output), FourSight
 * abstract (sparse BF16 channels spliced into the NVFP4 GEMM):
 *
 *   Y[m, n] = sum_k A[m, k] * B[n, k] + sum_j R[m, j] * B[n, S_j]
 *
 * with A = deq(a_q, a_s, a_ts) [M, K], B = deq(b_q, b_s, b_ts) [N, K]
 * (weights as W^T) and S = chan_idx.  Accumulation is FP32 (MFMA); the
 * result equals the exact sum within (K + n_chan) * 2^-23 * sum|terms|.
 *
 *   layout     layout of both operands' codes and scales (see above)
 *   a_q, a_s   packed activations and scales, [M, K/2], [M, K/blk] when
 *              row-major (codes 16-byte, scales 8-byte aligned)
 *   a_ts       device f32 [1] tensor scale (NVFP4), NULL for MXFP4
 *   b_q, b_s   packed W^T, [N, K/2], [N, K/blk] when row-major (same alignment)
 *   b_ts       device f32 [1] (NVFP4), NULL for MXFP4
 *   chan_idx   device int32 [n_chan] ascending, < K; resid bf16 [M, n_chan],
 *              16-byte aligned (both NULL iff n_chan == 0)
 *   y          out [M, ldy] f32 or bf16 (nearest-even), ldy >= N
 *   workspace  device scratch of fp4q_gemm_workspace_bytes() bytes, 16-byte
 *              aligned (may be NULL when that is 0); it receives the gathered
 *              compensation weights B[n, S_j] as BF16 and is left undefined
 *
 * K must be a multiple of 128 (FP4Q_ERR_UNSUPPORTED otherwise).
 * FP4Q_ERR_WORKSPACE if a needed workspace is missing, small or misaligned.
 * ------------------------------------------------------------------------ */
size_t fp4q_gemm_workspace_bytes(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M, int64_t N,
                                 int64_t K, int32_t n_chan);

int fp4q_gemm(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M, int64_t N, int64_t K,
              const uint8_t* a_q, const uint8_t* a_s, const float* a_ts, const uint8_t* b_q,
              const uint8_t* b_s, const float* b_ts, const int32_t* chan_idx, int32_t n_chan,
              const uint16_t* resid, void* y, fp4q_dtype_t y_dtype, int64_t ldy, void* workspace,
              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Prepared compensation weights.  The compensation term of fp4q_gemm
 * multiplies R by the dequantized weights on the selected channels,
 * B[n, S_j] (QUADS abstract: Residual Activation Compensation; FourSight
 * abstract: the selected channels effectively BF16).  With static weights
 * and a fixed channel list that slice is itself static:
 * fp4q_comp_weights writes it once, and fp4q_gemm_prepared streams it
 * instead of gathering it from the packed weights on every call.
 *
 * fp4q_comp_weights:
 *   b_q, b_s   packed W^T and block scales in `layout`, as for fp4q_gemm
 *   chan_idx   device int32 [n_chan] ascending, < K (NULL iff n_chan == 0)
 *   out        device buffer of fp4q_comp_weights_bytes() bytes, 16-byte
 *              aligned, owned by the caller.  Layout: 1 KB blocks, block
 *              (c, g) at (g * ceil(n_chan/32) + c) * 1024 for columns
 *              16g .. 16g+15 and channels 32c .. 32c+31; in a block, the 16
 *              bytes of channels 8u .. 8u+7 of column 16g + r at
 *              (16u + r) * 16, each the BF16 of e2m1 * block scale (exact,
 *              tensor scale excluded); entries past n_chan or N are zero.
 * N == 0 or n_chan == 0 writes nothing.  K % 128 != 0 is
 * FP4Q_ERR_UNSUPPORTED; out_bytes below the size is FP4Q_ERR_WORKSPACE.
 *
 * fp4q_gemm_prepared: fp4q_gemm's product with comp_w =
 * fp4q_comp_weights(fmt, layout, N, K, b_q, b_s, chan_idx, n_chan) of the
 * same operands (comp_w is read, not checked against them).  It needs no
 * workspace.  Shapes served by the general kernel (neither the decode form,
 * M <= 64 and n_chan <= 64, nor the 256-tile form) take the term from
 * chan_idx as fp4q_gemm does.  FP4Q_ERR_WORKSPACE if comp_w is missing,
 * small or misaligned when there is a term.
 * ------------------------------------------------------------------------ */
size_t fp4q_comp_weights_bytes(fp4q_format_t fmt, fp4q_layout_t layout, int64_t N, int64_t K,
                               int32_t n_chan);

int fp4q_comp_weights(fp4q_format_t fmt, fp4q_layout_t layout, int64_t N, int64_t K,
                      const uint8_t* b_q, const uint8_t* b_s, const int32_t* chan_idx,
                      int32_t n_chan, uint8_t* out, size_t out_bytes, void* stream);

int fp4q_gemm_prepared(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M, int64_t N, int64_t K,
                       const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                       const uint8_t* b_q, const uint8_t* b_s, const float* b_ts,
                       const int32_t* chan_idx, int32_t n_chan, const uint16_t* resid,
                       const uint8_t* comp_w, size_t comp_w_bytes, void* y,
                       fp4q_dtype_t y_dtype, int64_t ldy, void* stream);

/* Grouped forms, for fp4q_grouped_gemm's weights (w_layout as there, its
 * channels at chan_idx + g n_chan): the groups' blocks one after another,
 * group g's at g * fp4q_comp_weights_bytes(fmt, ROWMAJOR, N, K, n_chan)
 * (the same bytes for either weight layout).
 * fp4q_grouped_gemm_prepared is fp4q_grouped_gemm streaming them (no
 * workspace); with N < 256 (the general grouped kernel, row-major weights
 * only) the term comes from chan_idx.  Errors as the dense forms and
 * fp4q_grouped_gemm; more than 2048 groups is FP4Q_ERR_UNSUPPORTED. */
size_t fp4q_grouped_comp_weights_bytes(fp4q_format_t fmt, int64_t N, int64_t K,
                                       int32_t num_groups, int32_t n_chan);

int fp4q_grouped_comp_weights(fp4q_format_t fmt, fp4q_layout_t w_layout, int64_t N, int64_t K,
                              int32_t num_groups, const uint8_t* b_q, const uint8_t* b_s,
                              const int32_t* chan_idx, int32_t n_chan, uint8_t* out,
                              size_t out_bytes, void* stream);

int fp4q_grouped_gemm_prepared(fp4q_format_t fmt, fp4q_layout_t w_layout, int64_t total_rows,
                               int64_t N, int64_t K, const int32_t* group_offsets,
                               int32_t num_groups,
                               const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                               const uint8_t* b_q, const uint8_t* b_s, const float* b_ts,
                               const int32_t* chan_idx, int32_t n_chan, const uint16_t* resid,
                               const uint8_t* comp_w, size_t comp_w_bytes, void* y,
                               fp4q_dtype_t y_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Fused decode datapath (FourSight abstract: a fused kernel with separate
 * prefill and decode datapaths).  For decode shapes the activation
 * quantization moves into the GEMM: fp4q_gemm_prepared's product, with the
 * activations given as BF16 and quantized inside the kernel exactly as
 * fp4q_quantize(NVFP4, one group, channel list chan_idx) would:
 *
 *   Y = deq(Q(x)) deq(B)^T + R B_S,  R = the residual of x on chan_idx
 *
 *   x          bf16 [M, K], row stride ldx (ldx >= K, ldx % 8 == 0, 16-byte
 *              aligned)
 *   b_q, b_s, b_ts, layout   packed W^T as for fp4q_gemm (the layout is the
 *              weights'; nothing activation-side is packed)
 *   chan_idx, n_chan, comp_w, comp_w_bytes   as for fp4q_gemm_prepared
 *              (comp_w from fp4q_comp_weights of the same weights; unused
 *              when n_chan == 0)
 *   y, y_dtype, ldy   as for fp4q_gemm
 *   a_q_out, a_s_out, a_ts_out, resid_out   optional (all NULL, or all set;
 *              resid_out only with channels): the quantized activations,
 *              row-major [M, K/2] codes (16-byte aligned), [M, K/16]
 *              scales, the tensor scale, bf16 [M, n_chan] residual -- the
 *              values the kernel multiplied, for checking against
 *              fp4q_quantize
 *
 * NVFP4 only; M <= 64, K a multiple of 128 up to 2048, n_chan <= 64
 * (FP4Q_ERR_UNSUPPORTED otherwise).  Every workgroup reads all of x (at
 * most 256 KB, from the caches); each of its 8 waves quantizes the two K
 * steps it multiplies, and the tensor maximum is reduced inside the
 * workgroup, so no launch or grid-wide exchange precedes the GEMM.  The
 * price is that every workgroup quantizes all of x: on MI355X at
 * 64 x 2048 x 11008 this call takes about 56 us against about 16 us for
 * fp4q_quantize followed by fp4q_gemm_prepared, so the two-launch path is
 * the faster one there.
 * ------------------------------------------------------------------------ */
int fp4q_gemm_decode_fused(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M, int64_t N,
                           int64_t K, const uint16_t* x, int64_t ldx, const uint8_t* b_q,
                           const uint8_t* b_s, const float* b_ts, const int32_t* chan_idx,
                           int32_t n_chan, const uint8_t* comp_w, size_t comp_w_bytes, void* y,
                           fp4q_dtype_t y_dtype, int64_t ldy, uint8_t* a_q_out,
                           uint8_t* a_s_out, float* a_ts_out, uint16_t* resid_out,
                           void* stream);

/* ------------------------------------------------------------------------
 * Compensated W4A4 GEMM with a second-pass FP4 residual.  Explainer of the
 * QUADS paper, section 2.2 B: the high-residual channels are quantized a
 * second time and that correction term is added to the quantized output.
 * The residual R [M, n_chan] of the selected channels is itself quantized
 * by fp4q_quantize (same format, row-major layout, blocks along the channel
 * index j, NVFP4 with its own tensor scale), and
 *
 *   Y[m, n] = sum_k A[m, k] * B[n, k] + sum_j deq(R_q)[m, j] * B[n, S_j]
 *
 * Arguments as fp4q_gemm, except the residual:
 *   r_q, r_s   FP4 residual from fp4q_quantize(ROWMAJOR) of R: [M, n_chan/2]
 *              codes, [M, n_chan/blk] block scales (NULL iff n_chan == 0)
 *   r_ts       device f32 [1] its tensor scale (NVFP4), NULL for MXFP4
 *   workspace  device scratch of fp4q_gemm_residual_fp4_workspace_bytes()
 *              bytes, 16-byte aligned: it receives deq(R_q) / r_ts as BF16
 *              (exact: e2m1 times a block scale has at most 6 significant
 *              bits) and then serves the GEMM as fp4q_gemm's workspace
 *
 * n_chan must be a multiple of the block size (16 NVFP4, 32 MXFP4), else
 * FP4Q_ERR_INVALID.  Residual values must stay below 2^125 in magnitude (the
 * largest MXFP4 block scale times 6 is outside BF16).  The tensor scale
 * enters as y = t_w ((t_x / r_ts) main + comp) * r_ts, which differs from
 * the exact sum by a few FP32 roundings of the main term.
 * ------------------------------------------------------------------------ */
size_t fp4q_gemm_residual_fp4_workspace_bytes(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M,
                                              int64_t N, int64_t K, int32_t n_chan);

int fp4q_gemm_residual_fp4(fp4q_format_t fmt, fp4q_layout_t layout, int64_t M, int64_t N,
                           int64_t K, const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                           const uint8_t* b_q, const uint8_t* b_s, const float* b_ts,
                           const int32_t* chan_idx, int32_t n_chan, const uint8_t* r_q,
                           const uint8_t* r_s, const float* r_ts, void* y, fp4q_dtype_t y_dtype,
                           int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/* Grouped form (QUADS abstract: NVFP4 rollout for MoE; explainer section
 * 2.2 B): per group g (rows group_offsets[g] .. group_offsets[g+1]) the
 * dense form above with the group's weights, tensor scales and channel
 * list, and the group's residual quantized with its own tensor scale:
 * r_q, r_s from fp4q_quantize(ROWMAJOR) of R [total_rows, n_chan] with the
 * same group offsets, r_ts device f32 [num_groups] (NVFP4; NULL for MXFP4).
 * Other arguments (w_layout included) as fp4q_grouped_gemm; workspace of
 * fp4q_grouped_gemm_residual_fp4_workspace_bytes() bytes, 16-byte aligned.
 * Errors as the dense form and fp4q_grouped_gemm. */
size_t fp4q_grouped_gemm_residual_fp4_workspace_bytes(fp4q_format_t fmt,
                                                      fp4q_layout_t w_layout,
                                                      int64_t total_rows, int64_t N, int64_t K,
                                                      int32_t num_groups, int32_t n_chan);

int fp4q_grouped_gemm_residual_fp4(fp4q_format_t fmt, fp4q_layout_t w_layout,
                                   int64_t total_rows, int64_t N, int64_t K,
                                   const int32_t* group_offsets, int32_t num_groups,
                                   const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                                   const uint8_t* b_q, const uint8_t* b_s, const float* b_ts,
                                   const int32_t* chan_idx, int32_t n_chan, const uint8_t* r_q,
                                   const uint8_t* r_s, const float* r_ts, void* y,
                                   fp4q_dtype_t y_dtype, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* ------------------------------------------------------------------------
 * Online channel selection.  Explainer of the QUADS paper, section 2.2 B:
 * a binary mask keeps the top-k channels by residual magnitude.  With R the
 * residual fp4q_quantize would emit for a channel,
 * R[m, c] = bf16_rne(x[m, c] - deq(code[m, c])), the magnitude of channel c
 * is max over rows m of |R[m, c]|; the k channels of largest magnitude are
 * chosen (equal magnitudes: the lower index first) and returned ascending,
 * with R on them, ready for fp4q_gemm.
 *
 *   x             bf16 [rows, cols] as quantized (ldx as for fp4q_quantize)
 *   q, scales     fp4q_quantize's codes and block scales of x, in `layout`
 *                 (one quantization group; q 4-byte aligned)
 *   tensor_scale  device f32 [1] from that call (NVFP4), NULL for MXFP4
 *   k             channels to keep, 0 <= k <= cols (k == 0 launches nothing)
 *   chan_out      out device int32 [k], ascending
 *   resid_out     out bf16 [rows, k]: R[m, chan_out[j]] (may be NULL when
 *                 rows == 0)
 *   workspace     device scratch of fp4q_select_channels_workspace_bytes()
 *                 bytes, 16-byte aligned; needs no initialisation and is
 *                 left undefined
 *
 * rows * k must be below 2^31 and cols below 2^31 (FP4Q_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------ */
size_t fp4q_select_channels_workspace_bytes(int64_t rows, int64_t cols);

int fp4q_select_channels(fp4q_format_t fmt, fp4q_layout_t layout, const uint16_t* x,
                         int64_t rows, int64_t cols, int64_t ldx, const uint8_t* q,
                         const uint8_t* scales, const float* tensor_scale, int32_t k,
                         int32_t* chan_out, uint16_t* resid_out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Quantization and online channel selection in one call, the selection's
 * scores taken in the quantizer's own pass over x (the survey's fused
 * form of the QUADS top-k channel mask; explainer section 2.2 B): the
 * results are bit-identical to fp4q_quantize (one group, no channels)
 * followed by fp4q_select_channels with the same k, and x is read once for
 * codes and scores (then again only at the k chosen columns, for R).
 *
 *   fmt, layout, x, rows, cols, ldx   as fp4q_quantize (x 16-byte aligned,
 *                                     ldx a multiple of 8)
 *   k                                 channels to keep, 0 <= k <= cols
 *   q, scales, tensor_scale           out, as fp4q_quantize (q 4-byte aligned)
 *   chan_out, resid_out               out, as fp4q_select_channels
 *   workspace                         device scratch of
 *                                     fp4q_quantize_select_workspace_bytes()
 *                                     bytes, 16-byte aligned; for NVFP4 its
 *                                     first part is the quantize workspace
 *                                     and carries that workspace's state and
 *                                     status word (fp4q_quantize_status)
 *
 * A column count that is not a multiple of 32 takes the two steps one after
 * the other (same results).  Errors as the two calls; k == 0 quantizes only.
 * ------------------------------------------------------------------------ */
size_t fp4q_quantize_select_workspace_bytes(fp4q_format_t fmt, fp4q_layout_t layout,
                                            int64_t rows, int64_t cols);

int fp4q_quantize_select(fp4q_format_t fmt, fp4q_layout_t layout, const uint16_t* x,
                         int64_t rows, int64_t cols, int64_t ldx, int32_t k, uint8_t* q,
                         uint8_t* scales, float* tensor_scale, int32_t* chan_out,
                         uint16_t* resid_out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Grouped form (the MoE layer: QUADS abstract, NVFP4 rollout for MoE;
 * explainer section 2.2 B): each group g (rows group_offsets[g] ..
 * group_offsets[g+1]) chooses its own k channels from its own rows, with
 * its own tensor scale: chan_out [num_groups, k] (ascending per group) and
 * resid_out [rows, k], row r on its group's list.  An empty group has all
 * magnitudes zero and takes channels 0 .. k-1 (the tie rule).
 *   x, q, scales   row-major (fp4q_quantize(ROWMAJOR) with these offsets)
 *   tensor_scale   device f32 [num_groups] (NVFP4), NULL for MXFP4
 *   workspace      fp4q_select_channels_grouped_workspace_bytes() bytes,
 *                  16-byte aligned
 * cols above 30,720 or more than 2048 groups is FP4Q_ERR_UNSUPPORTED;
 * other errors as fp4q_select_channels. */
size_t fp4q_select_channels_grouped_workspace_bytes(int64_t rows, int64_t cols,
                                                    int32_t num_groups);

int fp4q_select_channels_grouped(fp4q_format_t fmt, const uint16_t* x, int64_t rows, int64_t cols,
                                 int64_t ldx, const int32_t* group_offsets, int32_t num_groups,
                                 const uint8_t* q, const uint8_t* scales,
                                 const float* tensor_scale, int32_t k, int32_t* chan_out,
                                 uint16_t* resid_out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ------------------------------------------------------------------------
 * Expert-grouped compensated GEMM (MoE layer; QUADS abstract: NVFP4 rollout
 * for Mixture-of-Experts).  Rows [off[g], off[g+1]) of the permuted
 * activations use expert g's weights, tensor scales and channel list:
 *
 *   w_layout       layout of every expert's weights.  FP4Q_LAYOUT_ROWMAJOR:
 *                  b_q, b_s are [G, N, K/2], [G, N, K/blk].
 *                  FP4Q_LAYOUT_TILED: expert g's codes and scales are
 *                  fp4q_quantize(TILED)'s of its W^T [N, K], at
 *                  b_q + g * code_bytes and b_s + g * scale_bytes with the
 *                  sizes of fp4q_packed_bytes(fmt, TILED, N, K).  Tiled
 *                  weights are served by the 128 x 512 NVFP4 kernel only:
 *                  MXFP4, N < 256 or n_chan % 8 != 0 is
 *                  FP4Q_ERR_UNSUPPORTED.
 *                  On MI355X at the MoE workload (N = 1536 / 2048, K =
 *                  2048 / 768) tiled weights took the two GEMM calls from
 *                  about 540 to 490 us (a stage's 512 weight columns are 32
 *                  contiguous 1 KB blocks instead of 512 rows K/2 apart).
 *   group_offsets  device int32 [G + 1]
 *   a_q, a_s       [total_rows, K/2], [total_rows, K/blk] (row-major)
 *   a_ts           device f32 [G] (NVFP4), NULL for MXFP4
 *   b_q, b_s       every expert's W^T, packed in w_layout
 *   b_ts           device f32 [G] (NVFP4), NULL for MXFP4
 *   chan_idx       device int32 [G, n_chan]; resid bf16 [total_rows, n_chan],
 *                  16-byte aligned
 *   y              out [total_rows, N] (row stride N)
 *   workspace      device scratch of fp4q_grouped_gemm_workspace_bytes()
 *                  bytes, 16-byte aligned (may be NULL when that is 0): the
 *                  gathered compensation weights of every group, as BF16
 *                  (N >= 256: whenever there are channels; the large-tile
 *                  kernels stream them)
 *
 * Empty groups produce nothing.  K must be a multiple of 128.
 * FP4Q_ERR_WORKSPACE if a needed workspace is missing, small or misaligned.
 * ------------------------------------------------------------------------ */
size_t fp4q_grouped_gemm_workspace_bytes(fp4q_format_t fmt, fp4q_layout_t w_layout,
                                         int64_t total_rows, int64_t N, int64_t K,
                                         int32_t num_groups, int32_t n_chan);

int fp4q_grouped_gemm(fp4q_format_t fmt, fp4q_layout_t w_layout, int64_t total_rows, int64_t N,
                      int64_t K, const int32_t* group_offsets, int32_t num_groups,
                      const uint8_t* a_q,
                      const uint8_t* a_s, const float* a_ts, const uint8_t* b_q,
                      const uint8_t* b_s, const float* b_ts, const int32_t* chan_idx,
                      int32_t n_chan, const uint16_t* resid, void* y, fp4q_dtype_t y_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Quantize-before-permute for the expert-grouped layer (QUADS abstract:
 * NVFP4 rollout for Mixture-of-Experts).  The token activations are
 * quantized once by fp4q_quantize (one group, row-major, no channels), and
 * this call builds the expert-ordered operand of fp4q_grouped_gemm from the
 * FP4 codes instead of quantizing every routed copy:
 *
 *   q_out[m] = q[row_src[m]], scales_out[m] = scales[row_src[m]],
 *   resid_out[m, j] = bf16_rne(x[t, c] - deq(code[t, c])), t = row_src[m],
 *                     c = chan_idx[g][j] for the group g holding row m,
 *   tensor_scale_out[g] = tensor_scale[0] for every group (NVFP4)
 *
 * with deq as in fp4q_quantize.  Every expert then sees one tensor scale,
 * that of all the tokens.
 *
 *   x              bf16 token activations [tokens, cols], row stride ldx
 *                  (read only for the residual; may be NULL when n_chan == 0)
 *   q, scales      fp4q_quantize(fmt, ROWMAJOR) of x: [tokens, cols/2],
 *                  [tokens, cols/blk] (q 8-byte aligned)
 *   tensor_scale   device f32 [1] from that call (NVFP4), NULL for MXFP4
 *   row_src        device int32 [rows]: the token of each expert-ordered row
 *   group_offsets  device int32 [num_groups + 1], as for fp4q_grouped_gemm
 *   chan_idx       device int32 [num_groups, n_chan], ascending per group;
 *                  NULL iff n_chan == 0
 *   q_out, scales_out   out [rows, cols/2] (8-byte aligned), [rows, cols/blk];
 *                  both NULL: only the residual and the tensor scales are
 *                  written (fp4q_grouped_gemm_gather then reads the codes
 *                  from the token matrix itself)
 *   tensor_scale_out    out device f32 [num_groups] (NVFP4), NULL for MXFP4
 *   resid_out      out bf16 [rows, n_chan]; NULL iff n_chan == 0
 *
 * Preconditions (not checked on the device): row_src[m] < tokens, offsets
 * as for the grouped GEMM.  Row-major layout only (the grouped GEMM's
 * activations').
 * num_groups <= 2048, rows < 2^31, cols < 2^30 (FP4Q_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------ */
int fp4q_permute_quantized(fp4q_format_t fmt, const uint16_t* x, int64_t tokens, int64_t cols,
                           int64_t ldx, const uint8_t* q, const uint8_t* scales,
                           const float* tensor_scale, const int32_t* row_src, int64_t rows,
                           const int32_t* group_offsets, int32_t num_groups,
                           const int32_t* chan_idx, int32_t n_chan, uint8_t* q_out,
                           uint8_t* scales_out, float* tensor_scale_out, uint16_t* resid_out,
                           void* stream);

/* ------------------------------------------------------------------------
 * Expert-grouped GEMM gathering the token codes (QUADS abstract: NVFP4
 * rollout for Mixture-of-Experts; quantize-before-permute).  The tokens
 * are quantized once (fp4q_quantize, one group, row-major) and every
 * routed row reads its token's codes and block scales straight from that
 * matrix -- no expert-ordered copy of them:
 *
 *   Y[m, n] = sum_k deq(Xq[row_src[m], k]) B_g[n, k] + sum_j R[m, j] B_g[n, S_gj]
 *
 * for m in group g's rows [off[g], off[g+1]).  The residual R [total_rows,
 * n_chan] is the routed rows' (fp4q_permute_quantized with q_out and
 * scales_out NULL writes it, and the per-group tensor scales).
 *
 *   row_src        device int32 [total_rows]: the token of each routed row
 *                  (< tokens; a precondition)
 *   a_q, a_s       the token matrix's codes and scales, row-major
 *                  [tokens, K/2], [tokens, K/blk]
 *   a_ts           device f32 [1] its tensor scale (NVFP4), NULL for MXFP4;
 *                  every group uses it
 *   w_layout, b_*, chan_idx, n_chan   as fp4q_grouped_gemm (tiled weights
 *                  also need tokens * K/2 below 2^32)
 *   resid          bf16 [total_rows, n_chan], 16-byte aligned
 *   comp_w         fp4q_grouped_comp_weights of the weights (needed when
 *                  n_chan > 0), comp_w_bytes its size
 *   y              out [total_rows, N]
 *
 * The large-tile grouped kernels only: N >= 256, K % 128 == 0, n_chan % 8
 * == 0 (FP4Q_ERR_UNSUPPORTED otherwise); more than 2048 groups is
 * FP4Q_ERR_UNSUPPORTED.  The output equals the permuted path's
 * (fp4q_permute_quantized, then fp4q_grouped_gemm_prepared) bit for bit.
 * On MI355X at the MoE workload (32,768 routed rows of 4096 tokens) the
 * gathering gate_up GEMM took about 25 us more than reading the permuted
 * copy (scattered token rows), against about 10 us saved in the permute.
 * ------------------------------------------------------------------------ */
int fp4q_grouped_gemm_gather(fp4q_format_t fmt, fp4q_layout_t w_layout, int64_t total_rows,
                             int64_t N, int64_t K, const int32_t* group_offsets,
                             int32_t num_groups,
                             const int32_t* row_src, int64_t tokens, const uint8_t* a_q,
                             const uint8_t* a_s, const float* a_ts, const uint8_t* b_q,
                             const uint8_t* b_s, const float* b_ts, const int32_t* chan_idx,
                             int32_t n_chan, const uint16_t* resid, const uint8_t* comp_w,
                             size_t comp_w_bytes, void* y, fp4q_dtype_t y_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Exact three-way MXFP4 error decomposition ("Decomposing MXFP4
 * quantization error ...", abstract).  Per 32-block with actual scale
 * s = 2^e and ideal scale s* = amax/6, per element x:
 *   total      = x - Q_s(x)
 *   deadzone   = x               where Q_s(x) = 0, else 0
 *   grid_noise = x - Q*(x)       where Q_s(x) != 0, else 0
 *   scale_bias = Q*(x) - Q_s(x)  where Q_s(x) != 0, else 0
 * Q_s is the MXFP4 quantizer, Q* the same E2M1 rounding with s*.  So
 * total = scale_bias + deadzone + grid_noise element by element, and the
 * exact integer sums below satisfy the identity bit for bit.
 *
 * The same split under the NVFP4 quantizer (16-element blocks): the actual
 * quantization is fp4q_quantize's own (one group): Q_s(x) = g * sb * t with
 * its code g, E4M3 block scale value sb and tensor scale t (the exact
 * product); the ideal scale is again s* = amax/6 of the 16-block.  The sums
 * stay exact while every term (6x, 6 g sb t, g* amax) is a multiple of
 * 2^-136, which holds for a tensor amax of at least 2^-89; below that (and
 * above 0) the kernel sets FP4Q_DEC_INEXACT in `flags`, and the sums may
 * have lost low-order terms.
 * ------------------------------------------------------------------------ */
typedef struct {
    /* 6 * (sum of component c) as a 320-bit two's complement integer in units
     * of 2^-136, 5 little-endian 64-bit limbs; c = 0 total, 1 scale_bias,
     * 2 deadzone, 3 grid_noise */
    int64_t exact[4][5];
    double sum[4];       /* the same sums as doubles (approximate) */
    double sumsq[4];     /* FP64 sums of squared components */
    double cross_sb_gn;  /* FP64 sum of scale_bias * grid_noise */
    int64_t n_elems;     /* rows * cols */
    int64_t n_deadzone;  /* non-zero inputs quantized to zero */
    int64_t n_clipped;   /* |x| > 6 * s: 0 for MXFP4 under its scale rule; for
                            NVFP4 where E4M3 rounded the block scale down */
    int64_t flags;       /* FP4Q_DEC_INEXACT: NVFP4 tensor amax in (0, 2^-89),
                            the exact sums are not guaranteed */
} fp4q_err_stats_t;

#define FP4Q_DEC_INEXACT 1

/*   fmt        FP4Q_MXFP4 or FP4Q_NVFP4
 *   x          bf16 [rows, cols], ldx as for fp4q_quantize; cols a multiple
 *              of the block size (32 MXFP4, 16 NVFP4)
 *   out        DEVICE pointer to one fp4q_err_stats_t (8-byte aligned)
 *   workspace  device scratch of fp4q_error_decompose_workspace_bytes() */
size_t fp4q_error_decompose_workspace_bytes(int64_t rows, int64_t cols);

int fp4q_error_decompose(fp4q_format_t fmt, const uint16_t* x, int64_t rows, int64_t cols,
                         int64_t ldx, fp4q_err_stats_t* out, void* workspace,
                         size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_H */
