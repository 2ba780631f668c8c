// permute.hip -- quantize-before-permute for the expert-grouped layer.
//
// QUADS abstract (NVFP4 rollout for Mixture-of-Experts): each token's
// activation row is routed to several experts.  Quantizing the routed copies
// one by one repeats the same work top_k times; here the token matrix is
// quantized once (one tensor scale for all tokens) and the expert-ordered
// operand is built from its FP4 codes, a quarter of the BF16 bytes.  Row m of
// the output copies the codes and block scales of token row_src[m], and the
// residual on the channels of the group holding m is the quantizer's residual
// at that token (the same FP32 operations as the quantizer).
//
// One wave per eight output rows: the code and scale bytes of all eight rows
// are spread over the lanes in the widest units the row lengths allow (16
// bytes for the codes at cols % 32 == 0), four units per lane in flight, and
// one lane per residual channel.
// The group of the first row comes from a binary search of the offsets
// (scalar loads); the following rows step forward from it.
#include "fp4q_device.h"
#include "fp4q_internal.h"

#include <type_traits>

namespace fp4q {

namespace {

constexpr int PM_THREADS = 256;  // four waves

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }
constexpr int PM_ROWS = 8;       // output rows per wave

// Copy the wave's rows (row r of the output from token row tok(r), held by
// lane r of tk) in units of T: the units of all rows are spread over the
// lanes, four per lane in flight.
template <typename T>
__device__ __forceinline__ void copy_rows(const uint8_t* __restrict__ src,
                                          uint8_t* __restrict__ dst, int64_t row_bytes, int tk,
                                          int64_t m0, int nr, int lane) {
  const uint32_t per = (uint32_t)(row_bytes / (int64_t)sizeof(T));  // < 2^27
  const uint32_t total = per * (uint32_t)nr;
  for (uint32_t u0 = 0; u0 < total; u0 += 4 * 64) {
    T v[4];
    int64_t d[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t u = u0 + lane + 64 * k;
      const bool ok = u < total;
      const int r = ok ? (int)(u / per) : 0;
      const int64_t tok = __shfl(tk, r);
      const int64_t i = ok ? (int64_t)(u - (uint32_t)r * per) : 0;
      v[k] = reinterpret_cast<const T*>(src + tok * row_bytes)[i];
      d[k] = ok ? (m0 + r) * per + i : -1;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (d[k] >= 0) reinterpret_cast<T*>(dst)[d[k]] = v[k];
  }
}

// CU, SU: bytes per copy unit of the code rows and of the scale rows.
template <int FMT, int CU, int SU>
__global__ __launch_bounds__(PM_THREADS) void k_permute_rows(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t tokens, int64_t cols,
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ scales,
    const float* __restrict__ tscale, const int32_t* __restrict__ row_src, int64_t rows,
    const int32_t* __restrict__ off, int G, const int32_t* __restrict__ chan, int nS,
    uint8_t* __restrict__ q_out, uint8_t* __restrict__ s_out, float* __restrict__ ts_out,
    uint16_t* __restrict__ r_out) {
  constexpr int BLK = (FMT == FP4Q_NVFP4) ? 16 : 32;
  const int lane = threadIdx.x & 63;
  if (FMT == FP4Q_NVFP4 && blockIdx.x == 0)
    for (int g = threadIdx.x; g < G; g += PM_THREADS) ts_out[g] = tscale[0];
  const int64_t m0 = ((int64_t)blockIdx.x * (PM_THREADS / 64) +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * PM_ROWS;
  if (m0 >= rows) return;
  const int nr = (int)min((int64_t)PM_ROWS, rows - m0);
  const int64_t cb = cols / 2, sb = cols / BLK;

  // the wave's tokens: lane r loads row m0 + r; a row past the end repeats
  // the last one (its copies are not stored).  The clamp keeps every load
  // inside the tokens; row_src is in range by precondition.
  const int tk = (int)min(max((int64_t)row_src[m0 + min(lane, nr - 1)], (int64_t)0), tokens - 1);

  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  typedef typename std::conditional<CU == 16, u32x4v, uint64_t>::type CodeUnit;
  typedef typename std::conditional<SU == 16, u32x4v,
                                    typename std::conditional<SU == 4, uint32_t, uint8_t>::type>::type
      ScaleUnit;
  copy_rows<CodeUnit>(q, q_out, cb, tk, m0, nr, lane);
  copy_rows<ScaleUnit>(scales, s_out, sb, tk, m0, nr, lane);

  if (nS > 0) {
    // group of the first row: the last g with off[g] <= m0 (empty groups
    // before it are skipped); later rows step forward from it
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= m0) lo = mid;
      else hi = mid;
    }
    int grp[PM_ROWS];
#pragma unroll
    for (int r = 0; r < PM_ROWS; ++r) {
      while (lo + 1 < G && off[lo + 1] <= m0 + r) ++lo;
      grp[r] = lo;
    }
    const float t = (FMT == FP4Q_NVFP4) ? tscale[0] : 1.0f;
    for (int j = lane; j < nS; j += 64) {
      uint32_t xv[PM_ROWS], cbt[PM_ROWS], sc[PM_ROWS];
      int64_t c[PM_ROWS];
#pragma unroll
      for (int r = 0; r < PM_ROWS; ++r)
        c[r] = min(max((int64_t)chan[(int64_t)grp[r] * nS + j], (int64_t)0), cols - 1);
#pragma unroll
      for (int r = 0; r < PM_ROWS; ++r) {
        const int64_t tok = __builtin_amdgcn_readlane(tk, r);
        xv[r] = x[tok * ldx + c[r]];
        cbt[r] = q[tok * cb + (c[r] >> 1)];
        sc[r] = scales[tok * sb + c[r] / BLK];
      }
#pragma unroll
      for (int r = 0; r < PM_ROWS; ++r) {
        if (r < nr) {
          const uint32_t code = (c[r] & 1) ? (cbt[r] >> 4) : (cbt[r] & 15u);
          float p = (FMT == FP4Q_NVFP4) ? (e2m1_mag_value(code) * e4m3_value(sc[r])) * t
                                        : e2m1_mag_value(code) * exp2i((int)sc[r] - 127);
          if (code & 8u) p = -p;
          r_out[(m0 + r) * nS + j] =
              (uint16_t)f32_to_bf16_rne(bf16_to_f32(xv[r]) - p);
        }
      }
    }
  }
}

}  // namespace

void launch_permute(int fmt, const uint16_t* x, int64_t ldx, int64_t tokens, int64_t cols,
                    const uint8_t* q, const uint8_t* scales, const float* tscale,
                    const int32_t* row_src, int64_t rows, const int32_t* off, int G,
                    const int32_t* chan, int nS, uint8_t* q_out, uint8_t* s_out, float* ts_out,
                    uint16_t* r_out, hipStream_t stream) {
  const int64_t per_wg = (PM_THREADS / 64) * PM_ROWS;
  const int64_t wgs = (rows + per_wg - 1) / per_wg;
  const dim3 grid((unsigned)(wgs > 0 ? wgs : 1));
  // widest units that divide the rows (buffers are at least 8-byte aligned
  // for the codes; 16-byte units need 16-byte aligned buffers)
  const int64_t cb = cols / 2, sb = cols / (fmt == FP4Q_NVFP4 ? 16 : 32);
  const bool c16 = cb % 16 == 0 && aligned16(q) && aligned16(q_out);
  const int su = (sb % 16 == 0 && aligned16(scales) && aligned16(s_out)) ? 16
                 : (sb % 4 == 0 && aligned4(scales) && aligned4(s_out)) ? 4 : 1;
#define FP4Q_PERMUTE(F, C, S)                                                                 \
  hipLaunchKernelGGL((k_permute_rows<F, C, S>), grid, dim3(PM_THREADS), 0, stream, x, ldx,   \
                     tokens, cols, q, scales, tscale, row_src, rows, off, G, chan, nS, q_out, \
                     s_out, ts_out, r_out)
#define FP4Q_PERMUTE_S(F, C) \
  if (su == 16) FP4Q_PERMUTE(F, C, 16); else if (su == 4) FP4Q_PERMUTE(F, C, 4); else FP4Q_PERMUTE(F, C, 1)
  if (fmt == FP4Q_NVFP4) {
    if (c16) { FP4Q_PERMUTE_S(FP4Q_NVFP4, 16); } else { FP4Q_PERMUTE_S(FP4Q_NVFP4, 8); }
  } else {
    if (c16) { FP4Q_PERMUTE_S(FP4Q_MXFP4, 16); } else { FP4Q_PERMUTE_S(FP4Q_MXFP4, 8); }
  }
#undef FP4Q_PERMUTE_S
#undef FP4Q_PERMUTE
}

}  // namespace fp4q
