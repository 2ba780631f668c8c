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
// A workgroup owns one class of tokens (token mod 8) within a chunk of 256
// output rows; its threads find their rows' tokens and groups (binary search
// of the offsets in LDS) and compact the rows of the class into a list.
// Waves then take eight listed rows at a time: the code and scale bytes of
// the eight rows are spread over the lanes in the widest units the row
// lengths allow (16 bytes for the codes at cols % 32 == 0), and so are the
// rows' (row, channel) residual pairs, four per lane in flight.
#include "fp4q_device.h"
#include "fp4q_internal.h"

#include <type_traits>

namespace fp4q {

namespace {

constexpr int PM_THREADS = 256;  // four waves
constexpr int PM_ROWS = 8;       // output rows per wave and step
constexpr int PM_CHUNK = 256;    // rows per chunk: one per thread
constexpr int PM_XCD = 8;        // workgroups per chunk, one per token class
constexpr int PM_MAX_GROUPS = 2048;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

// Copy rows of the wave's list in units of T: output row mrow(r) from token
// row tk(r), both held by lane r (r < nr); the units of all rows are spread
// over the lanes, four per lane in flight.
template <typename T>
__device__ __forceinline__ void copy_rows(const uint8_t* __restrict__ src,
                                          uint8_t* __restrict__ dst, int64_t row_bytes, int tk,
                                          int mrow, int nr, int lane) {
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
      const int64_t m = __shfl(mrow, r);
      const int64_t i = ok ? (int64_t)(u - (uint32_t)r * per) : 0;
      v[k] = reinterpret_cast<const T*>(src + tok * row_bytes)[i];
      d[k] = ok ? m * per + i : -1;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (d[k] >= 0) reinterpret_cast<T*>(dst)[d[k]] = v[k];
  }
}

// Workgroup b takes chunk b / 8 of the output rows and, of those, the rows
// whose token is congruent to b mod 8.  Workgroups are dispatched to the 8
// XCDs in turn, so each XCD's L2 holds the rows of one eighth of the tokens
// (their x rows for the residual gathers, their codes for the copies).  Any
// other dispatch order gives the same result, only with less L2 reuse.
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
  __shared__ int s_off[PM_MAX_GROUPS + 1];
  __shared__ int s_m[PM_CHUNK], s_tok[PM_CHUNK], s_g[PM_CHUNK];
  __shared__ int s_cnt[PM_THREADS / 64];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  if (FMT == FP4Q_NVFP4 && blockIdx.x == 0)
    for (int g = t; g < G; g += PM_THREADS) ts_out[g] = tscale[0];
  const int cls = (int)(blockIdx.x % PM_XCD);
  const int64_t base = (int64_t)(blockIdx.x / PM_XCD) * PM_CHUNK;
  if (base >= rows) return;
  if (nS > 0)
    for (int g = t; g <= G; g += PM_THREADS) s_off[g] = off[g];

  // this thread's row of the chunk: its token (clamped into range; in range
  // by precondition) and whether it belongs to this workgroup's class
  const int64_t m = base + t;
  const bool valid = m < rows;
  const int tok = valid ? (int)min(max((int64_t)row_src[m], (int64_t)0), tokens - 1) : 0;
  const bool mine = valid && (tok % PM_XCD) == cls;
  const uint64_t bal = __ballot(mine);
  if (lane == 0) s_cnt[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, n = 0;
#pragma unroll
  for (int w = 0; w < PM_THREADS / 64; ++w) {
    before += w < wave ? s_cnt[w] : 0;
    n += s_cnt[w];
  }
  if (mine) {
    const int pos = before + (int)__popcll(bal & ((1ull << lane) - 1ull));
    int g = 0;
    if (nS > 0) {  // the last group g with off[g] <= m (skips empty groups)
      int lo = 0, hi = G;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= m) lo = mid;
        else hi = mid;
      }
      g = lo;
    }
    s_m[pos] = (int)m;
    s_tok[pos] = tok;
    s_g[pos] = g;
  }
  __syncthreads();

  const int64_t cb = cols / 2, sb = cols / BLK;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  typedef typename std::conditional<CU == 16, u32x4v, uint64_t>::type CodeUnit;
  typedef typename std::conditional<SU == 16, u32x4v,
                                    typename std::conditional<SU == 4, uint32_t, uint8_t>::type>::type
      ScaleUnit;
  const float tt = (FMT == FP4Q_NVFP4) ? tscale[0] : 1.0f;
  for (int i0 = wave * PM_ROWS; i0 < n; i0 += PM_THREADS / 64 * PM_ROWS) {
    const int nr = min(PM_ROWS, n - i0);
    const int li = i0 + min(lane, nr - 1);  // lanes past the list repeat its last row
    const int mrow = s_m[li], tk = s_tok[li], gl = s_g[li];
    if (q_out != nullptr) {  // null: the grouped GEMM gathers the codes itself
      copy_rows<CodeUnit>(q, q_out, cb, tk, mrow, nr, lane);
      copy_rows<ScaleUnit>(scales, s_out, sb, tk, mrow, nr, lane);
    }

    // residual: the (row, channel) pairs of the eight rows spread over the
    // lanes, four per lane in flight
    const uint32_t pairs = (uint32_t)nr * (uint32_t)nS;
    for (uint32_t p0 = 0; p0 < pairs; p0 += 4 * 64) {
      int64_t c[4], tok_k[4], dst[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t pr = p0 + lane + 64 * k;
        const bool ok = pr < pairs;
        const int r = ok ? (int)(pr / (uint32_t)nS) : 0;
        const int j = ok ? (int)(pr - (uint32_t)r * (uint32_t)nS) : 0;
        const int64_t g = __shfl(gl, r);
        tok_k[k] = __shfl(tk, r);
        dst[k] = ok ? (int64_t)__shfl(mrow, r) * nS + j : -1;
        c[k] = min(max((int64_t)chan[g * nS + j], (int64_t)0), cols - 1);
      }
      uint32_t xv[4], cbt[4], sc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xv[k] = x[tok_k[k] * ldx + c[k]];
        cbt[k] = q[tok_k[k] * cb + (c[k] >> 1)];
        sc[k] = scales[tok_k[k] * sb + c[k] / BLK];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (dst[k] >= 0) {
          const uint32_t code = (c[k] & 1) ? (cbt[k] >> 4) : (cbt[k] & 15u);
          float p = (FMT == FP4Q_NVFP4) ? (e2m1_mag_value(code) * e4m3_value(sc[k])) * tt
                                        : e2m1_mag_value(code) * exp2i((int)sc[k] - 127);
          if (code & 8u) p = -p;
          r_out[dst[k]] = (uint16_t)f32_to_bf16_rne(bf16_to_f32(xv[k]) - p);
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
  const int64_t chunks = (rows + PM_CHUNK - 1) / PM_CHUNK;
  const dim3 grid((unsigned)(chunks > 0 ? chunks * PM_XCD : 1));
  // widest units that divide the rows (buffers are at least 8-byte aligned
  // for the codes; 16-byte units need 16-byte aligned buffers)
  const int64_t cb = cols / 2, sb = cols / (fmt == FP4Q_NVFP4 ? 16 : 32);
  const bool c16 = cb % 16 == 0 && aligned16(q) && aligned16(q_out);  // (null is aligned)
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
