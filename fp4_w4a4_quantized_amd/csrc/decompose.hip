// decompose.hip -- exact three-way MXFP4 quantization-error decomposition.
//
// "Decomposing MXFP4 quantization error for LLM reinforcement learning",
// abstract: the error splits exactly into scale bias (power-of-two rounding
// of the scale), deadzone truncation (small values zeroed) and grid noise
// (rounding to the 4-bit grid).  Per 32-block with actual scale s = 2^e and
// ideal scale s* = amax/6, per element x:
//   total = x - Q_s(x); deadzone = x where Q_s(x) = 0;
//   otherwise grid_noise = x - Q*(x), scale_bias = Q*(x) - Q_s(x).
// Everything is carried times 6: 6x, 6*Q_s = 6*g*2^e and 6*Q* = g* * amax are
// short dyadic numbers, so each component is exact in FP64.
//
// Sums are exact: each thread adds components into 320-bit two's complement
// fixed-point accumulators (LSB 2^-136, five 64-bit limbs).  Integer
// addition is associative, so the result is independent of the order and
// the three parts add up to the total bit for bit.  To keep the limb
// arithmetic off the per-element path, a block whose exponent span makes
// every FP64 partial sum exact (E(amax) - E(lsb of smallest element) small)
// is summed in FP64 first and added once; otherwise element by element.
// One thread owns one 32-element block; workgroups reduce in LDS and write a
// partial record; one final workgroup reduces the partials in a fixed order.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

constexpr int DEC_THREADS = 256;
constexpr int DEC_MAX_WG = 2048;

struct DecPartial {
  uint64_t fix[4][5];
  double sq[4];
  double cross;
  int64_t ndz, nclip;
  int64_t pad[5];
};
static_assert(sizeof(DecPartial) == 256, "partial record layout");

// a += v, v an FP64 multiple of 2^-136 below 2^183 in magnitude.
__device__ __forceinline__ void fix_add(uint64_t (&a)[5], double v) {
  if (v == 0.0) return;
  uint64_t bits = (uint64_t)__double_as_longlong(v);
  const bool neg = bits >> 63;
  const int ef = (int)((bits >> 52) & 0x7FF);
  uint64_t M = (bits & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  int sh = ef - 1075 + 136;     // bit position of M's least significant bit
  if (sh < 0) {                 // the shifted-out bits are zero by construction
    M >>= -sh;
    sh = 0;
  }
  const int li = sh >> 6, bo = sh & 63;
  const uint64_t lo = M << bo, hi = bo ? (M >> (64 - bo)) : 0ull;
  uint64_t carry = neg ? 1ull : 0ull;  // negative: add ~magnitude + 1
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    uint64_t m = (i == li) ? lo : ((i == li + 1) ? hi : 0ull);
    if (neg) m = ~m;
    uint64_t s = a[i] + m;
    uint64_t c1 = (s < m) ? 1ull : 0ull;
    uint64_t s2 = s + carry;
    uint64_t c2 = (s2 < s) ? 1ull : 0ull;
    a[i] = s2;
    carry = c1 | c2;
  }
}

__device__ __forceinline__ void fix_add_fix(uint64_t (&a)[5], const uint64_t* b) {
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    uint64_t s = a[i] + b[i];
    uint64_t c1 = (s < b[i]) ? 1ull : 0ull;
    uint64_t s2 = s + carry;
    uint64_t c2 = (s2 < s) ? 1ull : 0ull;
    a[i] = s2;
    carry = c1 | c2;
  }
}

// 6x times the components of one element; returns the E2M1 code magnitude.
__device__ __forceinline__ uint32_t elem_components(uint32_t h, float amax, float inv_s, int e,
                                                    double (&c6)[4]) {
  const float x = bf16_to_f32(h);
  const float ax = bf16_to_f32(h & 0x7FFFu);
  const double sgn = (h & 0x8000u) ? -1.0 : 1.0;
  const double x6 = 6.0 * (double)x;
  const uint32_t mag = e2m1_mag_code(ax * inv_s);
  const double qs6 = sgn * (6.0 * (double)e2m1_mag_value(mag)) * (double)exp2i(e);
  // Q*: nearest grid point to 6|x|/amax, decided exactly on 6|x| vs tau*amax
  const double a6 = 6.0 * (double)ax, A = (double)amax;
  uint32_t gs = 0;
  if (amax > 0.0f)
    gs = (uint32_t)(a6 > 0.25 * A) + (uint32_t)(a6 >= 0.75 * A) + (uint32_t)(a6 > 1.25 * A) +
         (uint32_t)(a6 >= 1.75 * A) + (uint32_t)(a6 > 2.5 * A) + (uint32_t)(a6 >= 3.5 * A) +
         (uint32_t)(a6 > 5.0 * A);
  const double qst6 = sgn * (double)e2m1_mag_value(gs) * A;
  c6[0] = x6 - qs6;
  if (mag == 0) {
    c6[1] = 0.0;
    c6[2] = x6;
    c6[3] = 0.0;
  } else {
    c6[1] = qst6 - qs6;
    c6[2] = 0.0;
    c6[3] = x6 - qst6;
  }
  return mag;
}

__global__ void __launch_bounds__(DEC_THREADS) k_decompose(const uint16_t* __restrict__ x,
                                                           int64_t rows, int64_t cols,
                                                           int64_t ldx,
                                                           DecPartial* __restrict__ part) {
  uint64_t fix[4][5];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 5; ++i) fix[c][i] = 0;
  double sq[4] = {0.0, 0.0, 0.0, 0.0}, cross = 0.0;
  int64_t ndz = 0, nclip = 0;

  const int64_t nb = cols >> 5, total = rows * nb;
  for (int64_t id = (int64_t)blockIdx.x * DEC_THREADS + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * DEC_THREADS) {
    const int64_t row = id / nb, b = id - row * nb;
    uint32_t w[16];
    const u32x4* src = reinterpret_cast<const u32x4*>(x + row * ldx + b * 32);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      u32x4 tv = __builtin_nontemporal_load(src + v);
      w[4 * v] = tv.x; w[4 * v + 1] = tv.y; w[4 * v + 2] = tv.z; w[4 * v + 3] = tv.w;
    }
    uint32_t am = 0, mn = 0xFFFFu;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
      am = max(am, max(lo, hi));
      mn = min(mn, min(lo ? lo : 0xFFFFu, hi ? hi : 0xFFFFu));
    }
    const float amax = bf16_to_f32(am);
    const int e = mx_exponent(amax);
    const float inv_s = exp2i(-e);
    // exponent of the least significant bit of the smallest non-zero element
    // and of amax; FP64 block sums are exact when the span is small
    const int ea = (int)(am >> 7) - 127;
    const int lsb_min = (mn == 0xFFFFu) ? ea : (((mn >> 7) == 0) ? -133 : (int)(mn >> 7) - 134);
    const bool fast = (am >> 7) == 0 || (ea + 11) - min(lsb_min + 1, ea - 8) <= 52;
    double bsum[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t h = (w[k >> 1] >> ((k & 1) * 16)) & 0xFFFFu;
      double c6[4];
      const uint32_t mag = elem_components(h, amax, inv_s, e, c6);
      ndz += (mag == 0 && (h & 0x7FFFu) != 0) ? 1 : 0;
      nclip += ((double)bf16_to_f32(h & 0x7FFFu) > 6.0 * (double)exp2i(e)) ? 1 : 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double cv = c6[c] / 6.0;
        sq[c] += cv * cv;
        if (fast) bsum[c] += c6[c];
        else fix_add(fix[c], c6[c]);
      }
      cross += (c6[1] / 6.0) * (c6[3] / 6.0);
    }
    if (fast) {
#pragma unroll
      for (int c = 0; c < 4; ++c) fix_add(fix[c], bsum[c]);
    }
  }

  // workgroup reduction through LDS in a fixed tree order
  __shared__ uint64_t sfix[DEC_THREADS][4][5];
  __shared__ double ssq[DEC_THREADS][5];
  __shared__ int64_t scnt[DEC_THREADS][2];
  const int t = threadIdx.x;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int i = 0; i < 5; ++i) sfix[t][c][i] = fix[c][i];
    ssq[t][c] = sq[c];
  }
  ssq[t][4] = cross;
  scnt[t][0] = ndz;
  scnt[t][1] = nclip;
  __syncthreads();
  for (int s = DEC_THREADS / 2; s > 0; s >>= 1) {
    if (t < s) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint64_t a[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) a[i] = sfix[t][c][i];
        fix_add_fix(a, &sfix[t + s][c][0]);
#pragma unroll
        for (int i = 0; i < 5; ++i) sfix[t][c][i] = a[i];
      }
#pragma unroll
      for (int c = 0; c < 5; ++c) ssq[t][c] += ssq[t + s][c];
      scnt[t][0] += scnt[t + s][0];
      scnt[t][1] += scnt[t + s][1];
    }
    __syncthreads();
  }
  if (t == 0) {
    DecPartial* o = part + blockIdx.x;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < 5; ++i) o->fix[c][i] = sfix[0][c][i];
      o->sq[c] = ssq[0][c];
    }
    o->cross = ssq[0][4];
    o->ndz = scnt[0][0];
    o->nclip = scnt[0][1];
  }
}

// Approximate double value of a 320-bit two's complement fixed-point sum.
__device__ double fix_to_double(const uint64_t (&a)[5]) {
  uint64_t m[5];
  const bool neg = a[4] >> 63;
  uint64_t carry = neg ? 1ull : 0ull;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    uint64_t v = neg ? ~a[i] : a[i];
    uint64_t s = v + carry;
    carry = (s < v) ? 1ull : 0ull;
    m[i] = s;
  }
  double r = 0.0;
  for (int i = 4; i >= 0; --i) r = r * 18446744073709551616.0 + (double)m[i];
  r = ldexp(r, -136);
  return neg ? -r : r;
}

__global__ void __launch_bounds__(DEC_THREADS) k_decompose_final(const DecPartial* __restrict__ part,
                                                                 int nparts, int64_t n_elems,
                                                                 fp4q_err_stats_t* __restrict__ out) {
  __shared__ uint64_t sfix[DEC_THREADS][4][5];
  __shared__ double ssq[DEC_THREADS][5];
  __shared__ int64_t scnt[DEC_THREADS][2];
  const int t = threadIdx.x;
  uint64_t fix[4][5];
  double sq[5] = {0, 0, 0, 0, 0};
  int64_t cnt[2] = {0, 0};
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 5; ++i) fix[c][i] = 0;
  for (int p = t; p < nparts; p += DEC_THREADS) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      fix_add_fix(fix[c], &part[p].fix[c][0]);
      sq[c] += part[p].sq[c];
    }
    sq[4] += part[p].cross;
    cnt[0] += part[p].ndz;
    cnt[1] += part[p].nclip;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 5; ++i) sfix[t][c][i] = fix[c][i];
#pragma unroll
  for (int c = 0; c < 5; ++c) ssq[t][c] = sq[c];
  scnt[t][0] = cnt[0];
  scnt[t][1] = cnt[1];
  __syncthreads();
  for (int s = DEC_THREADS / 2; s > 0; s >>= 1) {
    if (t < s) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint64_t a[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) a[i] = sfix[t][c][i];
        fix_add_fix(a, &sfix[t + s][c][0]);
#pragma unroll
        for (int i = 0; i < 5; ++i) sfix[t][c][i] = a[i];
      }
#pragma unroll
      for (int c = 0; c < 5; ++c) ssq[t][c] += ssq[t + s][c];
      scnt[t][0] += scnt[t + s][0];
      scnt[t][1] += scnt[t + s][1];
    }
    __syncthreads();
  }
  if (t == 0) {
    for (int c = 0; c < 4; ++c) {
      uint64_t a[5];
      for (int i = 0; i < 5; ++i) {
        a[i] = sfix[0][c][i];
        out->exact[c][i] = (int64_t)a[i];
      }
      out->sum[c] = fix_to_double(a) / 6.0;
      out->sumsq[c] = ssq[0][c];
    }
    out->cross_sb_gn = ssq[0][4];
    out->n_elems = n_elems;
    out->n_deadzone = scnt[0][0];
    out->n_clipped = scnt[0][1];
  }
}

static int64_t dec_grid(int64_t rows, int64_t cols) {
  int64_t nb = rows * (cols / 32);
  int64_t g = (nb + DEC_THREADS - 1) / DEC_THREADS;
  if (g < 1) g = 1;
  return g < DEC_MAX_WG ? g : DEC_MAX_WG;
}

size_t decompose_workspace_bytes(int64_t rows, int64_t cols) {
  return (size_t)dec_grid(rows, cols) * sizeof(DecPartial);
}

int launch_decompose(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                     fp4q_err_stats_t* out, void* ws, hipStream_t stream) {
  const int64_t g = dec_grid(rows, cols);
  DecPartial* part = static_cast<DecPartial*>(ws);
  hipLaunchKernelGGL(k_decompose, dim3((unsigned)g), dim3(DEC_THREADS), 0, stream, x, rows, cols,
                     ldx, part);
  hipLaunchKernelGGL(k_decompose_final, dim3(1), dim3(DEC_THREADS), 0, stream, part, (int)g,
                     rows * cols, out);
  return 0;
}

}  // namespace fp4q
