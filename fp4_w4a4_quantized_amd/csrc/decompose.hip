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
constexpr int DEC_MAX_WG = 512;   // two per CU: one round, and few partial records

// Partial records, one per workgroup of k_decompose, stored slot-major
// (word slot * G + record, G records) so that the final kernel's threads,
// one record each, read consecutive words: slots 0..19 the four 320-bit
// sums (c * 5 + limb), 20..23 the sums of squares, 24 the cross term (FP64
// bit patterns), 25 and 26 the counts.
constexpr int DEC_SLOTS = 32;
constexpr int DS_SQ = 20, DS_CROSS = 24, DS_NDZ = 25, DS_NCLIP = 26;

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

// A thread's (or a reduction's) share of the statistics.
struct DecAcc {
  uint64_t fix[4][5];
  double sq[5];  // four sums of squares, then the cross term
  int64_t cnt[2];
};

// Sum of the workgroup's DecAcc values into `res` (LDS; valid after the
// barrier this ends with), in a fixed order.  Every thread's values go to
// LDS field by field, the 320-bit sums as ten 32-bit digits each (their
// digit-wise sums, carried once at the end, give the sum modulo 2^320, as
// the two's complement fixed point needs); then four threads per field add
// a quarter of the threads each in thread order, one thread per field adds
// the quarters in order, and the carries are propagated.  The FP64 sums are
// therefore deterministic, and nothing waits on a chain of wide additions.
constexpr int DR_DIG = 40, DR_FIELDS = DR_DIG + 7;
__device__ __forceinline__ void dec_acc_reduce(const DecAcc& a, DecAcc& res) {
  __shared__ uint32_t sdig[DR_DIG][DEC_THREADS];
  __shared__ uint64_t sw[7][DEC_THREADS];  // five FP64 sums, two counts
  __shared__ uint64_t squ[DR_FIELDS][4];
  __shared__ uint64_t sfin[DR_FIELDS];
  const int t = threadIdx.x;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      sdig[10 * c + 2 * i][t] = (uint32_t)a.fix[c][i];
      sdig[10 * c + 2 * i + 1][t] = (uint32_t)(a.fix[c][i] >> 32);
    }
#pragma unroll
  for (int c = 0; c < 5; ++c) sw[c][t] = (uint64_t)__double_as_longlong(a.sq[c]);
  sw[5][t] = (uint64_t)a.cnt[0];
  sw[6][t] = (uint64_t)a.cnt[1];
  __syncthreads();
  constexpr int QN = DEC_THREADS / 4;
  if (t < 4 * DR_FIELDS) {
    const int f = t >> 2, b = (t & 3) * QN;
    uint64_t v = 0;
    if (f < DR_DIG) {
      for (int k = 0; k < QN; ++k) v += sdig[f][b + k];
    } else if (f < DR_DIG + 5) {
      double dv = 0.0;
      for (int k = 0; k < QN; ++k) dv += __longlong_as_double((long long)sw[f - DR_DIG][b + k]);
      v = (uint64_t)__double_as_longlong(dv);
    } else {
      for (int k = 0; k < QN; ++k) v += sw[f - DR_DIG][b + k];
    }
    squ[f][t & 3] = v;
  }
  __syncthreads();
  if (t < DR_FIELDS) {
    uint64_t v;
    if (t >= DR_DIG && t < DR_DIG + 5) {
      double dv = 0.0;
#pragma unroll
      for (int q = 0; q < 4; ++q) dv += __longlong_as_double((long long)squ[t][q]);
      v = (uint64_t)__double_as_longlong(dv);
    } else {
      v = squ[t][0] + squ[t][1] + squ[t][2] + squ[t][3];
    }
    sfin[t] = v;
  }
  __syncthreads();
  if (t < 4) {  // component t: carry the digit sums
    uint64_t carry = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      carry += sfin[10 * t + 2 * i];
      const uint64_t lo = carry & 0xFFFFFFFFull;
      carry = (carry >> 32) + sfin[10 * t + 2 * i + 1];
      res.fix[t][i] = lo | (carry << 32);
      carry >>= 32;
    }
  } else if (t == 4) {
#pragma unroll
    for (int c = 0; c < 5; ++c) res.sq[c] = __longlong_as_double((long long)sfin[DR_DIG + c]);
    res.cnt[0] = (int64_t)sfin[DR_DIG + 5];
    res.cnt[1] = (int64_t)sfin[DR_DIG + 6];
  }
  __syncthreads();
}

// Reduce the per-thread sums over the workgroup and write the workgroup's
// partial record.
__device__ __forceinline__ void write_partial(const uint64_t (&fix)[4][5], const double (&sq)[4],
                                              double cross, int64_t ndz, int64_t nclip,
                                              uint64_t* __restrict__ part) {
  DecAcc a;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int i = 0; i < 5; ++i) a.fix[c][i] = fix[c][i];
    a.sq[c] = sq[c];
  }
  a.sq[4] = cross;
  a.cnt[0] = ndz;
  a.cnt[1] = nclip;
  __shared__ DecAcc r;
  dec_acc_reduce(a, r);
  if (threadIdx.x == 0) {
    uint64_t* o = part + blockIdx.x;
    const int64_t G = gridDim.x;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < 5; ++i) o[(c * 5 + i) * G] = r.fix[c][i];
      o[(DS_SQ + c) * G] = (uint64_t)__double_as_longlong(r.sq[c]);
    }
    o[DS_CROSS * G] = (uint64_t)__double_as_longlong(r.sq[4]);
    o[DS_NDZ * G] = (uint64_t)r.cnt[0];
    o[DS_NCLIP * G] = (uint64_t)r.cnt[1];
  }
}

// ---- NVFP4 ------------------------------------------------------------------
//
// The same split under the NVFP4 quantizer: per 16-block with amax A, the
// quantizer's own decisions (scale code of (A / 6) / t, element code of
// x / (sb t) rounded on the E2M1 grid) give Q_s(x) = g sb t, and the ideal
// scale is again A / 6.  Terms times 6: x6 = 6x, qs6 = 6 g sb t, qst6 = g* A.
// One thread per block sums, per block and exactly in FP64,
//   S0 = x6 where g = 0,  S1 = x6 where g != 0,  S2 = qst6 where g != 0,
//   S3 = qs6  (= 3 sb t times an integer, S2 = A/2 times an integer),
// and the components are total = S0 + S1 - S3, scale_bias = S2 - S3,
// deadzone = S0, grid_noise = S1 - S2.  x6 sums take the fixed point
// element by element when the block's exponent span would make an FP64 sum
// inexact.  Exact while every term is a multiple of 2^-136: a tensor amax of
// at least 2^-89.

// Per-workgroup maximum of |x| (BF16 magnitude pattern).
__global__ void __launch_bounds__(DEC_THREADS) k_dec_amax(const uint16_t* __restrict__ x,
                                                          int64_t rows, int64_t cols, int64_t ldx,
                                                          uint32_t* __restrict__ amax_part) {
  __shared__ uint32_t red[DEC_THREADS / 64];
  const int64_t nb = cols >> 4, total = rows * nb;
  uint32_t m = 0;
  for (int64_t id = (int64_t)blockIdx.x * DEC_THREADS + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * DEC_THREADS) {
    const int64_t row = id / nb, b = id - row * nb;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + row * ldx + b * 16);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const u32x4 tv = __builtin_nontemporal_load(src + v);
      const uint32_t w[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    }
  }
  for (int s = 32; s > 0; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < DEC_THREADS / 64; ++i) r = max(r, red[i]);
    amax_part[blockIdx.x] = r;
  }
}

__device__ __forceinline__ void fix_neg(uint64_t (&a)[5]) {
  uint64_t carry = 1;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint64_t v = ~a[i];
    const uint64_t s = v + carry;
    carry = (s < v) ? 1ull : 0ull;
    a[i] = s;
  }
}

// One block of NE elements (w: NE/2 packed BF16 pairs) into the thread's
// sums.  Per block: the quantizer's decisions, then the term sums
//   S0 = sum of 6x where g = 0,  S1 = sum of 6x where g != 0,
//   S2 = sum of 6 Q*(x) where g != 0 (A times a multiple of 1/2),
//   S3 = sum of 6 Q_s(x) (6 s times a multiple of 1/2, s the block's scale),
// each added to the fixed point once per block (sums of x in FP64 when the
// block's exponent span keeps them exact, else element by element).
// Decisions, as the quantizer takes them, by the hardware conversion to
// E2M1 (nearest, ties to even, saturating, sign kept):
//  * g: of x / 2^e (MXFP4, exact: the BF16 pair converted directly), or of
//    the correctly rounded quotient x / (sb t) (NVFP4, the quantizer's own
//    reciprocal-and-FMA division with its operand scaling);
//  * g*: of RN(6x / A), the correctly rounded quotient: 6|x| has at most 10
//    significant bits and A at most 8, so a quotient within half an ulp of
//    a rounding threshold of the E2M1 grid equals it, and the rounded
//    quotient decides exactly as the exact one, ties included.
// The signed E2M1 values e = v_g and e* = v_g* (with x's sign) come back
// from the conversion to FP32.  The component values follow as before and
// are exact (FP32 for MXFP4; FP64 where the NVFP4 tensor scale enters).
template <int FMT, int NE>
__device__ __forceinline__ void block_terms(const uint32_t (&w)[NE / 2], float t,
                                            uint64_t (&S)[4][5], double (&sq)[4], double& cross,
                                            uint32_t& ndz, uint32_t& nclip) {
  typedef float v2f32t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2d __attribute__((ext_vector_type(2)));
  uint32_t am = 0, mn = 0xFFFFu;
#pragma unroll
  for (int i = 0; i < NE / 2; ++i) {
    const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
    am = max(am, max(lo, hi));
    mn = min(mn, min(lo ? lo : 0xFFFFu, hi ? hi : 0xFFFFu));
  }
  const float A = bf16_to_f32(am);
  // the block's scale s: MXFP4 2^e; NVFP4 sb * t (exact real product)
  float e8 = 0.0f, sbf = 1.0f, dq = 0.0f, yq = 0.0f, sx = 1.0f;
  double s_d;
  if (FMT == FP4Q_MXFP4) {
    const int e = mx_exponent(A);
    e8 = __uint_as_float((uint32_t)(e + 127) << 23);  // the E8M0 scale operand
    s_d = (double)exp2i(e);
  } else {
    sbf = e4m3_value(e4m3_encode((A / 6.0f) / t));
    // the quantizer's divisor sb t, its operand scaling and reciprocal
    sx = t >= 0x1p-87f ? 1.0f : 0x1p64f;
    dq = sbf * t * sx;
    yq = dq > 0.0f ? 1.0f / dq : 0.0f;
    s_d = (double)sbf * (double)t;
  }
  const double s6 = 6.0 * s_d;  // the block's largest representable magnitude
  // |x| > s6 exactly when |x| >= s6up, the least FP32 value above s6
  float s6up = (float)s6;
  if ((double)s6up <= s6) s6up = __uint_as_float(__float_as_uint(s6up) + 1u);
  // The FP32 work below (6|x|, the component values) is taken times a power
  // of two sc, exact and order-preserving, so that blocks near the top of the
  // BF16 range do not overflow (6 * 2^127 does); 1/sc undoes it in FP64.
  const float sc = (am >> 7) >= 127 + 120 ? 0x1p-16f : 1.0f;
  const double isc = (double)(1.0f / sc);
  const float As = A * sc;
  // the ideal-scale quotient 6x / A, its operands brought into the range of
  // the reciprocal-and-FMA division by a power of two sq
  const float sq6 = As < 0x1p-60f ? 0x1p64f : 1.0f;
  const float qa = As * sq6, ya = qa > 0.0f ? 1.0f / qa : 0.0f;
  const float six_sc = 6.0f * sc, six_scq = six_sc * sq6;
  const float q6u = (float)(s_d * 6.0 * (double)sc);  // MXFP4: 6 s sc, a power of two times 6
  const float six_sb = 6.0f * sbf;
  // FP64 sums of up to 32 values below 2^(ea+1) with least bit 2^lsb_min are
  // exact when (ea + 6) - lsb_min <= 53
  const int ea = (int)(am >> 7) - 127;
  const int lsb_min = (mn == 0xFFFFu) ? ea : (((mn >> 7) == 0) ? -133 : (int)(mn >> 7) - 134);
  const bool fast = (am >> 7) == 0 || (ea + 6) - lsb_min <= 53;
  double xa = 0.0, x1 = 0.0;  // sums of x over the block, and where g != 0
  float i1 = 0.0f, i2 = 0.0f;  // sums of e, and of e* where g != 0 (exact)
  // the block's statistics, of components taken times sc (1/sc^2 applied
  // once at the end; a power of two); NVFP4's t times sc, exact
  double bq[4] = {0.0, 0.0, 0.0, 0.0}, bx = 0.0;
  const double tsc = (double)t * (double)sc;
  // eight elements (one 16-byte piece) at a time keeps the unrolled body
  // within the register budget
#pragma unroll 1
  for (int v = 0; v < NE / 8; ++v) {
  uint32_t wv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wv[j] = NE == 16 ? (v == 0 ? w[j] : w[4 + j])
                     : (v == 0 ? w[j] : v == 1 ? w[4 + j] : v == 2 ? w[8 + j] : w[12 + j]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float xp[2] = {__uint_as_float(wv[i] << 16), __uint_as_float(wv[i] & 0xFFFF0000u)};
    uint32_t cg;
    if (FMT == FP4Q_MXFP4) {
      cg = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2d, wv[i]), e8, 0);
    } else {
      cg = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quot_rn(xp[0] * sx, dq, yq),
                                                    quot_rn(xp[1] * sx, dq, yq), 1.0f, 0);
    }
    const uint32_t cs = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
        0u, quot_rn(xp[0] * six_scq, qa, ya), quot_rn(xp[1] * six_scq, qa, ya), 1.0f, 0);
    const v2f32t ep = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cg, 1.0f, 0);
    const v2f32t esp = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cs, 1.0f, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float xv = xp[h], ax = fabsf(xv);
      const float e = ep[h], es = esp[h];
      const bool gz = e == 0.0f;  // code magnitude 0
      i1 += e;
      i2 += gz ? 0.0f : es;
      if (fast) {
        xa += (double)xv;
        x1 += (double)(gz ? 0.0f : xv);
      } else {
        fix_add(S[0], gz ? 6.0 * (double)xv : 0.0);
        fix_add(S[1], gz ? 0.0 : 6.0 * (double)xv);
      }
      ndz += (gz && ax != 0.0f) ? 1u : 0u;
      nclip += ax >= s6up ? 1u : 0u;
      // component values times 6 sc (exact: FP32 values and differences
      // within the block's range; NVFP4's products with t in FP64).  Q_s is
      // 0 where g = 0, so the selects act on FP32 operands.
      const float x6 = xv * six_sc;
      const float q6s = es * As;  // 6 Q*(x) sc
      double ct, csb;
      if (FMT == FP4Q_MXFP4) {
        const float q6a = e * q6u;  // 6 Q_s(x) sc, a power-of-two scale
        ct = (double)(x6 - q6a);
        csb = (double)((gz ? 0.0f : q6s) - q6a);
      } else {
        const double q6a = (double)(e * six_sb) * tsc;
        ct = (double)x6 - q6a;
        csb = (double)(gz ? 0.0f : q6s) - q6a;
      }
      const double cdz = (double)(gz ? x6 : 0.0f);
      const double cgn = (double)(gz ? 0.0f : x6 - q6s);
      bq[0] = __builtin_fma(ct, ct, bq[0]);
      bq[1] = __builtin_fma(csb, csb, bq[1]);
      bq[2] = __builtin_fma(cdz, cdz, bq[2]);
      bq[3] = __builtin_fma(cgn, cgn, bq[3]);
      bx = __builtin_fma(csb, cgn, bx);
    }
  }
  }
  const double isc2 = isc * isc;
#pragma unroll
  for (int c = 0; c < 4; ++c) sq[c] = __builtin_fma(bq[c], isc2, sq[c]);
  cross = __builtin_fma(bx, isc2, cross);
  if (fast) {
    fix_add(S[0], 6.0 * (xa - x1));
    fix_add(S[1], 6.0 * x1);
  }
  fix_add(S[2], (double)i2 * (double)A);
  fix_add(S[3], (double)i1 * 6.0 * s_d);
}

// One thread per block (32 elements MXFP4, 16 NVFP4).  NVFP4 first reduces
// the per-workgroup amax words of k_dec_amax to the tensor scale.
template <int FMT>
__global__ void __launch_bounds__(DEC_THREADS) k_decompose(const uint16_t* __restrict__ x,
                                                           int64_t rows, int64_t cols, int64_t ldx,
                                                           const uint32_t* __restrict__ amax_part,
                                                           int nparts,
                                                           uint64_t* __restrict__ part) {
  constexpr int NE = (FMT == FP4Q_NVFP4) ? 16 : 32;
  float t = 1.0f;
  if (FMT == FP4Q_NVFP4) {
    // the tensor amax: the workgroup reduces the per-workgroup words
    __shared__ uint32_t sred[DEC_THREADS / 64];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += DEC_THREADS) m = max(m, amax_part[i]);
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if ((threadIdx.x & 63) == 0) sred[threadIdx.x >> 6] = m;
    __syncthreads();
    m = 0;
#pragma unroll
    for (int i = 0; i < DEC_THREADS / 64; ++i) m = max(m, sred[i]);
    t = nv_tensor_scale(bf16_to_f32(m));
  }
  uint64_t S[4][5];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 5; ++i) S[c][i] = 0;
  double sq[4] = {0.0, 0.0, 0.0, 0.0}, cross = 0.0;
  uint32_t ndz = 0, nclip = 0;

  const int64_t nb = cols / NE, total = rows * nb;
  for (int64_t id = (int64_t)blockIdx.x * DEC_THREADS + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * DEC_THREADS) {
    const int64_t row = id / nb, b = id - row * nb;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + row * ldx + b * NE);
    uint32_t w[NE / 2];
#pragma unroll
    for (int v = 0; v < NE / 8; ++v) {
      const u32x4 tv = __builtin_nontemporal_load(src + v);
      w[4 * v] = tv.x; w[4 * v + 1] = tv.y; w[4 * v + 2] = tv.z; w[4 * v + 3] = tv.w;
    }
    block_terms<FMT, NE>(w, t, S, sq, cross, ndz, nclip);
  }

  // components from the term sums: total = S0 + S1 - S3, scale_bias =
  // S2 - S3, deadzone = S0, grid_noise = S1 - S2
  uint64_t fix[4][5], n2[5], n3[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    n2[i] = S[2][i];
    n3[i] = S[3][i];
    fix[0][i] = S[0][i];
    fix[1][i] = S[2][i];
    fix[2][i] = S[0][i];
    fix[3][i] = S[1][i];
  }
  fix_neg(n2);
  fix_neg(n3);
  fix_add_fix(fix[0], S[1]);
  fix_add_fix(fix[0], n3);
  fix_add_fix(fix[1], n3);
  fix_add_fix(fix[3], n2);
#pragma unroll
  for (int c = 0; c < 4; ++c) sq[c] /= 36.0;  // the squares were taken times 6
  write_partial(fix, sq, cross / 36.0, ndz, nclip, part);
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

// amax_part / namax: the NVFP4 path's per-workgroup amax words (BF16
// magnitude patterns), or null / 0 for MXFP4.  A tensor amax in (0, 2^-89)
// (patterns below 0x1300) lets terms fall below the fixed point's LSB: the
// sums are then flagged FP4Q_DEC_INEXACT.
__global__ void __launch_bounds__(DEC_THREADS) k_decompose_final(const uint64_t* __restrict__ part,
                                                                 int nparts, int64_t n_elems,
                                                                 const uint32_t* __restrict__ amax_part,
                                                                 int namax,
                                                                 fp4q_err_stats_t* __restrict__ out) {
  __shared__ uint32_t samax[DEC_THREADS / 64];
  const int t = threadIdx.x;
  uint32_t am = 0;
  for (int p = t; p < namax; p += DEC_THREADS) am = max(am, amax_part[p]);
  for (int o = 32; o > 0; o >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, o));
  if ((t & 63) == 0) samax[t >> 6] = am;
  DecAcc acc;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 5; ++i) acc.fix[c][i] = 0;
#pragma unroll
  for (int c = 0; c < 5; ++c) acc.sq[c] = 0.0;
  acc.cnt[0] = acc.cnt[1] = 0;
  // at most two records per thread: all loads issued before the sums
  static_assert(DEC_MAX_WG <= 2 * DEC_THREADS, "two partial records per thread");
  const int64_t G = nparts;
  uint64_t r[2][DS_NCLIP + 1];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = t + h * DEC_THREADS;
#pragma unroll
    for (int k = 0; k <= DS_NCLIP; ++k) r[h][k] = p < nparts ? part[k * G + p] : 0ull;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      fix_add_fix(acc.fix[c], &r[h][c * 5]);
      acc.sq[c] += __longlong_as_double((long long)r[h][DS_SQ + c]);
    }
    acc.sq[4] += __longlong_as_double((long long)r[h][DS_CROSS]);
    acc.cnt[0] += (int64_t)r[h][DS_NDZ];
    acc.cnt[1] += (int64_t)r[h][DS_NCLIP];
  }
  __shared__ DecAcc sres;
  dec_acc_reduce(acc, sres);  // its barriers also publish samax
  // lanes 0..3 convert one component each
  if (t < 4) {
    uint64_t a[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      a[i] = sres.fix[t][i];
      out->exact[t][i] = (int64_t)a[i];
    }
    out->sum[t] = fix_to_double(a) / 6.0;
    out->sumsq[t] = sres.sq[t];
  }
  if (t == 0) {
    out->cross_sb_gn = sres.sq[4];
    out->n_elems = n_elems;
    out->n_deadzone = sres.cnt[0];
    out->n_clipped = sres.cnt[1];
    uint32_t m = 0;
    for (int i = 0; i < DEC_THREADS / 64; ++i) m = max(m, samax[i]);
    out->flags = (m != 0u && m < 0x1300u) ? (int64_t)FP4Q_DEC_INEXACT : 0;
  }
}

// Workgroups for `blk`-element blocks, one block per thread.
static int64_t dec_grid(int64_t rows, int64_t cols, int blk) {
  int64_t nb = rows * (cols / blk);
  int64_t g = (nb + DEC_THREADS - 1) / DEC_THREADS;
  if (g < 1) g = 1;
  return g < DEC_MAX_WG ? g : DEC_MAX_WG;
}

// Partial records (for either format: the NVFP4 grid is the larger), then
// the NVFP4 path's per-workgroup amax words.
size_t decompose_workspace_bytes(int64_t rows, int64_t cols) {
  const int64_t g = dec_grid(rows, cols, 16);
  return (size_t)g * DEC_SLOTS * 8 + (size_t)((g * 4 + 255) / 256 * 256);
}

int launch_decompose(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                     fp4q_err_stats_t* out, void* ws, hipStream_t stream) {
  uint64_t* part = static_cast<uint64_t*>(ws);
  if (fmt == FP4Q_NVFP4) {
    const int64_t g = dec_grid(rows, cols, 16);
    uint32_t* amax = reinterpret_cast<uint32_t*>(part + (size_t)DEC_SLOTS * g);
    hipLaunchKernelGGL(k_dec_amax, dim3((unsigned)g), dim3(DEC_THREADS), 0, stream, x, rows, cols,
                       ldx, amax);
    hipLaunchKernelGGL(k_decompose<FP4Q_NVFP4>, dim3((unsigned)g), dim3(DEC_THREADS), 0, stream,
                       x, rows, cols, ldx, amax, (int)g, part);
    hipLaunchKernelGGL(k_decompose_final, dim3(1), dim3(DEC_THREADS), 0, stream, part, (int)g,
                       rows * cols, amax, (int)g, out);
    return 0;
  }
  const int64_t g = dec_grid(rows, cols, 32);
  hipLaunchKernelGGL(k_decompose<FP4Q_MXFP4>, dim3((unsigned)g), dim3(DEC_THREADS), 0, stream, x,
                     rows, cols, ldx, nullptr, 0, part);
  hipLaunchKernelGGL(k_decompose_final, dim3(1), dim3(DEC_THREADS), 0, stream, part, (int)g,
                     rows * cols, nullptr, 0, out);
  return 0;
}

}  // namespace fp4q
