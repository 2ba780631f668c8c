// fp4q_device.h -- device-side number-format helpers for gfx950 kernels.
//
// E2M1 / E4M3 / E8M0 / BF16 encode and decode as used by the quantizer and
// the GEMM prologues.  These are branch-light integer and compare forms
// (threshold tables, exponent-field arithmetic), written for VALU
// throughput; their results are defined by the format rules stated in
// include/fp4q.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Nearest-even float -> bf16 (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// E2M1 magnitude code of a >= 0 by its decision thresholds (the midpoints of
// the grid 0, .5, 1, 1.5, 2, 3, 4, 6): at a midpoint the even mantissa code
// wins, so 0.25, 1.25, 2.5, 5 round down and 0.75, 1.75, 3.5 round up.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

// E2M1 magnitude of a code's 3 low bits, as float.
__device__ __forceinline__ float e2m1_mag_value(uint32_t c) {
  // c = (exp << 1) | mant; exp 0 -> 0.5 * mant, else 2^(exp-1) * (1 + mant/2)
  uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float v = e ? __uint_as_float((126u + e) << 23 | (m << 22)) : 0.5f * (float)m;
  return v;
}

// E4M3 (FN) value of a non-negative code: the code's 7 low bits placed at
// the top of an FP32 exponent/mantissa field give 2^-120 times the value, for
// normal and subnormal codes alike.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  return __uint_as_float((c & 0x7Fu) << 20) * 0x1p120f;
}

// Nearest-even E4M3 code of v >= 0, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  if (v >= 448.0f) return 0x7Eu;
  if (v < 0x1p-6f) {
    // subnormal range: multiples of 2^-9; rintf rounds half to even
    return (uint32_t)rintf(v * 512.0f);
  }
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // round mantissa to 3 bits, ties to even
  return (u >> 20) - (120u << 3);     // rebias exponent 127 -> 7
}

// MXFP4 block exponent: smallest e in [-127, 127] with 6 * 2^e >= amax.
// amax = f * 2^E, f in [1, 2): e = E - 2 when f <= 1.5, else E - 1.
__device__ __forceinline__ int mx_exponent(float amax) {
  uint32_t u = __float_as_uint(amax);
  int ef = (int)(u >> 23);
  if (ef == 0) return -127;  // zero or subnormal amax: 6 * 2^-127 covers it
  int E = ef - 127;
  int e = ((u & 0x7FFFFFu) <= 0x400000u) ? E - 2 : E - 1;
  return e < -127 ? -127 : e;
}

// 2^e as float for e in [-127, 127] (2^-127 is an FP32 subnormal).
__device__ __forceinline__ float exp2i(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// NVFP4 tensor scale from the tensor amax.
__device__ __forceinline__ float nv_tensor_scale(float amax) {
  float t = amax / 2688.0f;
  return (amax == 0.0f || t == 0.0f) ? 1.0f : t;
}

// x / d rounded to nearest FP32, for the quotients the quantizer forms
// (|x| <= about 7 d).  With y = RN(1/d), q0 = RN(a y), a = |x|, is within two
// ulps of a/d; one FMA correction brings it within one ulp, and a second
// yields the correctly rounded quotient by Markstein's theorem (the residual
// a - q d is exact when nothing underflows).  The sign is x's sign bit: the
// corrections would turn -0 into +0.  Valid for d >= 2^-96; smaller divisors
// take the IEEE division instruction sequence.
__device__ __forceinline__ float div_rn(float x, float d, float y) {
  const float a = fabsf(x);
  float q = a * y;
  float r = __builtin_fmaf(-q, d, a);
  q = __builtin_fmaf(r, y, q);
  r = __builtin_fmaf(-q, d, a);
  q = __builtin_fmaf(r, y, q);
  return __uint_as_float(__float_as_uint(q) | (__float_as_uint(x) & 0x80000000u));
}

// x / d rounded to nearest from y = RN(1/d): two FMA corrections of x y
// (Markstein's theorem, as div_rn), on the signed value with the remainder
// formed negated, which keeps the sign of a zero quotient (d = 0 with y = 0
// gives the signed zero).  Correctly rounded while d >= 2^-96 and the
// remainder does not underflow; callers scale operands by powers of two
// into that range.
__device__ __forceinline__ float quot_rn(float x, float d, float y) {
  float q = x * y;
  float r = __builtin_fmaf(q, d, -x);
  q = __builtin_fmaf(-r, y, q);
  r = __builtin_fmaf(q, d, -x);
  return __builtin_fmaf(-r, y, q);
}

// E2M1 codes of 8 FP32 values, packed two per byte (even element in the low
// nibble), by gfx950's v_cvt_scalef32_pk_fp4_f32 with scale 1: nearest-even
// on the E2M1 grid, saturating at 6, sign kept (also for -0 and values that
// round to zero) -- the same decisions as the threshold rule of the grid.
// With an E8M0 scale 2^e (passed as the float whose exponent field is the
// code, 0.0f for code 0) the instruction divides by 2^e exactly before
// rounding, for every code 0..254 (checked on the GPU against pre-scaled
// inputs), which saves the MXFP4 path its eight multiplies.
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&v)[8], float scale = 1.0f) {
  uint32_t p = 0;
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[0], v[1], scale, 0);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2], v[3], scale, 1);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4], v[5], scale, 2);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6], v[7], scale, 3);
  return p;
}

// Byte offsets of packed FP4 operands in the two layouts (include/fp4q.h
// defines them).  Row-major: codes [rows][K/2], scales [rows][K/blk].
// Tiled (K % 128 == 0): codes in 1 KB blocks, one per (16-row group,
// 128-column step), the 16 bytes of row r and step-byte chunk c at
// (c*16 + r)*16 inside the block; scales in blocks per (64-row group, step)
// of 64 rows x (128/blk) bytes, NVFP4 as two dword planes [d][row], MXFP4 as
// one dword per row.  One wave's 16-byte loads of 16 rows x 64 bytes, and
// its dword loads of 64 rows' scales, are then single contiguous spans.
__device__ __forceinline__ int64_t code_off(bool tiled, int64_t row, int64_t byte_col, int64_t K) {
  if (!tiled) return row * (K >> 1) + byte_col;
  const int b64 = (int)(byte_col & 63);
  return (((row >> 4) * (K >> 7) + (byte_col >> 6)) << 10) +
         ((((b64 >> 4) << 4) + (row & 15)) << 4) + (b64 & 15);
}

// FMT: 0 NVFP4 (16-element blocks), 1 MXFP4 (32).
template <int FMT>
__device__ __forceinline__ int64_t scale_off(bool tiled, int64_t row, int64_t blk, int64_t K) {
  constexpr int BLK = (FMT == 0) ? 16 : 32;
  constexpr int SPS = 128 / BLK;  // scale bytes per row per 128-column step
  if (!tiled) return row * (K / BLK) + blk;
  const int e = (int)(blk % SPS);
  const int64_t base = ((row >> 6) * (K >> 7) + blk / SPS) * (SPS * 64);
  if (FMT == 0) return base + (((e >> 2) * 64 + (row & 63)) << 2) + (e & 3);
  return base + ((row & 63) << 2) + e;
}

}  // namespace fp4q
