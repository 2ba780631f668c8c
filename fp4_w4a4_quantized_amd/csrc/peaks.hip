// peaks.hip -- microbenchmarks of the attainable MI355X (gfx950) peaks that
// the GEMM and quantizer fractions are also reported against:
//  * matrix cores: long runs of independent v_mfma_f32_32x32x16_f16 (the
//    exact-NVFP4 GEMM's instruction) or v_mfma_scale_f32_32x32x64_f8f6f4
//    with FP4 operands (the MXFP4 GEMM's), no memory traffic;
//  * HBM: a streaming read (16 bytes per lane per load, grid-stride) and a
//    streaming copy of a caller buffer larger than the last-level cache.
// Built into its own library (libfp4q_peaks.so, include/fp4q_peaks.h): it is
// measurement infrastructure, not part of the quantized-GEMM boundary.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp4q_peaks.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;   // independent accumulators per wave
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t mix(uint32_t v) {
  v ^= v >> 16;
  v *= 0x7feb352dU;
  v ^= v >> 15;
  v *= 0x846ca68bU;
  v ^= v >> 16;
  return v;
}

// kind 0: f16 32x32x16; kind 1: FP4 x FP4 scaled 32x32x64 (E8M0 scale 127 = 1)
template <int KIND>
__global__ void __launch_bounds__(kThreads) k_mfma_peak(int iters, float* out) {
  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
  if (KIND == 0) {
    h16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // small values of a few significant bits: the sums stay finite
      a[e] = (_Float16)((int)(mix(gid * 16 + e) & 7) - 3) * (_Float16)0.125f;
      b[e] = (_Float16)((int)(mix(gid * 16 + 8 + e) & 7) - 3) * (_Float16)0.125f;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
  } else {
    // random FP4 codes: the matrix core's power draw with data like the GEMM's
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (int)(e < 4 ? mix(gid * 16 + e) : 0u);
      b[e] = (int)(e < 4 ? mix(gid * 16 + 8 + e) : 0u);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 4, 4, 0, 127, 0,
                                                                 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[gid] = s;
}

__global__ void __launch_bounds__(kThreads) k_read(const u32x4* __restrict__ p, uint64_t n16,
                                                   uint32_t* out) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(p + i);
    const u32x4 v1 = __builtin_nontemporal_load(p + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= v0 ^ v1 ^ v2 ^ v3;
  }
  for (; i < n16; i += stride) acc ^= p[i];
  out[(uint64_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ void __launch_bounds__(kThreads) k_copy(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + stride < n16; i += 2 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    __builtin_nontemporal_store(v0, dst + i);
    __builtin_nontemporal_store(v1, dst + i + stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

thread_local int g_last_error = 0;

int done() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_error = (int)e;
    return -4;
  }
  return 0;
}

}  // namespace

extern "C" {

int fp4q_peaks_last_hip_error(void) { return g_last_error; }

int64_t fp4q_peak_mfma_out_floats(int32_t blocks) {
  return blocks <= 0 ? 0 : (int64_t)blocks * kThreads;
}

int fp4q_peak_mfma(int32_t kind, int32_t blocks, int32_t iters, float* out, double* flops,
                   void* stream) {
  if ((kind != 0 && kind != 1) || blocks <= 0 || blocks > 65536 || iters <= 0 || !out || !flops)
    return -1;
  const double per = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  *flops = per * kChains * (double)iters * (kThreads / 64) * (double)blocks;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(k_mfma_peak<0>, dim3(blocks), dim3(kThreads), 0, st, iters, out);
  else
    hipLaunchKernelGGL(k_mfma_peak<1>, dim3(blocks), dim3(kThreads), 0, st, iters, out);
  return done();
}

int fp4q_peak_read(const void* buf, uint64_t bytes, int32_t blocks, uint32_t* out,
                   void* stream) {
  if (!buf || !out || bytes < 16 || bytes % 16 != 0 || blocks <= 0 || blocks > 65536 ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_read, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, out);
  return done();
}

int fp4q_peak_copy(const void* src, void* dst, uint64_t bytes, int32_t blocks, void* stream) {
  if (!src || !dst || bytes < 16 || bytes % 16 != 0 || blocks <= 0 || blocks > 65536 ||
      ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) != 0)
    return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return done();
}

}  // extern "C"
