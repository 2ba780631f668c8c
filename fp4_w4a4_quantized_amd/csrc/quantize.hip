// quantize.hip -- online activation (and weight) quantization to NVFP4 /
// MXFP4 with residual emission on selected channels.
//
// QUADS abstract: activations are quantized online every forward pass and
// suffer the coarse E2M1 grid; the explainer's section 2.2 B and the
// FourSight abstract keep a residual for a few selected channels.
//
// NVFP4 needs the tensor (or per-expert group) amax before any block scale,
// so it runs in two streaming passes: k_group_amax (atomic max of the FP32
// bit pattern, exact and order-free for non-negative values) and
// k_quantize.  MXFP4 is a single pass.  One thread owns one scale block:
// it loads the block with 16-byte vector loads, computes the block amax, the
// scale code, the E2M1 codes (nearest-even by threshold compares), packs two
// codes per byte and stores them with one vector store, and writes the BF16
// residual for the selected channels that fall in its block.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

// Group of a row: the g with off[g] <= row < off[g+1] (binary search).
__device__ __forceinline__ int group_of_row(const int32_t* __restrict__ off, int G, int64_t row) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Clear the amax words and pre-set every tensor scale to 1 (empty groups
// keep it).  A fill kernel rather than a memset so the sequence can be
// captured in a HIP graph.
__global__ void k_quant_init(uint32_t* __restrict__ amax_bits, float* __restrict__ tscale, int G) {
  int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g < G) {
    amax_bits[g] = 0u;
    tscale[g] = 1.0f;
  }
}

// Per-group amax.  Each workgroup owns a run of ROWS_PER_WG rows; waves take
// rows in turn, lanes stride along the row in 8-element (16-byte) chunks.
// When the whole run lies in one group (always when G == 1) the workgroup
// reduces in LDS and issues one atomic; otherwise each row issues its own.
constexpr int AMAX_ROWS_PER_WG = 16;

__global__ void __launch_bounds__(256) k_group_amax(const uint16_t* __restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ldx,
                                                    const int32_t* __restrict__ off, int G,
                                                    uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * AMAX_ROWS_PER_WG;
  const int64_t r1 = r0 + AMAX_ROWS_PER_WG < rows ? r0 + AMAX_ROWS_PER_WG : rows;
  const int g0 = (G > 1) ? group_of_row(off, G, r0) : 0;
  const int g1 = (G > 1) ? group_of_row(off, G, r1 - 1) : 0;
  const bool one_group = (g0 == g1);
  uint32_t wmax = 0;
  const int64_t nchunk = cols >> 3;
  for (int64_t r = r0 + wave; r < r1; r += 4) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + r * ldx);
    uint32_t m = 0;
    for (int64_t c = lane; c < nchunk; c += 64) {
      u32x4 v = __builtin_nontemporal_load(xr + c);
      // |bf16| patterns compare like the values (finite inputs)
      m = max(m, max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu));
      m = max(m, max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
      m = max(m, max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu));
      m = max(m, max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu));
    }
    for (int s = 32; s > 0; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s));
    if (one_group) {
      wmax = max(wmax, m);
    } else if (lane == 0) {
      atomicMax(&amax_bits[group_of_row(off, G, r)], m << 16);
    }
  }
  if (one_group) {
    if (lane == 0) red[wave] = wmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t m = max(max(red[0], red[1]), max(red[2], red[3]));
      if (m) atomicMax(&amax_bits[g0], m << 16);
    }
  }
}

// One thread per scale block of BLK elements (16 NVFP4, 32 MXFP4).
template <int FMT>
__global__ void __launch_bounds__(256) k_quantize(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    const int32_t* __restrict__ off, int G, const int32_t* __restrict__ chan, int nS,
    uint8_t* __restrict__ q, uint8_t* __restrict__ scales, float* __restrict__ tscale,
    uint16_t* __restrict__ resid, const uint32_t* __restrict__ amax_bits) {
  constexpr int BLK = (FMT == FP4Q_NVFP4) ? 16 : 32;
  constexpr int NV = BLK / 8;  // 16-byte vectors per block
  const int64_t nb = cols / BLK;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= rows * nb) return;
  const int64_t row = id / nb, b = id - row * nb;
  const int g = (G > 1) ? group_of_row(off, G, row) : 0;

  // load the block
  uint32_t w[BLK / 2];
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * ldx + b * BLK);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    u32x4 t = __builtin_nontemporal_load(src + v);
    w[4 * v + 0] = t.x; w[4 * v + 1] = t.y; w[4 * v + 2] = t.z; w[4 * v + 3] = t.w;
  }
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < BLK / 2; ++i) am = max(am, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  const float amax = bf16_to_f32(am);

  // block scale
  float t = 1.0f, d, sb = 0.0f, inv_pow2 = 1.0f;
  uint32_t sc;
  if (FMT == FP4Q_NVFP4) {
    t = nv_tensor_scale(__uint_as_float(amax_bits[g]));
    float v = (amax / 6.0f) / t;
    sc = e4m3_encode(v);
    sb = e4m3_value(sc);
    d = sb * t;
    if (row == (G > 1 ? (int64_t)off[g] : 0) && b == 0) tscale[g] = t;
  } else {
    int e = mx_exponent(amax);
    sc = (uint32_t)(e + 127);
    d = exp2i(e);
    inv_pow2 = exp2i(-e);
  }
  scales[row * nb + b] = (uint8_t)sc;

  // element codes, packed two per byte (even element in the low nibble)
  uint32_t packed[BLK / 8];
#pragma unroll
  for (int i = 0; i < BLK / 8; ++i) packed[i] = 0;
#pragma unroll
  for (int k = 0; k < BLK; ++k) {
    uint32_t h = (w[k >> 1] >> ((k & 1) * 16)) & 0xFFFFu;
    float a = bf16_to_f32(h & 0x7FFFu);
    uint32_t mag;
    if (FMT == FP4Q_NVFP4)
      mag = (d == 0.0f) ? 0u : e2m1_mag_code(a / d);
    else
      mag = e2m1_mag_code(a * inv_pow2);
    uint32_t code = ((h >> 15) << 3) | mag;
    packed[k >> 3] |= code << ((k & 7) * 4);
  }
  uint8_t* qdst = q + row * (cols >> 1) + b * (BLK / 2);
  if (BLK == 16) {
    *reinterpret_cast<u32x2*>(qdst) = u32x2{packed[0], packed[1]};
  } else {
    *reinterpret_cast<u32x4*>(qdst) = u32x4{packed[0], packed[1], packed[2], packed[3]};
  }

  // residual on the selected channels of this block
  if (nS > 0) {
    const int32_t* S = chan + (int64_t)g * nS;
    const int c0 = (int)(b * BLK);
    int lo = 0, hi = nS;  // first j with S[j] >= c0
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (S[mid] < c0) lo = mid + 1; else hi = mid;
    }
    int j = lo;
    int cn = (j < nS) ? S[j] : 0x7FFFFFFF;
    if (cn < c0 + BLK) {
#pragma unroll
      for (int k = 0; k < BLK; ++k) {
        if (c0 + k == cn) {
          uint32_t h = (w[k >> 1] >> ((k & 1) * 16)) & 0xFFFFu;
          float xv = bf16_to_f32(h);
          uint32_t code = (packed[k >> 3] >> ((k & 7) * 4)) & 15u;
          float p;
          if (FMT == FP4Q_NVFP4) {
            p = e2m1_mag_value(code) * sb;  // exact
            p = p * t;
          } else {
            p = e2m1_mag_value(code) * d;   // exact
          }
          if (code & 8u) p = -p;
          float r = xv - p;
          resid[row * nS + j] = (uint16_t)f32_to_bf16_rne(r);
          ++j;
          cn = (j < nS) ? S[j] : 0x7FFFFFFF;
        }
      }
    }
  }
}

int launch_quantize(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                    const int32_t* off, int G, const int32_t* chan, int nS, uint8_t* q,
                    uint8_t* scales, float* tscale, uint16_t* resid, void* ws,
                    hipStream_t stream) {
  const int64_t blk = (fmt == FP4Q_NVFP4) ? 16 : 32;
  const int64_t nthreads = rows * (cols / blk);
  uint32_t* amax_bits = static_cast<uint32_t*>(ws);
  if (fmt == FP4Q_NVFP4) {
    hipLaunchKernelGGL(k_quant_init, dim3((G + 255) / 256), dim3(256), 0, stream, amax_bits,
                       tscale, G);
    if (rows > 0) {
      const int64_t nwg = (rows + AMAX_ROWS_PER_WG - 1) / AMAX_ROWS_PER_WG;
      hipLaunchKernelGGL(k_group_amax, dim3((unsigned)nwg), dim3(256), 0, stream, x, rows, cols,
                         ldx, off, G, amax_bits);
    }
  }
  if (nthreads > 0) {
    dim3 grid((unsigned)((nthreads + 255) / 256));
    if (fmt == FP4Q_NVFP4)
      hipLaunchKernelGGL(k_quantize<FP4Q_NVFP4>, grid, dim3(256), 0, stream, x, rows, cols, ldx,
                         off, G, chan, nS, q, scales, tscale, resid, amax_bits);
    else
      hipLaunchKernelGGL(k_quantize<FP4Q_MXFP4>, grid, dim3(256), 0, stream, x, rows, cols, ldx,
                         off, G, chan, nS, q, scales, tscale, resid, amax_bits);
  }
  return 0;
}

}  // namespace fp4q
