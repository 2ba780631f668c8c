// gemm.hip -- W4A4 FP4 GEMM with fused sparse residual compensation, dense
// and expert-grouped, for gfx950.
//
// QUADS abstract: native W4A4 FP4 GEMM plus Residual Activation
// Compensation on high-error activation channels; explainer section 2.2 B:
// the residual term of the selected channels is added to the quantized
// output; FourSight abstract: the selected channels are effectively BF16
// inside the FP4 GEMM.
//
//   Y[m,n] = sum_k A[m,k] B[n,k] + sum_j R[m,j] B[n,S_j]
//
// Main loop (per 128-deep K step, packed FP4 tiles staged through LDS,
// double buffered, one barrier per step):
//  * MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 operands; each
//    lane's 32 K-elements are exactly one MX block, so the E8M0 codes feed
//    the instruction's per-lane scale operand directly.
//  * NVFP4: the 16-element E4M3 scales do not map onto the instruction's
//    power-of-two, 32-element scaling, and e2m1 * E4M3 needs up to 6
//    significant bits, which FP4/FP6/FP8 cannot hold.  Each lane decodes
//    its packed codes with v_cvt_scalef32_pk_f16_fp4 and one v_pk_mul_f16 by
//    the block scale -- exact in FP16 -- and feeds
//    v_mfma_f32_16x16x32_f16.  The tensor scales are factored out.
//  Both paths read the same LDS pattern: lane l takes the 16 bytes
//  (32 codes) of its row at chunk l/16.  For NVFP4 those 32 codes are two
//  scale blocks; sub-step s of the four f16 MFMAs uses dword s of every
//  lane, a K permutation that A and B share, so the sum is unchanged.
// Compensation: after the main loop the residual R (bf16) and the
// dequantized weight columns W[n, S_j] (e2m1 * block scale, exact in bf16)
// go through v_mfma_f32_16x16x32_bf16 into the same accumulators (NVFP4:
// acc = tw * (tx * main + comp)).
// LDS rows are padded to 80 bytes so the 16-byte reads of 16 consecutive
// rows fall in distinct banks.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct GemmArgs {
  int64_t M, N, K;
  const int32_t* off;
  int G;
  const uint8_t* aq;
  const uint8_t* as;
  const float* ats;
  const uint8_t* bq;
  const uint8_t* bs;
  const float* bts;
  const int32_t* chan;
  int nS;
  const uint16_t* resid;
  const float* cts;  // tensor scale of the compensation term, or null (1)
  void* y;
  int y_bf16;
  int64_t ldy;
  bool tiled;  // packed operands in the tiled layout (never for the grouped form)
};

constexpr int LDS_ROW = 80;  // bytes per staged row: 64 data + 16 pad

// Decode one dword of 8 NVFP4 codes into 8 f16 values times the block scale.
__device__ __forceinline__ f16x8 decode_nv8(uint32_t w, f16x2 s) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Dequantized weight element as bf16 bits, tensor scale excluded:
// e2m1 * E4M3 (NVFP4) or e2m1 * 2^(code-127) (MXFP4); exact in bf16.
template <int FMT>
__device__ __forceinline__ uint32_t wdeq_bf16(const uint8_t* __restrict__ bq,
                                              const uint8_t* __restrict__ bs, int64_t K,
                                              bool tiled, int64_t n, int c) {
  constexpr int BLK = (FMT == FP4Q_NVFP4) ? 16 : 32;
  uint32_t byte = bq[code_off(tiled, n, c >> 1, K)];
  uint32_t code = (c & 1) ? (byte >> 4) : (byte & 15u);
  uint32_t sc = bs[scale_off<FMT>(tiled, n, c / BLK, K)];
  float s = (FMT == FP4Q_NVFP4) ? e4m3_value(sc)
                                : (sc ? __uint_as_float(sc << 23) : __uint_as_float(0x00400000u));
  float v = e2m1_mag_value(code) * s;
  return (__float_as_uint(v) >> 16) | ((code & 8u) << 12);
}

template <int FMT, int BM, int BN, bool GROUPED>
__global__ void __launch_bounds__(256) k_gemm(GemmArgs p) {
  constexpr int BLK = (FMT == FP4Q_NVFP4) ? 16 : 32;
  constexpr int SPR = 128 / BLK;  // scale bytes per row per K step
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 16, TN = WN / 16;
  constexpr int CA = (BM * 4 + 255) / 256, CB = (BN * 4 + 255) / 256;
  static_assert(TM >= 1 && TN >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t sAs[2][BM * SPR];
  __shared__ __attribute__((aligned(16))) uint8_t sBs[2][BN * SPR];
  __shared__ int s_tile[2];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t K = p.K, N = p.N;
  const int64_t K2 = K >> 1, KS = K / BLK;
  const bool tiled = GROUPED ? false : p.tiled;

  // ---- which rows / group this workgroup owns
  int g = 0;
  int64_t row_begin, row_end;
  if (GROUPED) {
    // tiles of group g: ceil(rows_g / BM); find the group holding tile
    // blockIdx.x by a block-wide scan over per-thread runs of 8 groups
    __shared__ int s_wsum[4];
    const int G = p.G;
    int cnt = 0;
    for (int i = 0; i < 8; ++i) {
      int gg = t * 8 + i;
      if (gg < G) cnt += (p.off[gg + 1] - p.off[gg] + BM - 1) / BM;
    }
    int incl = cnt;
    for (int s = 1; s < 64; s <<= 1) {
      int v = __shfl_up(incl, s);
      if (lane >= s) incl += v;
    }
    if (lane == 63) s_wsum[wave] = incl;
    if (t == 0) s_tile[0] = -1;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_wsum[w];
    int excl = before + incl - cnt;
    const int tile = blockIdx.x;
    if (tile >= excl && tile < excl + cnt) {
      int acc = excl;
      for (int i = 0; i < 8; ++i) {
        int gg = t * 8 + i;
        int c = (gg < G) ? (p.off[gg + 1] - p.off[gg] + BM - 1) / BM : 0;
        if (tile < acc + c) {
          s_tile[0] = gg;
          s_tile[1] = tile - acc;
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
    if (s_tile[0] < 0) return;  // past the last tile: uniform exit
    g = s_tile[0];
    row_begin = (int64_t)p.off[g] + (int64_t)s_tile[1] * BM;
    row_end = min((int64_t)p.off[g + 1], row_begin + BM);
  } else {
    row_begin = (int64_t)blockIdx.x * BM;
    row_end = min(p.M, row_begin + BM);
  }
  const int64_t col0 = (int64_t)blockIdx.y * BN;
  const uint8_t* __restrict__ aq = p.aq;
  const uint8_t* __restrict__ as = p.as;
  const uint8_t* __restrict__ bq = p.bq + (GROUPED ? (int64_t)g * N * K2 : 0);
  const uint8_t* __restrict__ bs = p.bs + (GROUPED ? (int64_t)g * N * KS : 0);

  // ---- global -> register staging of one K step
  u32x4 ra[CA], rb[CB];
  uint32_t rsc[2];  // this thread's scale bytes (row t of A, or row t-BM of B)
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      int c = t + i * 256;
      int r = c >> 2, ch = c & 3;
      int64_t gr = row_begin + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c < BM * 4 && gr < row_end)
        v = *reinterpret_cast<const u32x4*>(aq + code_off(tiled, gr, (int64_t)kt * 64 + ch * 16, K));
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      int c = t + i * 256;
      int r = c >> 2, ch = c & 3;
      int64_t gc = col0 + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c < BN * 4 && gc < N)
        v = *reinterpret_cast<const u32x4*>(bq + code_off(tiled, gc, (int64_t)kt * 64 + ch * 16, K));
      rb[i] = v;
    }
    // scale dwords: bytes [0,4) and (NVFP4) [4,8) of the row's step; in the
    // tiled layout the two NVFP4 dwords sit in separate planes
    rsc[0] = rsc[1] = 0u;
    const uint8_t* src = nullptr;
    int64_t srow = 0;
    if (t < BM) {
      srow = row_begin + t;
      if (srow < row_end) src = as;
    } else if (t < BM + BN) {
      srow = col0 + (t - BM);
      if (srow < N) src = bs;
    }
    if (src) {
      rsc[0] = *reinterpret_cast<const uint32_t*>(
          src + scale_off<FMT>(tiled, srow, (int64_t)kt * SPR, K));
      if (SPR == 8)
        rsc[1] = *reinterpret_cast<const uint32_t*>(
            src + scale_off<FMT>(tiled, srow, (int64_t)kt * SPR + 4, K));
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      int c = t + i * 256;
      if (c < BM * 4)
        *reinterpret_cast<u32x4*>(&sA[buf][(c >> 2) * LDS_ROW + (c & 3) * 16]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      int c = t + i * 256;
      if (c < BN * 4)
        *reinterpret_cast<u32x4*>(&sB[buf][(c >> 2) * LDS_ROW + (c & 3) * 16]) = rb[i];
    }
    uint8_t* dst = nullptr;
    if (t < BM) dst = &sAs[buf][t * SPR];
    else if (t < BM + BN) dst = &sBs[buf][(t - BM) * SPR];
    if (dst) {
      if (SPR == 8) *reinterpret_cast<u32x2*>(dst) = u32x2{rsc[0], rsc[1]};
      else *reinterpret_cast<uint32_t*>(dst) = rsc[0];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int q = lane >> 4, lr = lane & 15;
  const int nk = (int)(K / 128);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    u32x4 fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[i] = *reinterpret_cast<const u32x4*>(&sA[buf][(wm * WM + i * 16 + lr) * LDS_ROW + q * 16]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[j] = *reinterpret_cast<const u32x4*>(&sB[buf][(wn * WN + j * 16 + lr) * LDS_ROW + q * 16]);
    if (FMT == FP4Q_MXFP4) {
      int sa[TM], sbv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) sa[i] = sAs[buf][(wm * WM + i * 16 + lr) * 4 + q];
#pragma unroll
      for (int j = 0; j < TN; ++j) sbv[j] = sBs[buf][(wn * WN + j * 16 + lr) * 4 + q];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          i32x8 av = {(int)fa[i].x, (int)fa[i].y, (int)fa[i].z, (int)fa[i].w, 0, 0, 0, 0};
          i32x8 bv = {(int)fb[j].x, (int)fb[j].y, (int)fb[j].z, (int)fb[j].w, 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              av, bv, acc[i][j], 4, 4, 0, sa[i], 0, sbv[j]);
        }
    } else {
      // two E4M3 block scales per lane row: blocks 2q (dwords 0,1) and 2q+1 (2,3)
      f16x2 sa[TM][2], sbv[TN][2];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        uint32_t s2 = *reinterpret_cast<const uint16_t*>(&sAs[buf][(wm * WM + i * 16 + lr) * 8 + 2 * q]);
        _Float16 s0 = (_Float16)e4m3_value(s2 & 0xFFu), s1 = (_Float16)e4m3_value(s2 >> 8);
        sa[i][0] = f16x2{s0, s0};
        sa[i][1] = f16x2{s1, s1};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        uint32_t s2 = *reinterpret_cast<const uint16_t*>(&sBs[buf][(wn * WN + j * 16 + lr) * 8 + 2 * q]);
        _Float16 s0 = (_Float16)e4m3_value(s2 & 0xFFu), s1 = (_Float16)e4m3_value(s2 >> 8);
        sbv[j][0] = f16x2{s0, s0};
        sbv[j][1] = f16x2{s1, s1};
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 da[TM], db[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) da[i] = decode_nv8(fa[i][s], sa[i][s >> 1]);
#pragma unroll
        for (int j = 0; j < TN; ++j) db[j] = decode_nv8(fb[j][s], sbv[j][s >> 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(da[i], db[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- tensor scales (NVFP4): y = tw (tx main + c comp), run as
  // (tw c) ((tx / c) main + comp); with c = 1 the factors are tw and tx exactly
  float tx = 1.0f, tw = 1.0f;
  if (FMT == FP4Q_NVFP4) {
    const float c = p.cts ? p.cts[GROUPED ? g : 0] : 1.0f;
    tx = p.ats[GROUPED ? g : 0] / c;
    tw = p.bts[GROUPED ? g : 0] * c;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] *= tx;
  }

  // ---- compensation: acc += R[:, S] * Wdeq[S, :]
  const int nS = p.nS;
  if (nS > 0) {
    const int32_t* __restrict__ S = p.chan + (GROUPED ? (int64_t)g * nS : 0);
    for (int j0 = 0; j0 < nS; j0 += 32) {
      const int jj = j0 + 8 * q;
      int ch[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ch[e] = (jj + e < nS) ? S[jj + e] : -1;
      bf16x8 ra8[TM], rb8[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        int64_t gr = row_begin + wm * WM + i * 16 + lr;
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          h[e] = (gr < row_end && ch[e] >= 0) ? p.resid[gr * nS + jj + e] : 0u;
        u32x4 pk = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                    h[6] | (h[7] << 16)};
        ra8[i] = __builtin_bit_cast(bf16x8, pk);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int64_t gc = col0 + wn * WN + j * 16 + lr;
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          h[e] = (gc < N && ch[e] >= 0) ? wdeq_bf16<FMT>(bq, bs, K, tiled, gc, ch[e]) : 0u;
        u32x4 pk = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                    h[6] | (h[7] << 16)};
        rb8[j] = __builtin_bit_cast(bf16x8, pk);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra8[i], rb8[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: lane holds rows 4q..4q+3 of column lr of each 16x16 tile
  const int64_t ldy = GROUPED ? N : p.ldy;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int64_t gc = col0 + wn * WN + j * 16 + lr;
      if (gc >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int64_t gr = row_begin + wm * WM + i * 16 + 4 * q + r;
        if (gr >= row_end) continue;
        float v = acc[i][j][r] * tw;
        if (p.y_bf16)
          reinterpret_cast<uint16_t*>(p.y)[gr * ldy + gc] = (uint16_t)f32_to_bf16_rne(v);
        else
          reinterpret_cast<float*>(p.y)[gr * ldy + gc] = v;
      }
    }
}

template <int FMT, int BM, int BN, bool GROUPED>
static void launch_one(const GemmArgs& a, unsigned mtiles, hipStream_t stream) {
  dim3 grid(mtiles, (unsigned)((a.N + BN - 1) / BN));
  hipLaunchKernelGGL((k_gemm<FMT, BM, BN, GROUPED>), grid, dim3(256), 0, stream, a);
}

GemmPath gemm_path(int64_t M, int64_t N, int64_t K, int nS) {
  if (skinny_gemm_eligible(M, N, K, nS)) return PATH_SKINNY;
  if (big_gemm_eligible(M, N, K, nS)) return PATH_BIG;
  return PATH_GENERIC;
}

// The large-tile kernels stream B_S: without a prepared array it is
// gathered into the workspace once per call.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int nS) {
  return gemm_path(M, N, K, nS) == PATH_BIG ? big_gemm_workspace_bytes(N, nS) : 0;
}

size_t grouped_workspace_bytes(int64_t N, int64_t K, int G, int nS) {
  return big_grouped_eligible(N, K, nS) ? (size_t)G * big_gemm_workspace_bytes(N, nS) : 0;
}

bool grouped_tiled_ok(int fmt, int64_t N, int64_t K, int nS) {
  return fmt == FP4Q_NVFP4 && big_grouped_eligible(N, K, nS);
}

// Second-pass residual decode: thread i takes elements 8i .. 8i+7 of the
// row-major [M, nS] residual (one 32-bit code word, one block scale) and
// writes e2m1 * block scale as BF16, exact (at most 6 significant bits; the
// tensor scale is applied by the GEMM).
template <int FMT>
__global__ void __launch_bounds__(256) k_deq_resid(const uint8_t* __restrict__ rq,
                                                   const uint8_t* __restrict__ rs, int64_t M,
                                                   int nS, uint16_t* __restrict__ out) {
  constexpr int BLK = (FMT == FP4Q_NVFP4) ? 16 : 32;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = nS >> 3;
  if (i >= M * per_row) return;
  const int64_t m = i / per_row;
  const int j0 = (int)(i - m * per_row) * 8;
  const uint8_t* cw = rq + m * (nS >> 1) + (j0 >> 1);
  const uint32_t w = (uint32_t)cw[0] | ((uint32_t)cw[1] << 8) | ((uint32_t)cw[2] << 16) |
                     ((uint32_t)cw[3] << 24);
  const uint32_t c8 = rs[m * (nS / BLK) + j0 / BLK];
  const float sv = (FMT == FP4Q_NVFP4)
                       ? e4m3_value(c8)
                       : (c8 ? __uint_as_float(c8 << 23) : __uint_as_float(0x00400000u));
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t code = (w >> (4 * e)) & 15u;
    h[e] = (__float_as_uint(e2m1_mag_value(code) * sv) >> 16) | ((code & 8u) << 12);
  }
  *reinterpret_cast<u32x4*>(out + m * nS + j0) =
      u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

void launch_deq_resid(int fmt, int64_t M, int nS, const uint8_t* rq, const uint8_t* rs,
                      uint16_t* out, hipStream_t stream) {
  const int64_t n = M * (nS >> 3);
  if (n <= 0) return;
  dim3 grid((unsigned)((n + 255) / 256));
  if (fmt == FP4Q_NVFP4)
    hipLaunchKernelGGL((k_deq_resid<FP4Q_NVFP4>), grid, dim3(256), 0, stream, rq, rs, M, nS, out);
  else
    hipLaunchKernelGGL((k_deq_resid<FP4Q_MXFP4>), grid, dim3(256), 0, stream, rq, rs, M, nS, out);
}

int launch_gemm(int fmt, bool tiled, int64_t M, int64_t N, int64_t K, const int32_t* off, int G,
                const uint8_t* aq, const uint8_t* as, const float* ats, const uint8_t* bq,
                const uint8_t* bs, const float* bts, const int32_t* chan, int nS,
                const uint16_t* resid, const float* cts, void* y, int y_bf16, int64_t ldy,
                void* ws, hipStream_t stream, const uint8_t* bsel_pre) {
  GemmArgs a{M, N, K, off, G, aq, as, ats, bq, bs, bts, chan, nS, resid, cts, y, y_bf16, ldy,
             tiled};
  if (M == 0 || N == 0) return 0;
  if (off != nullptr && big_grouped_eligible(N, K, nS)) {
    launch_gemm_big_grouped(fmt, M, N, K, off, G, aq, as, ats, bq, bs, bts, chan, nS, resid,
                            cts, bsel_pre, y, y_bf16, ws, stream, tiled);
    return 0;
  }
  if (off != nullptr) {
    constexpr int BM = 64;
    unsigned mt = (unsigned)((M + BM - 1) / BM + G);  // each group adds at most one partial tile
    if (fmt == FP4Q_NVFP4) launch_one<FP4Q_NVFP4, BM, 128, true>(a, mt, stream);
    else launch_one<FP4Q_MXFP4, BM, 128, true>(a, mt, stream);
    return 0;
  }
  switch (gemm_path(M, N, K, nS)) {
    case PATH_SKINNY:
      launch_gemm_skinny(fmt, tiled, M, N, K, aq, as, ats, bq, bs, bts, chan, nS, resid, cts,
                         bsel_pre, y, y_bf16, ldy, stream);
      break;
    case PATH_BIG:
      launch_gemm_big(fmt, tiled, M, N, K, aq, as, ats, bq, bs, bts, chan, nS, resid, cts,
                      bsel_pre, y, y_bf16, ldy, ws, stream);
      break;
    default:
      if (M <= 64) {
        unsigned mt = (unsigned)((M + 63) / 64);
        if (fmt == FP4Q_NVFP4) launch_one<FP4Q_NVFP4, 64, 32, false>(a, mt, stream);
        else launch_one<FP4Q_MXFP4, 64, 32, false>(a, mt, stream);
      } else {
        unsigned mt = (unsigned)((M + 127) / 128);
        if (fmt == FP4Q_NVFP4) launch_one<FP4Q_NVFP4, 128, 128, false>(a, mt, stream);
        else launch_one<FP4Q_MXFP4, 128, 128, false>(a, mt, stream);
      }
  }
  return 0;
}

}  // namespace fp4q
