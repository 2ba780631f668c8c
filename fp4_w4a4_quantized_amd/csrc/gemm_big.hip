// gemm_big.hip -- the prefill-shaped compensated W4A4 GEMM for gfx950.
//
// Same operation as gemm.hip (QUADS abstract: native W4A4 GEMM plus Residual
// Activation Compensation; explainer section 2.2 B; FourSight abstract:
// selected channels effectively BF16):
//   Y[m,n] = sum_k A[m,k] B[n,k] + sum_j R[m,j] B[n,S_j]
// for M, N >= 256.  Design:
//  * 256 x 256 output tile per workgroup of 8 waves (two per SIMD); each
//    wave owns 64 rows x 128 columns as 4 x 8 tiles of 16x16 MFMAs (128 FP32
//    accumulators per lane).
//  * K advances 128 per stage.  Packed FP4 tiles and block scales go from
//    HBM straight into LDS with global_load_lds (no register staging); three
//    stages rotate, two in flight while the third is multiplied.
//  * LDS layout per 16-row group and stage: 16-byte slot (chunk c, row r) at
//    c*16 + r, one global_load_lds_dwordx4 per group, and the MFMA operand
//    read of a wave is 64 consecutive slots (no bank conflicts).
//  * MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4; a lane's 32 K-values are one
//    MX block and its E8M0 code comes from LDS.  NVFP4: E4M3 scales on 16
//    elements and 6-bit products do not fit the FP4/FP8 MFMAs exactly, so
//    each lane decodes its codes to f16 (v_cvt_scalef32_pk_f16_fp4, then
//    v_pk_mul_f16 by the block scale, both exact) for
//    v_mfma_f32_16x16x32_f16.
//  * Compensation: as each B stage passes through LDS, the codes of the
//    selected channels in that K range are decoded to bf16 (e2m1 * block
//    scale, exact) into a 16-channel staging buffer (double buffered); each
//    complete group of 16 channels is multiplied at once with
//    v_mfma_f32_16x16x16_bf16 against R (bf16), which global_load_lds brings
//    into LDS well ahead of use.  MXFP4 accumulates it directly; NVFP4 adds
//    it times 1/t_x so that the final y = (t_x t_w) * acc equals
//    t_w (t_x main + comp).  Weights are read from HBM once.
//  * Workgroup ids are remapped so that the 32 workgroups resident on one
//    XCD (ids congruent mod 8) share a compact block of tiles in L2.
// Rows past M / columns past N load a clamped valid row and are not stored.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef float v4f32 __attribute__((ext_vector_type(4)));
typedef int i32x8b __attribute__((ext_vector_type(8)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2b __attribute__((ext_vector_type(2)));

constexpr int GB_TILE = 256;             // rows (M) and columns (N) per workgroup
constexpr int GB_GRP = 1024;             // bytes per 16-row group per stage
constexpr int GB_DATA = 16 * GB_GRP;     // 16 KB per operand per stage
constexpr int GB_CG = 16;                // channels per compensation group
constexpr int GB_COMP = GB_CG * GB_TILE; // bf16 entries per staging buffer (8 KB)
constexpr int GB_MAX_NS = 1024;          // channel list held in LDS
constexpr int GB_GROUP_M = 4;            // tile rows per L2 group

struct BigArgs {
  int64_t M, N, K;
  const uint8_t* aq;
  const uint8_t* as;
  const float* ats;
  const uint8_t* bq;
  const uint8_t* bs;
  const float* bts;
  const int32_t* chan;
  int nS;
  const uint16_t* resid;
  void* y;
  int y_bf16;
  int64_t ldy;
  int mt, nt;  // tile counts
};

template <int FMT>
struct Stage {
  static constexpr int SC = (FMT == FP4Q_NVFP4) ? 2048 : 1024;  // scale bytes per operand
  uint8_t a[GB_DATA];
  uint8_t b[GB_DATA];
  uint8_t sa[SC];
  uint8_t sb[SC];
};

// Direct-to-LDS loads (global_load_lds): lane l's bytes land at the
// wave-uniform LDS address in M0 plus l * size.  They are issued through
// inline asm so that their completion is governed only by the explicit
// vmcnt waits of the pipeline below; the compiler's own waits for the few
// loads it does see can then only be stricter than needed, never looser.
// M0 is set right before each load and is not used for anything else here.
__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
}
__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_addr(lds)), "v"(g) : "memory");
}
__device__ __forceinline__ void lds_load4(const void* g, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds_addr(lds)), "v"(g) : "memory");
}

__device__ __forceinline__ h16x8 nv_decode8(uint32_t w, h16x2 s) {
  h16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  h16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  h16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  h16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  h16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ h16x2 e4m3_h2(uint32_t code) {
  _Float16 v = (_Float16)e4m3_value(code & 0xFFu);
  return h16x2{v, v};
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those make the compiler wait for every outstanding global load, which
// would drain the load pipeline at each stage.  LDS visibility is handled
// explicitly: this wave's LDS operations complete (lgkmcnt) before it
// arrives, and direct-to-LDS loads are waited for with explicit vmcnt
// counts.  The empty asm statements keep the compiler from moving memory
// operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Loads each wave issues per stage (the explicit vmcnt waits count on it).
template <int FMT>
constexpr int loads_per_stage() { return FMT == FP4Q_NVFP4 ? 6 : 5; }

// Issue the direct-to-LDS loads of one K stage (this wave's share).
// Data: 16 instructions per operand (one per 16-row group g): lane l loads
// row 16g + l%16, 16-byte chunk l/16.  Scales: NVFP4 2 dwords per row stored
// [d][row]; MXFP4 1 dword per row stored [row] (waves 0-3 load the A
// scales, waves 4-7 the B scales).
template <int FMT>
__device__ __forceinline__ void issue_stage(const BigArgs& p, int kt, int wave, int lane,
                                            int64_t r0, int64_t c0, Stage<FMT>& st) {
  const int64_t K2 = p.K >> 1;
  constexpr int BLK = (FMT == FP4Q_NVFP4) ? 16 : 32;
  const int64_t KS = p.K / BLK;
  const int64_t off = (int64_t)kt * 64 + (lane >> 4) * 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int g = wave * 2 + i;
    int64_t ra = r0 + 16 * g + (lane & 15), rb = c0 + 16 * g + (lane & 15);
    ra = ra < p.M ? ra : p.M - 1;
    rb = rb < p.N ? rb : p.N - 1;
    lds_load16(p.aq + ra * K2 + off, st.a + g * GB_GRP);
    lds_load16(p.bq + rb * K2 + off, st.b + g * GB_GRP);
  }
  if (FMT == FP4Q_NVFP4) {
    // 8 instructions per operand, (d, c): rows 64c + lane, dword d
    const int d = wave >> 2, c = wave & 3;
    int64_t ra = r0 + 64 * c + lane, rb = c0 + 64 * c + lane;
    ra = ra < p.M ? ra : p.M - 1;
    rb = rb < p.N ? rb : p.N - 1;
    const int64_t so = (int64_t)kt * 8 + 4 * d;
    lds_load4(p.as + ra * KS + so, st.sa + (d * 256 + 64 * c) * 4);
    lds_load4(p.bs + rb * KS + so, st.sb + (d * 256 + 64 * c) * 4);
  } else {
    const int c = wave & 3;
    const int64_t so = (int64_t)kt * 4;
    if (wave < 4) {
      int64_t ra = r0 + 64 * c + lane;
      ra = ra < p.M ? ra : p.M - 1;
      lds_load4(p.as + ra * KS + so, st.sa + 64 * c * 4);
    } else {
      int64_t rb = c0 + 64 * c + lane;
      rb = rb < p.N ? rb : p.N - 1;
      lds_load4(p.bs + rb * KS + so, st.sb + 64 * c * 4);
    }
  }
}

// Multiply one K stage: the wave covers rows wm*64 .. +64 (4 fragments of
// 16) and columns wn*128 .. +128 (8 fragments).
template <int FMT>
__device__ __forceinline__ void compute_stage(v4f32 (&acc)[4][8], const Stage<FMT>& st, int wm,
                                              int wn, int lane) {
  const int q = lane >> 4, lr = lane & 15;
  if (FMT == FP4Q_MXFP4) {
    u32x4 fa[4];
    int sa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 64 + i * 16 + lr;
      fa[i] = *reinterpret_cast<const u32x4*>(st.a + (wm * 4 + i) * GB_GRP + lane * 16);
      sa[i] = (int)(*reinterpret_cast<const uint32_t*>(st.sa + row * 4) >> (8 * q));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = wn * 128 + j * 16 + lr;
      const u32x4 fb = *reinterpret_cast<const u32x4*>(st.b + (wn * 8 + j) * GB_GRP + lane * 16);
      const int sb = (int)(*reinterpret_cast<const uint32_t*>(st.sb + col * 4) >> (8 * q));
      const i32x8b bv = {(int)fb.x, (int)fb.y, (int)fb.z, (int)fb.w, 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x8b av = {(int)fa[i].x, (int)fa[i].y, (int)fa[i].z, (int)fa[i].w, 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0,
                                                                     sa[i], 0, sb);
      }
    }
  } else {
    // lane q takes chunk q of its row: 32 codes, blocks 2q and 2q+1 (dword
    // q/2 of the scales, bytes (2q)%4 and (2q+1)%4); sub-step s uses dword s
    u32x4 fa[4];
    h16x2 sa[4][2];
    uint32_t sbw[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 64 + i * 16 + lr;
      fa[i] = *reinterpret_cast<const u32x4*>(st.a + (wm * 4 + i) * GB_GRP + lane * 16);
      const uint32_t sw =
          *reinterpret_cast<const uint32_t*>(st.sa + ((q >> 1) * 256 + row) * 4) >> (16 * (q & 1));
      sa[i][0] = e4m3_h2(sw);
      sa[i][1] = e4m3_h2(sw >> 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = wn * 128 + j * 16 + lr;
      sbw[j] =
          *reinterpret_cast<const uint32_t*>(st.sb + ((q >> 1) * 256 + col) * 4) >> (16 * (q & 1));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      h16x8 da[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) da[i] = nv_decode8(fa[i][s], sa[i][s >> 1]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w =
            *reinterpret_cast<const uint32_t*>(st.b + (wn * 8 + j) * GB_GRP + lane * 16 + 4 * s);
        const h16x8 db = nv_decode8(w, e4m3_h2(sbw[j] >> (8 * (s >> 1))));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(da[i], db, acc[i][j], 0, 0, 0);
      }
    }
  }
}

// Decode the code at K offset k (within this stage) of column t of the B
// tile to bf16 into the staging buffer, laid out as the bf16 MFMA's B
// operand: slot (jj/4, column) of 4 values, value jj%4.
template <int FMT>
__device__ __forceinline__ void extract_one(const Stage<FMT>& st, int k, int t, int jj,
                                            uint16_t* comp) {
  const int byte_idx = k >> 1;  // 0..63
  const uint32_t b =
      st.b[(t >> 4) * GB_GRP + ((byte_idx >> 4) * 16 + (t & 15)) * 16 + (byte_idx & 15)];
  const uint32_t code = (k & 1) ? (b >> 4) : (b & 15u);
  float sc;
  if (FMT == FP4Q_NVFP4) {
    const int blkk = k >> 4;  // 0..7
    sc = e4m3_value(st.sb[((blkk >> 2) * 256 + t) * 4 + (blkk & 3)]);
  } else {
    const uint32_t e = st.sb[t * 4 + (k >> 5)];
    sc = e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
  }
  const float v = e2m1_mag_value(code) * sc;
  const uint16_t bits = (uint16_t)((__float_as_uint(v) >> 16) | ((code & 8u) << 12));
  comp[((jj >> 2) * 256 + t) * 4 + (jj & 3)] = bits;
}

// Bring R[rows, channels of group g] into an LDS staging buffer laid out
// [row][16 channels]: wave w loads rows 32w .. 32w+31, two lanes per row.
__device__ __forceinline__ void issue_resid(const BigArgs& p, int64_t r0, int wave, int lane,
                                            int g, uint16_t* rbuf) {
  int64_t row = r0 + 32 * wave + (lane >> 1);
  row = row < p.M ? row : p.M - 1;
  lds_load16(p.resid + row * p.nS + g * GB_CG + 8 * (lane & 1), rbuf + wave * 32 * GB_CG);
}

// acc += (R_group x Wdeq_group) * scale (scale = 1/t_x for NVFP4, 1 for MXFP4).
// A operand: lane takes row lr of each 16-row fragment, channels 4q .. 4q+3.
template <int FMT>
__device__ __forceinline__ void flush_group(v4f32 (&acc)[4][8], const uint16_t* comp,
                                            const uint16_t* rbuf, float scale, int wm, int wn,
                                            int lane) {
  const int q = lane >> 4, lr = lane & 15;
  s16x4 ra[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ra[i] = __builtin_bit_cast(
        s16x4, *reinterpret_cast<const u32x2b*>(rbuf + (wm * 64 + i * 16 + lr) * GB_CG + 4 * q));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const s16x4 rb = __builtin_bit_cast(
        s16x4, *reinterpret_cast<const u32x2b*>(comp + (q * 256 + wn * 128 + j * 16 + lr) * 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (FMT == FP4Q_MXFP4) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ra[i], rb, acc[i][j], 0, 0, 0);
      } else {
        const v4f32 z = {0.f, 0.f, 0.f, 0.f};
        const v4f32 c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ra[i], rb, z, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(c[e], scale, acc[i][j][e]);
      }
    }
  }
}

template <int FMT>
__global__ void __launch_bounds__(512, 1) k_gemm_big(BigArgs p) {
  __shared__ __attribute__((aligned(16))) Stage<FMT> st0, st1, st2;
  __shared__ __attribute__((aligned(16))) uint16_t sComp[2][GB_COMP];
  __shared__ __attribute__((aligned(16))) uint16_t sR[2][GB_COMP];
  __shared__ int sS[GB_MAX_NS];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave tile: rows wm*64, columns wn*128

  // ---- tile id: XCD-aware, then grouped along M for L2 reuse
  const int T = p.mt * p.nt;
  int tile = blockIdx.x;
  if ((T & 7) == 0) tile = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
  const int gsize = GB_GROUP_M * p.nt;
  const int gid = tile / gsize, first_m = gid * GB_GROUP_M;
  const int gm = min(p.mt - first_m, GB_GROUP_M);
  const int pid_m = first_m + (tile % gsize) % gm;
  const int pid_n = (tile % gsize) / gm;
  const int64_t r0 = (int64_t)pid_m * GB_TILE, c0 = (int64_t)pid_n * GB_TILE;

  const int nS = p.nS;
  const int nk = (int)(p.K / 128);
  constexpr int L = loads_per_stage<FMT>();
  float tx = 1.0f, tw = 1.0f, inv_tx = 1.0f;
  if (FMT == FP4Q_NVFP4) {
    tx = *p.ats;
    tw = *p.bts;
    inv_tx = 1.0f / tx;
  }

  // prologue: the first residual group, then two stages in flight; channel
  // list and zeroed staging buffers
  if (nS > 0) issue_resid(p, r0, wave, lane, 0, sR[0]);
  issue_stage<FMT>(p, 0, wave, lane, r0, c0, st0);
  if (nk > 1) issue_stage<FMT>(p, 1, wave, lane, r0, c0, st1);
  if (nS > 0) {
    for (int j = t; j < nS; j += 512) sS[j] = p.chan[j];
    for (int i = t; i < 2 * GB_COMP / 8; i += 512)
      reinterpret_cast<u32x4*>(&sComp[0][0])[i] = u32x4{0u, 0u, 0u, 0u};
  }

  v4f32 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f32{0.f, 0.f, 0.f, 0.f};

  // Compensation bookkeeping is identical in every lane; readfirstlane keeps
  // it in scalar registers so the loops around the barriers below are
  // uniform branches the compiler can see as such.
  int jx = 0;        // channels extracted so far
  int gf = 0;        // compensation groups flushed so far
  int r_iter = -3;   // iteration that issued the residual loads of group gf
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };

  // Flush group gf.  Its residual loads are covered by the pipeline's own
  // waits once three iterations have passed since they were issued;
  // otherwise wait for them explicitly.  Then prefetch the next group's
  // residual into the buffer just freed.
  auto flush = [&](int kt) {
    if (kt < r_iter + 3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    flush_group<FMT>(acc, sComp[gf & 1], sR[gf & 1], inv_tx, wm, wn, lane);
    gf = uni(gf + 1);
    if (gf * GB_CG < nS) {
      lds_barrier();  // every wave is done with the buffer about to be refilled
      issue_resid(p, r0, wave, lane, gf, sR[gf & 1]);
      r_iter = kt;
    }
  };

  // one pipeline step: stage kt sits in `cur`; stage kt+2 goes into `nxt`
  auto step = [&](int kt, Stage<FMT>& cur, Stage<FMT>& nxt) {
    if (kt + 1 < nk)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (kt + 2 < nk) issue_stage<FMT>(p, kt + 2, wave, lane, r0, c0, nxt);
    compute_stage<FMT>(acc, cur, wm, wn, lane);
    if (nS > 0) {
      // channels whose K position lies in this stage (S is ascending)
      const int kbase = kt * 128;
      // number of channels below the end of this stage
      int jend = jx;
      while (jend < nS && uni(sS[jend]) < kbase + 128) jend = uni(jend + 1);
      for (; jx < jend; jx = uni(jx + 1)) {
        const int g = jx / GB_CG;
        if (g >= gf + 2) flush(kt);  // both staging buffers hold unflushed groups
        const int ch = uni(sS[jx]);
        if (ch >= kbase && (t >> 8) == (jx & 1))
          extract_one<FMT>(cur, ch - kbase, t & 255, jx % GB_CG, sComp[g & 1]);
      }
      if (gf * GB_CG + GB_CG <= jx) flush(kt);  // the oldest group is complete
    }
  };

  for (int kt = 0; kt < nk; kt += 3) {
    step(kt, st0, st2);
    if (kt + 1 >= nk) break;
    step(kt + 1, st1, st0);
    if (kt + 2 >= nk) break;
    step(kt + 2, st2, st1);
  }

  // remaining compensation groups (every channel is < K, so all extracted)
  while (gf * GB_CG < nS) flush(nk);

  // ---- epilogue: y = (t_x t_w) * acc; lane holds column lr, rows 4q..4q+3
  // of each 16x16 tile
  const float ys = (FMT == FP4Q_NVFP4) ? tx * tw : 1.0f;
  const int q = lane >> 4, lr = lane & 15;
  const bool interior = (r0 + GB_TILE <= p.M) && (c0 + GB_TILE <= p.N);
  const int64_t rw = r0 + wm * 64 + 4 * q, cw = c0 + wn * 128 + lr;
  if (!p.y_bf16) {
    float* y = reinterpret_cast<float*>(p.y);
    if (interior) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_nontemporal_store(acc[i][j][e] * ys,
                                        y + (rw + i * 16 + e) * p.ldy + cw + j * 16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t row = rw + i * 16 + e, col = cw + j * 16;
            if (row < p.M && col < p.N)
              __builtin_nontemporal_store(acc[i][j][e] * ys, y + row * p.ldy + col);
          }
    }
  } else {
    uint16_t* y = reinterpret_cast<uint16_t*>(p.y);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t row = rw + i * 16 + e, col = cw + j * 16;
          if (interior || (row < p.M && col < p.N))
            y[row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][e] * ys);
        }
  }
}

bool big_gemm_eligible(int64_t M, int64_t N, int64_t K, int nS) {
  return M >= 256 && N >= 256 && K % 128 == 0 && nS <= GB_MAX_NS && nS % GB_CG == 0;
}

int launch_gemm_big(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* aq,
                    const uint8_t* as, const float* ats, const uint8_t* bq, const uint8_t* bs,
                    const float* bts, const int32_t* chan, int nS, const uint16_t* resid,
                    void* y, int y_bf16, int64_t ldy, hipStream_t stream) {
  BigArgs a{M, N, K, aq, as, ats, bq, bs, bts, chan, nS, resid, y, y_bf16, ldy,
            (int)((M + GB_TILE - 1) / GB_TILE), (int)((N + GB_TILE - 1) / GB_TILE)};
  dim3 grid((unsigned)(a.mt * a.nt));
  if (fmt == FP4Q_NVFP4)
    hipLaunchKernelGGL(k_gemm_big<FP4Q_NVFP4>, grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(k_gemm_big<FP4Q_MXFP4>, grid, dim3(512), 0, stream, a);
  return 0;
}

}  // namespace fp4q
