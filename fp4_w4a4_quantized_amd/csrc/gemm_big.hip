// gemm_big.hip -- the prefill-shaped compensated W4A4 GEMM for gfx950.
//
// Same operation as gemm.hip (QUADS abstract: native W4A4 GEMM plus Residual
// Activation Compensation; explainer section 2.2 B; FourSight abstract:
// selected channels effectively BF16):
//   Y[m,n] = sum_k A[m,k] B[n,k] + sum_j R[m,j] B[n,S_j]
// for M, N >= 256.  Design:
//  * 256 x 256 output tile per workgroup of 8 waves (two per SIMD); wave
//    (wm, wn) owns rows 64 wm .. 64 wm + 63 and columns 128 wn .. +127 as
//    2 x 4 blocks of 32 x 32.  The 32x32 MFMA shapes are used throughout:
//    measured on MI355X, v_mfma_scale_f32_32x32x64_f8f6f4 keeps the matrix
//    pipe about 97% busy even from one wave per SIMD, where the 16x16x128
//    form reaches about 70%, and the LDS fragment reads that run beside it
//    are slowed less.
//  * The K loop is a sequence of stages that all look alike to the
//    pipeline: first K/128 FP4 stages (packed codes of A and B plus block
//    scales), then ceil(|S|/32) compensation stages (32 channels of the
//    residual R and of the gathered compensation weights B_S, both BF16).
//    Stages go from memory straight into LDS with global_load_lds (no
//    register staging); three LDS buffers rotate, two stages are in flight
//    and one barrier per stage is the only synchronisation.
//  * LDS layout per 16-row group and stage: 16-byte slot (chunk c, row r)
//    at (16c + r) * 16 -- the tiled operand layout itself, and for BF16
//    stages the same arrangement of 8-channel pieces.  A 32x32 fragment read
//    (rows 32i + (l & 31), chunk 2h + (l >> 5)) is then two contiguous
//    512-byte halves, free of bank conflicts, for all three stage kinds.
//  * MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4; a lane's 32 K-values are one
//    MX block and its E8M0 code comes from LDS.  NVFP4: E4M3 scales on 16
//    elements and 6-bit products do not fit the FP4/FP8 MFMAs exactly, so
//    each lane decodes its codes to f16 (v_cvt_scalef32_pk_f16_fp4, then
//    v_pk_mul_f16 by the block scale, both exact) for
//    v_mfma_f32_32x32x16_f16.  The tensor scales are applied as
//    y = t_w (t_x main + comp).
//  * Compensation: B_S[n, j] = e2m1(B[n, S_j]) * blockscale (exact in
//    BF16, tensor scale excluded) is gathered once per call by a small
//    kernel into a tiled BF16 workspace, so the GEMM streams R and B_S like
//    any other operand and multiplies them with v_mfma_f32_32x32x16_bf16.
//  * Epilogue: each wave stages 32 x 64 pieces of its tile through LDS and
//    writes full 16-byte vectors.
//  * Workgroup ids are remapped so that the workgroups resident on one XCD
//    (ids congruent mod 8) share a compact block of tiles in L2.
//  * Dense NVFP4 with the compensation weights streamed (gathered or
//    prepared) runs on k_gemm_nv4 below: four waves of 128 x 128, which
//    decode a third fewer fragments per MFMA and interleave the decode with
//    their own MFMAs.
// Rows past M / columns past N load a clamped valid row and are not stored.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8b __attribute__((ext_vector_type(8)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8b __attribute__((ext_vector_type(8)));
typedef float f32x4b __attribute__((ext_vector_type(4)));

constexpr int GB_TILE = 256;             // rows (M) and columns (N) per workgroup
constexpr int GB_W = 8;                  // waves per workgroup
constexpr int GB_T = 64 * GB_W;
constexpr int GB_GRP = 1024;             // bytes per 16-row group per stage
constexpr int GB_DATA = 16 * GB_GRP;     // 16 KB per operand per stage
constexpr int GB_CS = 32;                // channels per compensation stage
constexpr int GB_GROUP_M = 4;            // tile rows per L2 group
constexpr int GB_EP_STRIDE = 68;         // epilogue LDS row stride (floats)

struct BigArgs {
  int64_t M, N, K;
  const uint8_t* aq;
  const uint8_t* as;
  const float* ats;
  const uint8_t* bq;
  const uint8_t* bs;
  const float* bts;
  int nS;
  const uint16_t* resid;
  const uint8_t* bsel;  // gathered B_S, tiled BF16 (see k_gather_bsel)
  const int32_t* chan;  // channel lists (not read by the kernels; B_S is gathered)
  const float* cts;     // tensor scale of the compensation term, or null (1)
  void* y;
  int y_bf16;
  int64_t ldy;
  int mt, nt;  // tile counts
  int nk, nc;  // FP4 stages, compensation stages
  // grouped (expert) form: row ranges [off[g], off[g+1]) use operand set g
  const int32_t* off;
  int G;
  // grouped, gathering: row m of A is row row_src[m] of the token matrix
  // (null: row m itself), and every group has the tensor scale ats[0]
  const int32_t* row_src;
};

// The operands and row range of one output tile.  Grouped: B, its scales,
// B_S and the tensor scales of the tile's group.
struct TileCtx {
  int64_t r0, c0, rend;
  const uint8_t* bq;
  const uint8_t* bs;
  const uint8_t* bsel;
  const int* src;  // gathering (GA): the source row of tile row r at src[r] (LDS)
};

// Byte offsets inside one LDS stage and the direct-to-LDS loads a wave
// issues per stage: 2 data groups per operand, then scales (NVFP4 16 dword
// instructions per stage, MXFP4 8, spread over the waves).  Compensation
// stages issue the same count (their scale-slot loads are placeholders), so
// one vmcnt figure serves every stage.
template <int FMT>
struct StageLayout {
  static constexpr int SC = (FMT == FP4Q_NVFP4) ? 2048 : 1024;  // scale bytes per operand
  static constexpr int A = 0;
  static constexpr int B = GB_DATA;
  static constexpr int SA = 2 * GB_DATA;
  static constexpr int SB = 2 * GB_DATA + SC;
  static constexpr int BYTES = 2 * GB_DATA + 2 * SC;
  static constexpr int SCALE_INSTR = (FMT == FP4Q_NVFP4) ? 16 : 8;
  static constexpr int SPW = SCALE_INSTR / GB_W;
  static constexpr int LOADS = 4 + SPW;
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
// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (the tiled layout's loads: block base + 16 l or 4 l).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void lds_load16s(const void* base, uint32_t voff, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr(lds)), "v"(voff), "s"(uniform_ptr(base)) : "memory");
}
__device__ __forceinline__ void lds_load4s(const void* base, uint32_t voff, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds_addr(lds)), "v"(voff), "s"(uniform_ptr(base)) : "memory");
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
// counts.  The lgkmcnt wait is the builtin (simm16 0xC07F: lgkmcnt 0,
// vmcnt and expcnt unconstrained) so that the compiler's wait counting
// knows the LDS reads issued before it are complete.  The scheduling
// barriers keep the compiler from moving any instruction across, so each
// stage's LDS reads and MFMAs stay in their own interval.
// a *= s, an accumulator block kept in its AGPRs: eight values at a time
// are read out, multiplied (the IEEE single product, as a plain multiply
// would give) and written back through eight scratch VGPRs.  Written out
// because in the four-wave kernels the compiler's own form of this step,
// between the main loop and the compensation stages, spilled to scratch
// memory (about 130 bytes per lane and tile) and cost about 10 us per
// prefill GEMM; the eight-wave kernel keeps the plain multiply, which does
// not spill there.
__device__ __forceinline__ void scale_acc(f32x16& a, float s) {
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float t[8];
    asm volatile("v_accvgpr_read_b32 %8, %0\n\tv_accvgpr_read_b32 %9, %1\n\tv_accvgpr_read_b32 %10, %2\n\tv_accvgpr_read_b32 %11, %3\n\tv_accvgpr_read_b32 %12, %4\n\tv_accvgpr_read_b32 %13, %5\n\tv_accvgpr_read_b32 %14, %6\n\tv_accvgpr_read_b32 %15, %7\n\t"
                 "v_mul_f32 %8, %8, %16\n\tv_mul_f32 %9, %9, %16\n\tv_mul_f32 %10, %10, %16\n\tv_mul_f32 %11, %11, %16\n\tv_mul_f32 %12, %12, %16\n\tv_mul_f32 %13, %13, %16\n\tv_mul_f32 %14, %14, %16\n\tv_mul_f32 %15, %15, %16\n\t"
                 "v_accvgpr_write_b32 %0, %8\n\tv_accvgpr_write_b32 %1, %9\n\tv_accvgpr_write_b32 %2, %10\n\tv_accvgpr_write_b32 %3, %11\n\tv_accvgpr_write_b32 %4, %12\n\tv_accvgpr_write_b32 %5, %13\n\tv_accvgpr_write_b32 %6, %14\n\tv_accvgpr_write_b32 %7, %15"
                 : "+a"(a[8 * g + 0]), "+a"(a[8 * g + 1]), "+a"(a[8 * g + 2]), "+a"(a[8 * g + 3]), "+a"(a[8 * g + 4]), "+a"(a[8 * g + 5]), "+a"(a[8 * g + 6]), "+a"(a[8 * g + 7]),
                   "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
                 : "v"(s));
  }
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Issue the direct-to-LDS loads of stage s (this wave's share).
// FP4 stage: 16 instructions per operand, one per 16-row group g: lane l
// loads row 16g + l%16, 16-byte chunk l/16.  Scales: NVFP4 two dwords per
// row stored [d][row]; MXFP4 one dword per row stored [row]; scale
// instruction n covers operand A (first half of n) or B, 64-row chunk n % 4,
// and for NVFP4 dword (n / 4) % 2.  This LDS arrangement is the tiled operand
// layout itself, so with TL each instruction reads one contiguous span (1 KB
// of codes or 256 bytes of scales); row-major operands are gathered from
// rows K/2 bytes apart.
// Compensation stage cs: per 16-row group, R rows (channels 32cs + 8(l/16)
// .. +7 of row 16g + l%16; a piece past |S| is re-read from the last valid
// one and meets zero weights) and the matching 1 KB block of B_S.
template <int FMT, bool TL, bool GA = false>
__device__ __forceinline__ void issue_stage(const BigArgs& p, int s, int wave, int lane,
                                            const TileCtx& tc, uint8_t* st) {
  using SL = StageLayout<FMT>;
  constexpr int SPS = (FMT == FP4Q_NVFP4) ? 8 : 4;  // scale bytes per row per step
  const int64_t r0 = tc.r0, c0 = tc.c0, rend = tc.rend;
  if (s >= p.nk) {
    const int cs = s - p.nk;
    const int64_t gN = ((p.N + 15) >> 4) - 1;
    int ch = GB_CS * cs + 8 * (lane >> 4);
    ch = ch < p.nS - 8 ? ch : p.nS - 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = wave * 2 + i;
      int64_t row = r0 + 16 * g + (lane & 15);
      row = row < rend ? row : rend - 1;
      int64_t gb = (c0 >> 4) + g;
      gb = gb < gN ? gb : gN;
      lds_load16(p.resid + row * p.nS + ch, st + SL::A + g * GB_GRP);
      lds_load16s(tc.bsel + ((gb * p.nc + cs) << 10), lane * 16, st + SL::B + g * GB_GRP);
    }
#pragma unroll
    for (int i = 0; i < SL::SPW; ++i)  // placeholders keeping the per-stage load count
      lds_load4(p.resid, st + SL::SA + (wave * SL::SPW + i) * 256);
    return;
  }
  const int kt = s;
  if (TL) {
    // block indices are wave-uniform (16- or 64-row group, clamped to the
    // last padded group); lane l reads bytes [16 l, 16 l + 16) or [4 l, 4 l + 4)
    const int64_t KB = p.K >> 7;
    const int64_t gM = ((p.M + 15) >> 4) - 1, gN = ((p.N + 15) >> 4) - 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = wave * 2 + i;
      int64_t ga = (r0 >> 4) + g, gb = (c0 >> 4) + g;
      ga = ga < gM ? ga : gM;
      gb = gb < gN ? gb : gN;
      lds_load16s(p.aq + ((ga * KB + kt) << 10), lane * 16, st + SL::A + g * GB_GRP);
      lds_load16s(tc.bq + ((gb * KB + kt) << 10), lane * 16, st + SL::B + g * GB_GRP);
    }
    const int64_t hM = ((p.M + 63) >> 6) - 1, hN = ((p.N + 63) >> 6) - 1;
#pragma unroll
    for (int i = 0; i < SL::SPW; ++i) {
      const int n = wave * SL::SPW + i;
      const int c = n & 3;
      const bool isb = n >= SL::SCALE_INSTR / 2;
      int64_t h = ((isb ? c0 : r0) >> 6) + c;
      const int64_t hl = isb ? hN : hM;
      h = h < hl ? h : hl;
      const uint8_t* src = (isb ? tc.bs : p.as) + (h * KB + kt) * (SPS * 64);
      uint8_t* dst = st + (isb ? SL::SB : SL::SA);
      if (FMT == FP4Q_NVFP4) {
        const int d = (n >> 2) & 1;
        lds_load4s(src + d * 256, lane * 4, dst + (d * 256 + 64 * c) * 4);
      } else {
        lds_load4s(src, lane * 4, dst + 64 * c * 4);
      }
    }
    return;
  }
  const int64_t K2 = p.K >> 1, KS = p.K / (FMT == FP4Q_NVFP4 ? 16 : 32);
  const int64_t off = (int64_t)kt * 64 + (lane >> 4) * 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int g = wave * 2 + i;
    int64_t ra = r0 + 16 * g + (lane & 15), rb = c0 + 16 * g + (lane & 15);
    ra = ra < rend ? ra : rend - 1;
    if (GA) ra = tc.src[ra - r0];
    rb = rb < p.N ? rb : p.N - 1;
    lds_load16(p.aq + ra * K2 + off, st + SL::A + g * GB_GRP);
    lds_load16(tc.bq + rb * K2 + off, st + SL::B + g * GB_GRP);
  }
#pragma unroll
  for (int i = 0; i < SL::SPW; ++i) {
    const int n = wave * SL::SPW + i;
    const int c = n & 3;
    const bool isb = n >= SL::SCALE_INSTR / 2;
    int64_t row = (isb ? c0 : r0) + 64 * c + lane;
    const int64_t lim = isb ? p.N : rend;
    row = row < lim ? row : lim - 1;
    if (GA && !isb) row = tc.src[row - r0];
    const uint8_t* src = isb ? tc.bs : p.as;
    uint8_t* dst = st + (isb ? SL::SB : SL::SA);
    if (FMT == FP4Q_NVFP4) {
      const int d = (n >> 2) & 1;
      lds_load4(src + row * KS + (int64_t)kt * SPS + 4 * d, dst + (d * 256 + 64 * c) * 4);
    } else {
      lds_load4(src + row * KS + (int64_t)kt * SPS, dst + 64 * c * 4);
    }
  }
}

// One stage's operands for one wave, in registers.  Lane l holds, for row
// block i (rows 64 wm + 32 i + (l & 31)) and column block j (columns
// 128 wn + 32 j + (l & 31)), K half h: the 16 bytes of chunk 2h + (l >> 5)
// (FP4: 32 codes, elements 64h + 32(l >> 5) .. +31 of the stage; BF16: 8
// channels).  Scales: MXFP4 the row's dword (byte 2h + (l >> 5) is the
// block of that chunk); NVFP4 the row's dword h (bytes 2(l >> 5) and
// 2(l >> 5) + 1 scale the chunk's two 16-element blocks).  The words are
// kept raw and shifted where they are used.
struct Frag {
  u32x4 a[2][2];
  u32x4 b[4][2];
  uint32_t sa[2][2];
  uint32_t sb[4][2];
};

struct FragT4 {
  u32x4 a[4][2];
  u32x4 b[4][2];
  uint32_t sa[4][2];
  uint32_t sb[4][2];
};

template <int FMT, bool SCALES>
__device__ __forceinline__ void read_frags(const uint8_t* st, const uint8_t* bsrc, int wm, int wn,
                                           int lane, Frag& f) {
  using SL = StageLayout<FMT>;
  const uint32_t l32 =
      (uint32_t)((((lane >> 4) & 1) * GB_GRP) + ((lane >> 5) * 16 + (lane & 15)) * 16);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      f.a[i][h] = *reinterpret_cast<const u32x4*>(st + SL::A + (wm * 4 + 2 * i) * GB_GRP + l32 +
                                                  h * 512);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      f.b[j][h] = *reinterpret_cast<const u32x4*>(bsrc + (wn * 8 + 2 * j) * GB_GRP + l32 + h * 512);
  if (!SCALES) return;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wm * 64 + 32 * i + (lane & 31);
    if (FMT == FP4Q_MXFP4) {
      f.sa[i][0] = *reinterpret_cast<const uint32_t*>(st + SL::SA + row * 4);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        f.sa[i][h] = *reinterpret_cast<const uint32_t*>(st + SL::SA + (h * 256 + row) * 4);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = wn * 128 + 32 * j + (lane & 31);
    if (FMT == FP4Q_MXFP4) {
      f.sb[j][0] = *reinterpret_cast<const uint32_t*>(st + SL::SB + col * 4);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        f.sb[j][h] = *reinterpret_cast<const uint32_t*>(st + SL::SB + (h * 256 + col) * 4);
    }
  }
}

// One FP4 stage into the 2 x 4 accumulator blocks.
template <int FMT>
__device__ __forceinline__ void compute_fp4(f32x16 (&acc)[2][4], const Frag& f, int lane) {
  const int hi = lane >> 5;
  if (FMT == FP4Q_MXFP4) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int sa[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) sa[i] = (int)(f.sa[i][0] >> (8 * (2 * h + hi)));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 bb = f.b[j][h];
        const i32x8b bv = {(int)bb.x, (int)bb.y, (int)bb.z, (int)bb.w, 0, 0, 0, 0};
        const int sb = (int)(f.sb[j][0] >> (8 * (2 * h + hi)));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const u32x4 aa = f.a[i][h];
          const i32x8b av = {(int)aa.x, (int)aa.y, (int)aa.z, (int)aa.w, 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 4, 4, 0,
                                                                      sa[i], 0, sb);
        }
      }
    }
  } else {
    // sub-step (h, s): lane feeds elements 64h + 32hi + 8s .. +7 (block
    // 4h + 2hi + s/2) as K positions 8hi .. 8hi+7 of a 16-deep MFMA step; A
    // and B use the same K permutation, so the sum is unchanged
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int sh = 16 * hi + 8 * (s >> 1);
        h16x8 da[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) da[i] = nv_decode8(f.a[i][h][s], e4m3_h2(f.sa[i][h] >> sh));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const h16x8 db = nv_decode8(f.b[j][h][s], e4m3_h2(f.sb[j][h] >> sh));
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[i], db, acc[i][j], 0, 0, 0);
        }
      }
  }
}

// One compensation stage: 32 channels of R x B_S^T, BF16 products (exact)
// accumulated in FP32.
__device__ __forceinline__ void compute_comp(f32x16 (&acc)[2][4], const Frag& f) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8b bv = __builtin_bit_cast(bf16x8b, f.b[j][h]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8b, f.a[i][h]),
                                                            bv, acc[i][j], 0, 0, 0);
    }
}

// Epilogue of a TM x TN tile.  acc[i][j][e] is row 32 RI wm + 32 i +
// 8 (e / 4) + 4 (l / 32) + e % 4, column 128 wn + 32 j + l % 32, scaled by
// tw on the way out.  Interior tiles are staged through LDS (each wave its
// own 32 x 64 region) and written as 16-byte vectors: rows of 256 bytes
// (FP32) or 128 bytes (BF16); edge tiles store element by element.
template <int RI, int TM = GB_TILE, int TN = GB_TILE>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[RI][4], const BigArgs& p,
                                           int64_t r0, int64_t c0, int64_t rend, int wm, int wn,
                                           int wave, int lane, float tw, uint8_t* sStage) {
  const int hi = lane >> 5, l31 = lane & 31;
  const int64_t rw = r0 + wm * 32 * RI, cw = c0 + wn * 128;
  const bool interior = (r0 + TM <= rend) && (c0 + TN <= p.N);
  const bool vec = interior && (p.ldy % 8) == 0 && (reinterpret_cast<uintptr_t>(p.y) & 15) == 0;
  if (vec) {
    lds_barrier();  // every wave is done with the last stage
    float* ep = reinterpret_cast<float*>(sStage) + wave * 32 * GB_EP_STRIDE;
#pragma unroll
    for (int i = 0; i < RI; ++i)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            ep[(8 * (e >> 2) + 4 * hi + (e & 3)) * GB_EP_STRIDE + 32 * jj + l31] =
                acc[i][2 * jp + jj][e] * tw;
        const int64_t row0 = rw + 32 * i, col0 = cw + 64 * jp;
        if (!p.y_bf16) {
          float* y = reinterpret_cast<float*>(p.y);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int rr = 4 * k + (lane >> 4), cc = 4 * (lane & 15);
            const f32x4b v = *reinterpret_cast<const f32x4b*>(ep + rr * GB_EP_STRIDE + cc);
            __builtin_nontemporal_store(
                v, reinterpret_cast<f32x4b*>(y + (row0 + rr) * p.ldy + col0 + cc));
          }
        } else {
          uint16_t* y = reinterpret_cast<uint16_t*>(p.y);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rr = 8 * k + (lane >> 3), cc = 8 * (lane & 7);
            const f32x4b v0 = *reinterpret_cast<const f32x4b*>(ep + rr * GB_EP_STRIDE + cc);
            const f32x4b v1 = *reinterpret_cast<const f32x4b*>(ep + rr * GB_EP_STRIDE + cc + 4);
            const u32x4 w = {f32_to_bf16_rne(v0.x) | (f32_to_bf16_rne(v0.y) << 16),
                             f32_to_bf16_rne(v0.z) | (f32_to_bf16_rne(v0.w) << 16),
                             f32_to_bf16_rne(v1.x) | (f32_to_bf16_rne(v1.y) << 16),
                             f32_to_bf16_rne(v1.z) | (f32_to_bf16_rne(v1.w) << 16)};
            __builtin_nontemporal_store(
                w, reinterpret_cast<u32x4*>(y + (row0 + rr) * p.ldy + col0 + cc));
          }
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = rw + 32 * i + 8 * (e >> 2) + 4 * hi + (e & 3);
        const int64_t col = cw + 32 * j + l31;
        if (row < rend && col < p.N) {
          const float v = acc[i][j][e] * tw;
          if (p.y_bf16)
            reinterpret_cast<uint16_t*>(p.y)[row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
          else
            reinterpret_cast<float*>(p.y)[row * p.ldy + col] = v;
        }
      }
}

// The compensation weights B_S stream through the compensation stages, from
// the prepared array or gathered once per call (k_gather_bsel).
// GR: 0 dense, 1 grouped, 2 grouped with the rows of A gathered by row_src
// (a separate instance, so the plain grouped kernel keeps its registers).
template <int FMT, bool TL, int GR>
__global__ void __launch_bounds__(GB_T, 1) k_gemm_big(BigArgs args) {
  using SL = StageLayout<FMT>;
  constexpr int L = SL::LOADS;
  __shared__ __attribute__((aligned(16))) uint8_t sStage[3 * SL::BYTES];
  static_assert(GB_W * 32 * GB_EP_STRIDE * 4 <= 3 * SL::BYTES, "epilogue staging");

  const BigArgs& p = args;
  // the wave index is made visibly uniform, so block-address arithmetic
  // stays in scalar registers
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  TileCtx tc;
  int grp = 0;
  if (GR) {
    // Tiles in group order, then M, then N (the N tiles of one 256-row
    // block of A run together): group g has ceil(rows_g / 256) * nt tiles.
    // Find this workgroup's group by a block-wide scan over per-thread runs
    // of 4 groups (G <= 2048).
    __shared__ int s_wsum[GB_W];
    __shared__ int s_tile[2];
    const int G = p.G;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int gg = t * 4 + i;
      if (gg < G) cnt += (p.off[gg + 1] - p.off[gg] + GB_TILE - 1) / GB_TILE * p.nt;
    }
    int incl = cnt;
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    if (lane == 63) s_wsum[wave] = incl;
    if (t == 0) s_tile[0] = -1;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_wsum[w];
    const int excl = before + incl - cnt;
    const int tile = blockIdx.x;
    if (tile >= excl && tile < excl + cnt) {
      int acc0 = excl;
      for (int i = 0; i < 4; ++i) {
        const int gg = t * 4 + i;
        const int c = (gg < G) ? (p.off[gg + 1] - p.off[gg] + GB_TILE - 1) / GB_TILE * p.nt : 0;
        if (tile < acc0 + c) {
          s_tile[0] = gg;
          s_tile[1] = tile - acc0;
          break;
        }
        acc0 += c;
      }
    }
    __syncthreads();
    if (s_tile[0] < 0) return;  // past the last tile: uniform exit
    grp = s_tile[0];
    const int local = s_tile[1];
    tc.r0 = (int64_t)p.off[grp] + (int64_t)(local / p.nt) * GB_TILE;
    tc.c0 = (int64_t)(local % p.nt) * GB_TILE;
    tc.rend = p.off[grp + 1];
    const int blk = (FMT == FP4Q_NVFP4) ? 16 : 32;
    tc.bq = p.bq + (int64_t)grp * p.N * (p.K >> 1);
    tc.bs = p.bs + (int64_t)grp * p.N * (p.K / blk);
    tc.bsel = p.bsel + (int64_t)grp * ((p.N + 15) / 16) * p.nc * 1024;
    tc.src = nullptr;
    if (GR == 2) {
      // the tile's source rows (rows past the group repeat its last row)
      __shared__ int sSrc[GB_TILE];
      const int64_t rr = tc.r0 + t;
      if (t < GB_TILE) sSrc[t] = p.row_src[rr < tc.rend ? rr : tc.rend - 1];
      __syncthreads();
      tc.src = sSrc;
    }
  } else {
    // XCD-aware, then grouped along M for L2 reuse
    const int T = p.mt * p.nt;
    int tile = blockIdx.x;
    if ((T & 7) == 0) tile = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
    const int gsize = GB_GROUP_M * p.nt;
    const int gid = tile / gsize, first_m = gid * GB_GROUP_M;
    const int gm = min(p.mt - first_m, GB_GROUP_M);
    const int pid_m = first_m + (tile % gsize) % gm;
    const int pid_n = (tile % gsize) / gm;
    tc.r0 = (int64_t)pid_m * GB_TILE;
    tc.c0 = (int64_t)pid_n * GB_TILE;
    tc.rend = p.M;
    tc.bq = p.bq;
    tc.bs = p.bs;
    tc.bsel = p.bsel;
    tc.src = nullptr;
  }
  const int64_t r0 = tc.r0, c0 = tc.c0;

  const int nk = p.nk, ns = p.nk + p.nc;
  // y = t_w (t_x main + c comp), run as (t_w c) ((t_x / c) main + comp):
  // with c = 1 both factors are exactly t_w and t_x
  float tx = 1.0f, tw = 1.0f;
  if (FMT == FP4Q_NVFP4) {
    const float c = p.cts ? p.cts[GR ? grp : 0] : 1.0f;
    tx = p.ats[GR == 2 ? 0 : grp] / c;
    tw = p.bts[grp] * c;
  }
  auto stage = [&](int s) __attribute__((always_inline)) { return sStage + (s % 3) * SL::BYTES; };

  // MXFP4 runs the two waves of each SIMD half a stage apart (below); only
  // waves 0..3 load, each the share of two waves
  const bool late = FMT == FP4Q_MXFP4 && wave >= GB_W / 2;
  auto issue = [&](int s) __attribute__((always_inline)) {
    if (FMT == FP4Q_MXFP4) {
      issue_stage<FMT, TL, GR == 2>(p, s, 2 * wave, lane, tc, stage(s));
      issue_stage<FMT, TL, GR == 2>(p, s, 2 * wave + 1, lane, tc, stage(s));
    } else {
      issue_stage<FMT, TL, GR == 2>(p, s, wave, lane, tc, stage(s));
    }
  };
  if (!late) {
    issue(0);
    if (ns > 1) issue(1);
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Stage s: wait for its loads, barrier (it landed everywhere; the buffer
  // of stage s-1 is free), issue stage s+2, then read and multiply stage s.
  // The second wave on the SIMD covers this wave's LDS read latency.  The
  // FP4 and the compensation stages run as two loops (one loop with both
  // bodies makes the register allocator spill).
  auto pipe = [&](int s) __attribute__((always_inline)) {
    if (s + 1 < ns)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (s + 2 < ns) issue_stage<FMT, TL, GR == 2>(p, s + 2, wave, lane, tc, stage(s + 2));
  };
  if constexpr (FMT == FP4Q_MXFP4) {
    // Ping-pong.  Each stage is two barrier intervals: LDS fragment reads,
    // then MFMAs.  Waves 4..7 (the second wave of each SIMD) pass one extra
    // barrier first, so they multiply while the first wave of their SIMD
    // reads, and read while it multiplies: a wave's own LDS reads do not
    // overlap its MFMAs, but they do overlap the other wave's, so the matrix
    // pipe stays busy.  Waves 0..3 issue all loads and wait for them before
    // the barrier that opens a stage's read interval, so the stage has
    // landed for both groups.  The buffer of stage s - 1 is free once the
    // late waves have read it, which is before that barrier too.
    constexpr int L2 = 2 * L;
    auto open = [&](int s) __attribute__((always_inline)) {
      if (!late) {
        if (s + 1 < ns)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L2) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();
      if (!late && s + 2 < ns) issue(s + 2);
    };
    if (late) lds_barrier();
    for (int s = 0; s < nk; ++s) {
      open(s);
      Frag f;
      read_frags<FMT, true>(stage(s), stage(s) + SL::B, wm, wn, lane, f);
      lds_barrier();
      compute_fp4<FMT>(acc, f, lane);
    }
    for (int s = nk; s < ns; ++s) {
      open(s);
      Frag f;
      read_frags<FMT, false>(stage(s), stage(s) + SL::B, wm, wn, lane, f);
      lds_barrier();
      compute_comp(acc, f);
    }
    if (!late) lds_barrier();
  } else {
    for (int s = 0; s < nk; ++s) {
      pipe(s);
      Frag f;
      read_frags<FMT, true>(stage(s), stage(s) + SL::B, wm, wn, lane, f);
      compute_fp4<FMT>(acc, f, lane);
    }
    // y = t_w (t_x main + comp): scale the main sum once, before R B_S
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] *= tx;
    for (int s = nk; s < ns; ++s) {
      pipe(s);
      Frag f;
      read_frags<FMT, false>(stage(s), stage(s) + SL::B, wm, wn, lane, f);
      compute_comp(acc, f);
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    }
  }

  // ---- epilogue
  store_tile<2>(acc, p, r0, c0, tc.rend, wm, wn, wave, lane, tw, sStage);
}

// ---- dense NVFP4, four waves ----------------------------------------------------
//
// The exact NVFP4 decode (v_cvt_scalef32_pk_f16_fp4 then v_pk_mul_f16 by the
// block scale) costs about 6 clocks per element and wave on gfx950, as much
// per stage as the f16 MFMAs, so the redundancy of decoding matters: a wave
// owning 64 x 128 of the tile decodes 6 fragments per 8 MFMAs.  Here four
// waves, one per SIMD, own 128 x 128 each (4 x 4 blocks of 32 x 32,
// accumulators in the AGPRs): 8 fragments per 16 MFMAs.  A wave's VALU work
// overlaps its own MFMAs when the two are interleaved, so the decode of
// sub-step n + 1 is placed between the 16 MFMAs of sub-step n (scheduling
// groups of one MFMA and a few VALU instructions).  Stages, direct-to-LDS
// loads, the compensation stages and the epilogue are those of k_gemm_big.
struct NvDec4 {
  h16x8 a[4];
  h16x8 b[4];
};

__device__ __forceinline__ void nv4_decode(const FragT4& f, const h16x2 (&sca)[4][2],
                                           const h16x2 (&scb)[4][2], int n, NvDec4& d) {
  const int h = n >> 2, st = n & 3, k = st >> 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d.a[i] = nv_decode8(f.a[i][h][st], h16x2{sca[i][h][k], sca[i][h][k]});
#pragma unroll
  for (int j = 0; j < 4; ++j)
    d.b[j] = nv_decode8(f.b[j][h][st], h16x2{scb[j][h][k], scb[j][h][k]});
}

// Half h of a stage's fragments (the 16-byte pieces and scale dwords).
__device__ __forceinline__ void nv4_read_half(const uint8_t* st, int wm, int wn, int lane, int h,
                                              FragT4& f) {
  using SL = StageLayout<FP4Q_NVFP4>;
  const uint32_t l32 =
      (uint32_t)((((lane >> 4) & 1) * GB_GRP) + ((lane >> 5) * 16 + (lane & 15)) * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i][h] = *reinterpret_cast<const u32x4*>(st + SL::A + (wm * 8 + 2 * i) * GB_GRP + l32 +
                                                h * 512);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.b[j][h] = *reinterpret_cast<const u32x4*>(st + SL::B + (wn * 8 + 2 * j) * GB_GRP + l32 +
                                                h * 512);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.sa[i][h] = *reinterpret_cast<const uint32_t*>(
        st + SL::SA + (h * 256 + wm * 128 + 32 * i + (lane & 31)) * 4);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.sb[j][h] = *reinterpret_cast<const uint32_t*>(
        st + SL::SB + (h * 256 + wn * 128 + 32 * j + (lane & 31)) * 4);
}

// The lane's two block scales of half h, as f16 (exact for every E4M3 code).
__device__ __forceinline__ void nv4_scales(const FragT4& f, int h, int lane, h16x2 (&sca)[4][2],
                                           h16x2 (&scb)[4][2]) {
  const int hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    sca[i][h] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.sa[i][h] >> (16 * hi), 1.0f, false);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    scb[j][h] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.sb[j][h] >> (16 * hi), 1.0f, false);
}

// The 16 MFMAs of one sub-step, with the VALU instructions placed before
// them in program order (the next decode) spread between them.
__device__ __forceinline__ void nv4_mma(f32x16 (&acc)[4][4], const NvDec4& d) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(d.a[i], d.b[j], acc[i][j], 0, 0, 0);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
  }
}

__device__ __forceinline__ void comp4_stage(f32x16 (&acc)[4][4], const uint8_t* st,
                                            const uint8_t* bsrc, int wm, int wn, int lane) {
  using SL = StageLayout<FP4Q_NVFP4>;
  const uint32_t l32 =
      (uint32_t)((((lane >> 4) & 1) * GB_GRP) + ((lane >> 5) * 16 + (lane & 15)) * 16);
  u32x4 a[4][2], b[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      a[i][h] = *reinterpret_cast<const u32x4*>(st + SL::A + (wm * 8 + 2 * i) * GB_GRP + l32 +
                                                h * 512);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      b[j][h] = *reinterpret_cast<const u32x4*>(bsrc + (wn * 8 + 2 * j) * GB_GRP + l32 + h * 512);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8b, a[i][h]), __builtin_bit_cast(bf16x8b, b[j][h]), acc[i][j],
            0, 0, 0);
}

template <bool TL>
__global__ void __launch_bounds__(256, 1) k_gemm_nv4(BigArgs args) {
  using SL = StageLayout<FP4Q_NVFP4>;
  constexpr int L = 2 * SL::LOADS;  // each wave issues the share of two
  __shared__ __attribute__((aligned(16))) uint8_t sStage[3 * SL::BYTES];
  const BigArgs& p = args;
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile order, grouped along M for L2 reuse (as k_gemm_big)
  TileCtx tc;
  {
    const int T = p.mt * p.nt;
    int tile = blockIdx.x;
    if ((T & 7) == 0) tile = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
    const int gsize = GB_GROUP_M * p.nt;
    const int gid = tile / gsize, first_m = gid * GB_GROUP_M;
    const int gm = min(p.mt - first_m, GB_GROUP_M);
    tc.r0 = (int64_t)(first_m + (tile % gsize) % gm) * GB_TILE;
    tc.c0 = (int64_t)((tile % gsize) / gm) * GB_TILE;
    tc.rend = p.M;
    tc.bq = p.bq;
    tc.bs = p.bs;
    tc.bsel = p.bsel;
    tc.src = nullptr;
  }
  const int nk = p.nk, ns = p.nk + p.nc;
  const float c = p.cts ? *p.cts : 1.0f;
  const float tx = p.ats[0] / c, tw = p.bts[0] * c;
  auto stage = [&](int s) __attribute__((always_inline)) { return sStage + (s % 3) * SL::BYTES; };
  auto issue = [&](int s) __attribute__((always_inline)) {
    issue_stage<FP4Q_NVFP4, TL, false>(p, s, 2 * wave, lane, tc, stage(s));
    issue_stage<FP4Q_NVFP4, TL, false>(p, s, 2 * wave + 1, lane, tc, stage(s));
  };
  issue(0);
  if (ns > 1) issue(1);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto open = [&](int s) __attribute__((always_inline)) {
    if (s + 1 < ns)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (s + 2 < ns) issue(s + 2);
  };
  // stage s: wait for its loads, barrier (it landed everywhere; the buffer
  // of stage s - 1 is free), issue stage s + 2, read it, then decode ahead
  // of the MFMAs sub-step by sub-step
  for (int s = 0; s < nk; ++s) {
    open(s);
    FragT4 f;
    nv4_read_half(stage(s), wm, wn, lane, 0, f);
    nv4_read_half(stage(s), wm, wn, lane, 1, f);
    h16x2 sca[4][2], scb[4][2];
    nv4_scales(f, 0, lane, sca, scb);
    nv4_scales(f, 1, lane, sca, scb);
    NvDec4 cur, nxt;
    nv4_decode(f, sca, scb, 0, cur);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      __builtin_amdgcn_sched_barrier(0);
      if (n < 7) nv4_decode(f, sca, scb, n + 1, nxt);
      nv4_mma(acc, cur);
      cur = nxt;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // y = t_w (t_x main + comp): scale the main sum once, before R B_S
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) scale_acc(acc[i][j], tx);
  for (int s = nk; s < ns; ++s) {
    open(s);
    comp4_stage(acc, stage(s), stage(s) + SL::B, wm, wn, lane);
  }
  store_tile<4>(acc, p, tc.r0, tc.c0, tc.rend, wm, wn, wave, lane, tw, sStage);
}


// ---- grouped NVFP4: 128 x 512 tiles on four waves ---------------------------
// The expert-grouped form of k_gemm_nv4 (QUADS abstract: MoE rollout; the
// same Y = A B^T + R[:, S] B_S^T per group).  The groups of a mixture-of-
// experts layer are small and uneven, so rows are tiled by 128, not 256
// (fewer MFMAs on padding rows), and the four waves sit side by side along
// N, each owning 128 x 128 exactly as in k_gemm_nv4 (same decode work per
// MFMA).  The expert-ordered activations are row-major: every direct-to-LDS
// load takes a wave-uniform base (tile origin and K step, in SGPRs) plus a
// 32-bit lane offset fixed for the whole tile, so the row addressing holds
// few VGPRs.  The experts' weights are row-major, or (TW) each expert's in
// the tiled layout, where a stage's 16 columns are one contiguous 1 KB block
// and 64 columns' scales one 512-byte block; both layouts put the same bytes
// in LDS.
// Tiles run group by group, row tile by row tile, the N tiles of one row
// tile together, and each XCD (block b runs on XCD b % 8) takes one
// contiguous run of that order: the weight panels of a group and the code
// rows of a row tile are shared inside one L2.
constexpr int G4_TM = 128, G4_TN = 512;

struct G4Layout {
  static constexpr int A = 0;                        // 8 groups of 16 rows, 1 KB each
  static constexpr int B = 8 * GB_GRP;               // 32 groups of 16 columns
  static constexpr int SA = 40 * GB_GRP;             // scale dwords [d][row], 2 x 128
  static constexpr int SB = SA + 2 * G4_TM * 4;      // scale dwords [d][col], 2 x 512
  static constexpr int BYTES = SB + 2 * G4_TN * 4;   // 46080
  static constexpr int LOADS = 2 + 8 + 5;            // per wave and stage
};

// This wave's loads of stage s: A groups 2w, 2w + 1; B groups 8w .. 8w + 7;
// scale instructions 5w .. 5w + 4 of 20 (4 for A: dword d, 64-row chunk c;
// 16 for B).  Compensation stages load R pieces and the prepared B_S blocks
// into the same places, and placeholders keep the count.  GA (rows of A
// gathered by row_src): the lane's A code offsets gao[i] (group 2w + i) and
// scale offsets gso[c] (chunk c) from the token matrix's base, fixed per tile.
// TW: the expert's weights in the tiled layout (blocks clamped to the last
// padded 16- or 64-column group, as the dense tiled path does).
template <bool GA, bool TW>
__device__ __forceinline__ void g4_issue(const BigArgs& p, int s, int wave, int lane,
                                         const TileCtx& tc, uint8_t* st, const uint32_t (&gao)[2],
                                         const uint32_t (&gso)[2]) {
  using GL = G4Layout;
  const int64_t r0 = tc.r0, c0 = tc.c0;
  const int rlast = (int)(tc.rend - 1 - r0), clast = (int)(p.N - 1 - c0);
  if (s >= p.nk) {
    const int cs = s - p.nk;
    const int64_t gN = ((p.N + 15) >> 4) - 1;
    int ch = GB_CS * cs + 8 * (lane >> 4);
    ch = ch < p.nS - 8 ? ch : p.nS - 8;
    const uint16_t* rb = p.resid + r0 * p.nS;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = 2 * wave + i;
      int r = 16 * g + (lane & 15);
      r = r < rlast ? r : rlast;
      lds_load16s(rb, (uint32_t)((r * p.nS + ch) * 2), st + GL::A + g * GB_GRP);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = 8 * wave + i;
      int64_t gb = (c0 >> 4) + g;
      gb = gb < gN ? gb : gN;
      lds_load16s(tc.bsel + ((gb * p.nc + cs) << 10), lane * 16, st + GL::B + g * GB_GRP);
    }
#pragma unroll
    for (int i = 0; i < 5; ++i) lds_load4(p.resid, st + GL::SA + (wave * 5 + i) * 256);
    return;
  }
  const int kt = s;
  const int64_t K2 = p.K >> 1, KS = p.K >> 4;
  const uint8_t* ab = p.aq + (GA ? 0 : r0 * K2) + kt * 64;
  const uint8_t* bb = tc.bq + c0 * K2 + kt * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int g = 2 * wave + i;
    int r = 16 * g + (lane & 15);
    r = r < rlast ? r : rlast;
    lds_load16s(ab, GA ? gao[i] : (uint32_t)(r * K2 + (lane >> 4) * 16), st + GL::A + g * GB_GRP);
  }
  const int64_t KB = p.K >> 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int g = 8 * wave + i;
    if (TW) {
      const int64_t gN = ((p.N + 15) >> 4) - 1;
      int64_t gb = (c0 >> 4) + g;
      gb = gb < gN ? gb : gN;
      lds_load16s(tc.bq + ((gb * KB + kt) << 10), lane * 16, st + GL::B + g * GB_GRP);
    } else {
      int r = 16 * g + (lane & 15);
      r = r < clast ? r : clast;
      lds_load16s(bb, (uint32_t)(r * K2 + (lane >> 4) * 16), st + GL::B + g * GB_GRP);
    }
  }
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int n = 5 * wave + i;
    if (n < 4) {
      const int d = n >> 1, c = n & 1;
      int r = 64 * c + lane;
      r = r < rlast ? r : rlast;
      lds_load4s(p.as + (GA ? 0 : r0 * KS) + kt * 8 + 4 * d, GA ? gso[c] : (uint32_t)(r * KS),
                 st + GL::SA + (d * G4_TM + 64 * c) * 4);
    } else {
      const int m = n - 4, d = m >> 3, c = m & 7;
      if (TW) {
        const int64_t hN = ((p.N + 63) >> 6) - 1;
        int64_t h = (c0 >> 6) + c;
        h = h < hN ? h : hN;
        lds_load4s(tc.bs + (h * KB + kt) * 512 + d * 256, lane * 4,
                   st + GL::SB + (d * G4_TN + 64 * c) * 4);
      } else {
        int r = 64 * c + lane;
        r = r < clast ? r : clast;
        lds_load4s(tc.bs + c0 * KS + kt * 8 + 4 * d, (uint32_t)(r * KS),
                   st + GL::SB + (d * G4_TN + 64 * c) * 4);
      }
    }
  }
}

// Half h of a stage's fragments for wave w (all 128 rows, columns 128 w ..).
__device__ __forceinline__ void g4_read_half(const uint8_t* st, int wave, int lane, int h,
                                             FragT4& f) {
  using GL = G4Layout;
  const uint32_t l32 =
      (uint32_t)((((lane >> 4) & 1) * GB_GRP) + ((lane >> 5) * 16 + (lane & 15)) * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i][h] = *reinterpret_cast<const u32x4*>(st + GL::A + (2 * i) * GB_GRP + l32 + h * 512);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.b[j][h] = *reinterpret_cast<const u32x4*>(st + GL::B + (wave * 8 + 2 * j) * GB_GRP + l32 +
                                                h * 512);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.sa[i][h] = *reinterpret_cast<const uint32_t*>(
        st + GL::SA + (h * G4_TM + 32 * i + (lane & 31)) * 4);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.sb[j][h] = *reinterpret_cast<const uint32_t*>(
        st + GL::SB + (h * G4_TN + wave * 128 + 32 * j + (lane & 31)) * 4);
}

template <bool GA, bool TW>
__global__ void __launch_bounds__(256, 1) k_gemm_nv4g(BigArgs args) {
  using GL = G4Layout;
  constexpr int L = GL::LOADS;
  __shared__ __attribute__((aligned(16))) uint8_t sStage[3 * GL::BYTES];
  __shared__ int s_wsum[4];
  __shared__ int s_tile[2];
  const BigArgs& p = args;
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);

  // tiles per group: ceil(rows / 128) * nt; thread t counts groups 8t .. 8t + 7
  // (G <= 2048), a block-wide scan gives every thread its first tile
  const int G = p.G, nt = p.nt;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int gg = t * 8 + i;
    if (gg < G) cnt += (p.off[gg + 1] - p.off[gg] + G4_TM - 1) / G4_TM * nt;
  }
  int incl = cnt;
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == 63) s_wsum[wave] = incl;
  if (t == 0) s_tile[0] = -1;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? s_wsum[w] : 0;
    total += s_wsum[w];
  }
  const int b = blockIdx.x;
  if (b >= total) return;  // past the last tile: uniform exit
  // XCD x (blocks b = 8 idx + x) takes the contiguous run of tiles
  // [x base + min(x, rem), ...) of length base + (x < rem)
  const int base = total >> 3, rem = total & 7, x = b & 7;
  const int tile = x * base + (x < rem ? x : rem) + (b >> 3);
  const int excl = before + incl - cnt;
  if (tile >= excl && tile < excl + cnt) {
    int acc0 = excl;
    for (int i = 0; i < 8; ++i) {
      const int gg = t * 8 + i;
      const int c = (gg < G) ? (p.off[gg + 1] - p.off[gg] + G4_TM - 1) / G4_TM * nt : 0;
      if (tile < acc0 + c) {
        s_tile[0] = gg;
        s_tile[1] = tile - acc0;
        break;
      }
      acc0 += c;
    }
  }
  __syncthreads();
  const int grp = s_tile[0], local = s_tile[1];
  TileCtx tc;
  tc.r0 = (int64_t)p.off[grp] + (int64_t)(local / nt) * G4_TM;
  tc.c0 = (int64_t)(local % nt) * G4_TN;
  tc.rend = p.off[grp + 1];
  // one expert's weights: N (tiled: N padded to 16 / 64) rows of K/2 code
  // bytes and K/16 scale bytes
  tc.bq = p.bq + (int64_t)grp * (TW ? (p.N + 15) & ~(int64_t)15 : p.N) * (p.K >> 1);
  tc.bs = p.bs + (int64_t)grp * (TW ? (p.N + 63) & ~(int64_t)63 : p.N) * (p.K >> 4);
  tc.bsel = p.bsel + (int64_t)grp * ((p.N + 15) / 16) * p.nc * 1024;
  tc.src = nullptr;
  // gathering: this lane's source rows of the tile (rows past the group
  // repeat its last row), as byte offsets into the token matrix's codes and
  // scales (the host keeps them below 2^32)
  uint32_t gao[2] = {0, 0}, gso[2] = {0, 0};
  if (GA) {
    const int64_t K2 = p.K >> 1, KS = p.K >> 4;
    const int rlast = (int)(tc.rend - 1 - tc.r0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int r = 16 * (2 * wave + i) + (lane & 15);
      r = r < rlast ? r : rlast;
      gao[i] = (uint32_t)(p.row_src[tc.r0 + r] * K2 + (lane >> 4) * 16);
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      int r = 64 * cc + lane;
      r = r < rlast ? r : rlast;
      gso[cc] = (uint32_t)(p.row_src[tc.r0 + r] * KS);
    }
  }

  const int nk = p.nk, ns = p.nk + p.nc;
  const float c = p.cts ? p.cts[grp] : 1.0f;
  // gathered rows share the token matrix's one tensor scale
  const float tx = p.ats[GA ? 0 : grp] / c, tw = p.bts[grp] * c;
  auto stage = [&](int s) __attribute__((always_inline)) { return sStage + (s % 3) * GL::BYTES; };
  auto issue = [&](int s) __attribute__((always_inline)) {
    g4_issue<GA, TW>(p, s, wave, lane, tc, stage(s), gao, gso);
  };
  issue(0);
  if (ns > 1) issue(1);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto open = [&](int s) __attribute__((always_inline)) {
    if (s + 1 < ns)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (s + 2 < ns) issue(s + 2);
  };
  for (int s = 0; s < nk; ++s) {
    open(s);
    FragT4 f;
    g4_read_half(stage(s), wave, lane, 0, f);
    g4_read_half(stage(s), wave, lane, 1, f);
    h16x2 sca[4][2], scb[4][2];
    nv4_scales(f, 0, lane, sca, scb);
    nv4_scales(f, 1, lane, sca, scb);
    NvDec4 cur, nxt;
    nv4_decode(f, sca, scb, 0, cur);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      __builtin_amdgcn_sched_barrier(0);
      if (n < 7) nv4_decode(f, sca, scb, n + 1, nxt);
      nv4_mma(acc, cur);
      cur = nxt;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) scale_acc(acc[i][j], tx);
  for (int s = nk; s < ns; ++s) {
    open(s);
    comp4_stage(acc, stage(s), stage(s) + G4Layout::B, 0, wave, lane);
  }
  store_tile<4, G4_TM, G4_TN>(acc, p, tc.r0, tc.c0, tc.rend, 0, wave, wave, lane, tw, sStage);
}

// ---- B_S gather ---------------------------------------------------------------
// bsel holds B_S[n, j] (bf16 bits of e2m1 * block scale, tensor scale
// excluded; exact) for n < ceil16(N), j < ceil32(|S|), zero past N or |S|,
// as 1 KB blocks per (16-row group G, 32-channel chunk C) at (G nc + C) * 1024,
// inside which channels 8c .. 8c+7 of row 16G + r are the 16 bytes at
// (16c + r) * 16.  Grouped: one such array per group, back to back, from
// the group's weights and channel list.  One wave writes one block; lane
// l = 16c + r.
template <int FMT, bool TL>
__global__ void __launch_bounds__(256) k_gather_bsel(const uint8_t* __restrict__ bq,
                                                     const uint8_t* __restrict__ bs, int64_t N,
                                                     int64_t K, const int32_t* __restrict__ chan,
                                                     int nS, int nc, int64_t nblocks, int G,
                                                     uint8_t* __restrict__ bsel) {
  constexpr int BLK = (FMT == FP4Q_NVFP4) ? 16 : 32;
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks * G) return;
  const int64_t grp = blk / nblocks, lb = blk - grp * nblocks;
  // a group's weights: N rows (tiled: N padded to 16 for codes, 64 for scales)
  const uint8_t* gq = bq + grp * (TL ? (N + 15) & ~(int64_t)15 : N) * (K >> 1);
  const uint8_t* gs = bs + grp * (TL ? (N + 63) & ~(int64_t)63 : N) * (K / BLK);
  const int32_t* gc = chan + grp * nS;
  const int64_t Gr = lb / nc;
  const int C = (int)(lb - Gr * nc);
  const int64_t n = 16 * Gr + (lane & 15);
  const int64_t nn = n < N ? n : N - 1;
  const int j0 = GB_CS * C + 8 * (lane >> 4);
  // every load is unconditional (clamped row and channel), so all of a
  // lane's loads are in flight together; out-of-range entries become 0
  int c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) c[e] = gc[j0 + e < nS ? j0 + e : nS - 1];
  uint32_t byte[8], sc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    byte[e] = gq[code_off(TL, nn, c[e] >> 1, K)];
    sc[e] = gs[scale_off<FMT>(TL, nn, c[e] / BLK, K)];
  }
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t code = (c[e] & 1) ? (byte[e] >> 4) : (byte[e] & 15u);
    const float s = (FMT == FP4Q_NVFP4)
                        ? e4m3_value(sc[e])
                        : (sc[e] ? __uint_as_float(sc[e] << 23) : __uint_as_float(0x00400000u));
    const float v = e2m1_mag_value(code) * s;
    const uint32_t bits = (__float_as_uint(v) >> 16) | ((code & 8u) << 12);
    h[e] = (j0 + e < nS && n < N) ? bits : 0u;
  }
  const u32x4 w = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                   h[6] | (h[7] << 16)};
  *reinterpret_cast<u32x4*>(bsel + (blk << 10) + lane * 16) = w;
}

// ---- host side ---------------------------------------------------------------

// Residual rows are brought in as 16-byte pieces of 8 channels.
static bool big_ok(int64_t K, int nS) { return K % 128 == 0 && nS % 8 == 0; }

bool big_gemm_eligible(int64_t M, int64_t N, int64_t K, int nS) {
  return M >= GB_TILE && N >= GB_TILE && big_ok(K, nS);
}

bool big_grouped_eligible(int64_t N, int64_t K, int nS) { return N >= GB_TILE && big_ok(K, nS); }

// B_S gathered per call (no prepared array): one array of N columns.
size_t big_gemm_workspace_bytes(int64_t N, int nS) { return comp_weights_bytes(N, nS); }

template <int FMT, bool GR>
static void launch_big(const BigArgs& a, bool tiled, unsigned grid, hipStream_t stream) {
  if constexpr (GR) {  // grouped operands are row-major
    if (a.row_src)
      hipLaunchKernelGGL((k_gemm_big<FMT, false, 2>), dim3(grid), dim3(GB_T), 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemm_big<FMT, false, 1>), dim3(grid), dim3(GB_T), 0, stream, a);
  } else if (FMT == FP4Q_NVFP4) {
    if (tiled)
      hipLaunchKernelGGL((k_gemm_nv4<true>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemm_nv4<false>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    if (tiled)
      hipLaunchKernelGGL((k_gemm_big<FMT, true, 0>), dim3(grid), dim3(GB_T), 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemm_big<FMT, false, 0>), dim3(grid), dim3(GB_T), 0, stream, a);
  }
}

template <int FMT>
static void launch_gather(bool tiled, const uint8_t* bq, const uint8_t* bs, int64_t N, int64_t K,
                          const int32_t* chan, int nS, int nc, int G, uint8_t* bsel,
                          hipStream_t stream) {
  const int64_t nblocks = ((N + 15) / 16) * nc;
  dim3 grid((unsigned)((nblocks * G + 3) / 4));
  if (tiled)
    hipLaunchKernelGGL((k_gather_bsel<FMT, true>), grid, dim3(256), 0, stream, bq, bs, N, K, chan,
                       nS, nc, nblocks, G, bsel);
  else
    hipLaunchKernelGGL((k_gather_bsel<FMT, false>), grid, dim3(256), 0, stream, bq, bs, N, K,
                       chan, nS, nc, nblocks, G, bsel);
}

int launch_gemm_big(int fmt, bool tiled, int64_t M, int64_t N, int64_t K, const uint8_t* aq,
                    const uint8_t* as, const float* ats, const uint8_t* bq, const uint8_t* bs,
                    const float* bts, const int32_t* chan, int nS, const uint16_t* resid,
                    const float* cts, const uint8_t* bsel_pre, void* y, int y_bf16, int64_t ldy,
                    void* ws, hipStream_t stream) {
  const int nc = nS > 0 ? (nS + GB_CS - 1) / GB_CS : 0;
  // prepared compensation weights (the gather kernel's output, made once)
  // replace the per-call gather
  const bool prepared = bsel_pre != nullptr && nS > 0;
  uint8_t* bsel = prepared ? const_cast<uint8_t*>(bsel_pre) : static_cast<uint8_t*>(ws);
  BigArgs a{M, N, K, aq, as, ats, bq, bs, bts, nS, resid, bsel, chan, cts, y, y_bf16, ldy,
            (int)((M + GB_TILE - 1) / GB_TILE), (int)((N + GB_TILE - 1) / GB_TILE),
            (int)(K / 128), nc, nullptr, 1, nullptr};
  const bool gather = nS > 0 && !prepared;
  const unsigned grid = (unsigned)(a.mt * a.nt);
  if (fmt == FP4Q_NVFP4) {
    if (gather) launch_gather<FP4Q_NVFP4>(tiled, bq, bs, N, K, chan, nS, nc, 1, bsel, stream);
    launch_big<FP4Q_NVFP4, false>(a, tiled, grid, stream);
  } else {
    if (gather) launch_gather<FP4Q_MXFP4>(tiled, bq, bs, N, K, chan, nS, nc, 1, bsel, stream);
    launch_big<FP4Q_MXFP4, false>(a, tiled, grid, stream);
  }
  return 0;
}

// The compensation weights alone, in the layout the GEMMs stream: the G groups'
// blocks one after another (group g's weights at bq + g N K/2).
void launch_comp_weights(int fmt, bool tiled, const uint8_t* bq, const uint8_t* bs, int64_t N,
                         int64_t K, const int32_t* chan, int nS, int G, uint8_t* out,
                         hipStream_t stream) {
  if (N <= 0 || nS <= 0 || G <= 0) return;
  const int nc = (nS + GB_CS - 1) / GB_CS;
  if (fmt == FP4Q_NVFP4) launch_gather<FP4Q_NVFP4>(tiled, bq, bs, N, K, chan, nS, nc, G, out, stream);
  else launch_gather<FP4Q_MXFP4>(tiled, bq, bs, N, K, chan, nS, nc, G, out, stream);
}

size_t comp_weights_bytes(int64_t N, int nS) {
  if (N <= 0 || nS <= 0) return 0;
  return (size_t)(((N + 15) / 16) * ((nS + GB_CS - 1) / GB_CS) * 1024);
}

int launch_gemm_big_grouped(int fmt, int64_t total_rows, int64_t N, int64_t K,
                            const int32_t* off, int G, const uint8_t* aq, const uint8_t* as,
                            const float* ats, const uint8_t* bq, const uint8_t* bs,
                            const float* bts, const int32_t* chan, int nS,
                            const uint16_t* resid, const float* cts, const uint8_t* bsel_pre,
                            void* y, int y_bf16, void* ws, hipStream_t stream, bool wtiled,
                            const int32_t* row_src, int64_t src_rows) {
  const int nc = nS > 0 ? (nS + GB_CS - 1) / GB_CS : 0;
  // prepared compensation weights (every group's, made once) replace the
  // per-call gather
  const bool prepared = bsel_pre != nullptr && nS > 0;
  uint8_t* bsel = prepared ? const_cast<uint8_t*>(bsel_pre) : static_cast<uint8_t*>(ws);
  BigArgs a{total_rows, N, K, aq, as, ats, bq, bs, bts, nS, resid, bsel, chan, cts, y, y_bf16, N,
            0, (int)((N + GB_TILE - 1) / GB_TILE), (int)(K / 128), nc, off, G, row_src};
  const bool gather = nS > 0 && !prepared;
  // the gathering form keeps 32-bit offsets into the token matrix (tiled
  // weights: NVFP4 with 32-bit offsets, checked by the caller)
  const bool ga32 = row_src == nullptr || src_rows * (K / 2) <= (int64_t)UINT32_MAX;
  if (fmt == FP4Q_NVFP4 && ga32) {
    // 128 x 512 tiles; every group adds at most one partial row tile
    a.nt = (int)((N + G4_TN - 1) / G4_TN);
    const unsigned g4 = (unsigned)(((total_rows + G4_TM - 1) / G4_TM + G) * a.nt);
    if (gather) launch_gather<FP4Q_NVFP4>(wtiled, bq, bs, N, K, chan, nS, nc, G, bsel, stream);
    if (row_src && wtiled)
      hipLaunchKernelGGL((k_gemm_nv4g<true, true>), dim3(g4), dim3(256), 0, stream, a);
    else if (row_src)
      hipLaunchKernelGGL((k_gemm_nv4g<true, false>), dim3(g4), dim3(256), 0, stream, a);
    else if (wtiled)
      hipLaunchKernelGGL((k_gemm_nv4g<false, true>), dim3(g4), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemm_nv4g<false, false>), dim3(g4), dim3(256), 0, stream, a);
    return 0;
  }
  // every group adds at most one partial 256-row tile
  const unsigned grid = (unsigned)(((total_rows + GB_TILE - 1) / GB_TILE + G) * a.nt);
  if (fmt == FP4Q_NVFP4) {
    if (gather) launch_gather<FP4Q_NVFP4>(false, bq, bs, N, K, chan, nS, nc, G, bsel, stream);
    launch_big<FP4Q_NVFP4, true>(a, false, grid, stream);
  } else {
    if (gather) launch_gather<FP4Q_MXFP4>(false, bq, bs, N, K, chan, nS, nc, G, bsel, stream);
    launch_big<FP4Q_MXFP4, true>(a, false, grid, stream);
  }
  return 0;
}

}  // namespace fp4q
