// gemm_big.hip -- the prefill-shaped compensated W4A4 GEMM for gfx950.
//
// Same operation as gemm.hip (QUADS abstract: native W4A4 GEMM plus Residual
// Activation Compensation; explainer section 2.2 B; FourSight abstract:
// selected channels effectively BF16):
//   Y[m,n] = sum_k A[m,k] B[n,k] + sum_j R[m,j] B[n,S_j]
// for M, N >= 256.  Design:
//  * 256 x 256 output tile per workgroup; the waves split it WM x 2, each
//    owning (256/WM) x 128 outputs as FI x 8 tiles of 16x16 MFMAs.  The wave
//    count is a template parameter (measured: two waves per SIMD with
//    64 x 128 wave tiles keep the FP4 MFMA pipe busier than one wave per
//    SIMD with 128 x 128).
//  * K advances 128 per stage.  Packed FP4 tiles and block scales go from
//    HBM straight into LDS with global_load_lds (no register staging); three
//    LDS stages rotate.  With fragment double buffering a wave reads the
//    next stage's operand fragments into registers while its MFMAs work on
//    the current stage; otherwise it reads the current stage after the
//    barrier and a second wave on the SIMD covers the wait.  One barrier
//    per stage is the only synchronisation on the main path.
//  * LDS layout per 16-row group and stage: 16-byte slot (chunk c, row r) at
//    c*16 + r, one global_load_lds_dwordx4 per group, and the MFMA operand
//    read of a wave is 64 consecutive slots (no bank conflicts).
//  * MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4; a lane's 32 K-values are one
//    MX block and its E8M0 code comes from LDS.  NVFP4: E4M3 scales on 16
//    elements and 6-bit products do not fit the FP4/FP8 MFMAs exactly, so
//    each lane decodes its codes to f16 (v_cvt_scalef32_pk_f16_fp4, then
//    v_pk_mul_f16 by the block scale, both exact) for
//    v_mfma_f32_16x16x32_f16.
//  * Compensation: the selected channels are sorted, so each stage holds a
//    run of them.  A per-stage table (count, first index, and the LDS
//    offsets of up to 4 channels) is built once per tile.  While a B stage
//    sits in LDS, each thread (one column of the tile) reads the code and
//    scale bytes of the stage's channels before the stage's MFMAs and
//    decodes them to bf16 (e2m1 * block scale, exact) after, into a
//    16-channel staging buffer (double buffered).  Each complete group of 16
//    channels is multiplied at once with v_mfma_f32_16x16x16_bf16 against R
//    (bf16), which global_load_lds brings into LDS well ahead of use.  MXFP4
//    accumulates it directly; NVFP4 scales R by 1/t_x, split into a high and
//    a low bf16 part, so that the final y = (t_x t_w) * acc equals
//    t_w (t_x main + comp) and only MFMAs touch the accumulators.
//  * Workgroup ids are remapped so that the workgroups resident on one XCD
//    (ids congruent mod 8) share a compact block of tiles in L2.
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
constexpr int GB_MAX_NK = 256;           // stages covered by the channel table (K <= 32768)
constexpr int GB_XB = 4;                 // channels per stage handled in the MFMA shadow
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

// Wave layout: W waves as WM x 2; wave tile (256 / WM) x 128 = FI x FJ
// fragments of 16 x 16.
template <int W>
struct WaveLayout {
  static constexpr int T = 64 * W;
  static constexpr int WM = W / 2;
  static constexpr int FI = GB_TILE / WM / 16;
  static constexpr int FJ = 8;
  static constexpr int GPW = 16 / W;  // 16-row data groups per operand a wave loads per stage
};

// Byte offsets inside one LDS stage, and the direct-to-LDS loads a wave
// issues per stage (data, then scales: NVFP4 16 dword instructions per
// stage, MXFP4 8, spread over the waves).
template <int FMT, int W>
struct StageLayout {
  static constexpr int SC = (FMT == FP4Q_NVFP4) ? 2048 : 1024;  // scale bytes per operand
  static constexpr int A = 0;
  static constexpr int B = GB_DATA;
  static constexpr int SA = 2 * GB_DATA;
  static constexpr int SB = 2 * GB_DATA + SC;
  static constexpr int BYTES = 2 * GB_DATA + 2 * SC;
  static constexpr int SCALE_INSTR = (FMT == FP4Q_NVFP4) ? 16 : 8;
  static constexpr int LOADS = 2 * WaveLayout<W>::GPW + SCALE_INSTR / W;
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
// counts.  The lgkmcnt wait is the builtin (simm16 0xC07F: lgkmcnt 0,
// vmcnt and expcnt unconstrained) so that the compiler's wait counting
// knows the LDS reads issued before it are complete and does not wait for
// later ones in their place.  The empty asm statements keep the compiler
// from moving memory operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Issue the direct-to-LDS loads of one K stage (this wave's share).
// Data: 16 instructions per operand, one per 16-row group g: lane l loads
// row 16g + l%16, 16-byte chunk l/16.  Scales: NVFP4 two dwords per row
// stored [d][row]; MXFP4 one dword per row stored [row]; scale instruction
// n covers operand A (first half of n) or B, 64-row chunk n % 4, and for
// NVFP4 dword (n / 4) % 2.  This LDS arrangement is the tiled operand
// layout itself, so with TL each instruction reads one contiguous span (1 KB
// of codes or 256 bytes of scales); row-major operands are gathered from
// rows K/2 bytes apart.
template <int FMT, int W, bool TL>
__device__ __forceinline__ void issue_stage(const BigArgs& p, int kt, int wave, int lane,
                                            int64_t r0, int64_t c0, uint8_t* st) {
  using SL = StageLayout<FMT, W>;
  constexpr int GPW = WaveLayout<W>::GPW;
  constexpr int SPW = SL::SCALE_INSTR / W;
  constexpr int SPS = (FMT == FP4Q_NVFP4) ? 8 : 4;  // scale bytes per row per step
  if (TL) {
    // block indices are wave-uniform (16- or 64-row group, clamped to the
    // last padded group); lane l reads bytes [16 l, 16 l + 16) or [4 l, 4 l + 4)
    const int64_t KB = p.K >> 7;
    const int64_t gM = ((p.M + 15) >> 4) - 1, gN = ((p.N + 15) >> 4) - 1;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int g = wave * GPW + i;
      int64_t ga = (r0 >> 4) + g, gb = (c0 >> 4) + g;
      ga = ga < gM ? ga : gM;
      gb = gb < gN ? gb : gN;
      lds_load16(p.aq + ((ga * KB + kt) << 10) + lane * 16, st + SL::A + g * GB_GRP);
      lds_load16(p.bq + ((gb * KB + kt) << 10) + lane * 16, st + SL::B + g * GB_GRP);
    }
    const int64_t hM = ((p.M + 63) >> 6) - 1, hN = ((p.N + 63) >> 6) - 1;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int n = wave * SPW + i;
      const int c = n & 3;
      const bool isb = n >= SL::SCALE_INSTR / 2;
      int64_t h = ((isb ? c0 : r0) >> 6) + c;
      const int64_t hl = isb ? hN : hM;
      h = h < hl ? h : hl;
      const uint8_t* src = (isb ? p.bs : p.as) + (h * KB + kt) * (SPS * 64) + lane * 4;
      uint8_t* dst = st + (isb ? SL::SB : SL::SA);
      if (FMT == FP4Q_NVFP4) {
        const int d = (n >> 2) & 1;
        lds_load4(src + d * 256, dst + (d * 256 + 64 * c) * 4);
      } else {
        lds_load4(src, dst + 64 * c * 4);
      }
    }
    return;
  }
  const int64_t K2 = p.K >> 1, KS = p.K / (FMT == FP4Q_NVFP4 ? 16 : 32);
  const int64_t off = (int64_t)kt * 64 + (lane >> 4) * 16;
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int g = wave * GPW + i;
    int64_t ra = r0 + 16 * g + (lane & 15), rb = c0 + 16 * g + (lane & 15);
    ra = ra < p.M ? ra : p.M - 1;
    rb = rb < p.N ? rb : p.N - 1;
    lds_load16(p.aq + ra * K2 + off, st + SL::A + g * GB_GRP);
    lds_load16(p.bq + rb * K2 + off, st + SL::B + g * GB_GRP);
  }
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int n = wave * SPW + i;
    const int c = n & 3;
    const bool isb = n >= SL::SCALE_INSTR / 2;
    int64_t row = (isb ? c0 : r0) + 64 * c + lane;
    const int64_t lim = isb ? p.N : p.M;
    row = row < lim ? row : lim - 1;
    const uint8_t* src = isb ? p.bs : p.as;
    uint8_t* dst = st + (isb ? SL::SB : SL::SA);
    if (FMT == FP4Q_NVFP4) {
      const int d = (n >> 2) & 1;
      lds_load4(src + row * KS + (int64_t)kt * SPS + 4 * d, dst + (d * 256 + 64 * c) * 4);
    } else {
      lds_load4(src + row * KS + (int64_t)kt * SPS, dst + 64 * c * 4);
    }
  }
}

// One stage's operands for one wave, in registers.  Lane (lr, q) holds for
// row fragment i (rows wm*16*FI + 16i + lr) and column fragment j (columns
// wn*128 + 16j + lr) the 16 bytes of K chunk q (elements 32q .. 32q+31) and
// the scale word holding the scales of those 32 elements (MXFP4: byte q;
// NVFP4: bytes 2(q%2) and 2(q%2)+1 of dword q/2 -- blocks 2q and 2q+1).  The
// words are kept raw and shifted where they are used, so reading the next
// stage never forces a wait before the current stage's MFMAs.
template <int FI, int FJ>
struct Frag {
  u32x4 a[FI];
  u32x4 b[FJ];
  uint32_t sa[FI];
  uint32_t sb[FJ];
};

template <int FMT, int W, int FI, int FJ>
__device__ __forceinline__ void read_frags(const uint8_t* st, int wm, int wn, int lane,
                                           Frag<FI, FJ>& f) {
  using SL = StageLayout<FMT, W>;
  const int q = lane >> 4, lr = lane & 15;
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    f.a[i] = *reinterpret_cast<const u32x4*>(st + SL::A + (wm * FI + i) * GB_GRP + lane * 16);
    const int row = wm * 16 * FI + i * 16 + lr;
    f.sa[i] = (FMT == FP4Q_MXFP4)
                  ? *reinterpret_cast<const uint32_t*>(st + SL::SA + row * 4)
                  : *reinterpret_cast<const uint32_t*>(st + SL::SA + ((q >> 1) * 256 + row) * 4);
  }
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    f.b[j] = *reinterpret_cast<const u32x4*>(st + SL::B + (wn * FJ + j) * GB_GRP + lane * 16);
    const int col = wn * 16 * FJ + j * 16 + lr;
    f.sb[j] = (FMT == FP4Q_MXFP4)
                  ? *reinterpret_cast<const uint32_t*>(st + SL::SB + col * 4)
                  : *reinterpret_cast<const uint32_t*>(st + SL::SB + ((q >> 1) * 256 + col) * 4);
  }
}

// Multiply one stage held in registers into the FI x FJ accumulator tiles.
template <int FMT, int FI, int FJ>
__device__ __forceinline__ void compute_frags(v4f32 (&acc)[FI][FJ], const Frag<FI, FJ>& f,
                                              int lane) {
  const int q = lane >> 4;
  if (FMT == FP4Q_MXFP4) {
    int sa[FI];
#pragma unroll
    for (int i = 0; i < FI; ++i) sa[i] = (int)(f.sa[i] >> (8 * q));
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const i32x8b bv = {(int)f.b[j].x, (int)f.b[j].y, (int)f.b[j].z, (int)f.b[j].w, 0, 0, 0, 0};
      const int sb = (int)(f.sb[j] >> (8 * q));
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const i32x8b av = {(int)f.a[i].x, (int)f.a[i].y, (int)f.a[i].z, (int)f.a[i].w, 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0,
                                                                     sa[i], 0, sb);
      }
    }
  } else {
    const int sh = 16 * (q & 1);
    // sub-step s: lane q holds elements 32q + 8s .. +7 (block 2q + s/2)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      h16x8 da[FI];
#pragma unroll
      for (int i = 0; i < FI; ++i)
        da[i] = nv_decode8(f.a[i][s], e4m3_h2(f.sa[i] >> (sh + 8 * (s >> 1))));
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const h16x8 db = nv_decode8(f.b[j][s], e4m3_h2(f.sb[j] >> (sh + 8 * (s >> 1))));
#pragma unroll
        for (int i = 0; i < FI; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(da[i], db, acc[i][j], 0, 0, 0);
      }
    }
  }
}

// Per-channel LDS offsets inside a stage for channel position k = S_j % 128:
// bits 0-9 the code byte's offset less the column part, bit 10 the nibble
// (odd k: high nibble), bits 11-21 the scale byte's offset less the column
// part.  Column t adds (t/16)*1024 + (t%16)*16 to the code offset (group,
// slot row) and 4t to the scale offset.
template <int FMT>
__device__ __forceinline__ uint32_t chan_desc(int k) {
  const int bi = k >> 1;
  const uint32_t cpart = (uint32_t)((bi >> 4) * 256 + (bi & 15));
  uint32_t spart;
  if (FMT == FP4Q_NVFP4) {
    const int blkk = k >> 4;  // 0..7: dword blkk/4, byte blkk%4
    spart = (uint32_t)((blkk >> 2) * 1024 + (blkk & 3));
  } else {
    spart = (uint32_t)(k >> 5);
  }
  return cpart | ((uint32_t)(k & 1) << 10) | (spart << 11);
}

// bf16 bits of the B value (e2m1 code * block scale, exact) for a code byte,
// the channel's nibble and the scale byte.
template <int FMT>
__device__ __forceinline__ uint16_t comp_bits(uint32_t cbyte, uint32_t desc, uint32_t sbyte) {
  const uint32_t code = ((desc >> 10) & 1u) ? (cbyte >> 4) : (cbyte & 15u);
  float sc;
  if (FMT == FP4Q_NVFP4)
    sc = e4m3_value(sbyte);
  else
    sc = sbyte ? __uint_as_float(sbyte << 23) : __uint_as_float(0x00400000u);
  const float v = e2m1_mag_value(code) * sc;
  return (uint16_t)((__float_as_uint(v) >> 16) | ((code & 8u) << 12));
}

// Bring R[rows, channels of group g] into an LDS staging buffer laid out
// [row][16 channels]: 8 instructions of 32 rows, two lanes per row.
template <int W>
__device__ __forceinline__ void issue_resid(const BigArgs& p, int64_t r0, int wave, int lane,
                                            int g, uint16_t* rbuf) {
  constexpr int RPW = 8 / W;
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int n = wave * RPW + i;
    int64_t row = r0 + 32 * n + (lane >> 1);
    row = row < p.M ? row : p.M - 1;
    lds_load16(p.resid + row * p.nS + g * GB_CG + 8 * (lane & 1), rbuf + 32 * n * GB_CG);
  }
}

// acc += R_group x Wdeq_group, with R scaled by 1/t_x for NVFP4 (so that the
// final y = (t_x t_w) * acc equals t_w (t_x main + comp)).  The scaled R
// goes into the bf16 MFMA as a high and a low bf16 part (h = bf16(r),
// l = bf16(r - h): relative error about 2^-17 over the whole FP32 range),
// so the accumulators are only ever touched by MFMAs.  A operand: lane takes
// row lr of each 16-row fragment, channels 4q .. 4q+3.
template <int FMT, int FI, int FJ>
__device__ __forceinline__ void flush_group(v4f32 (&acc)[FI][FJ], const uint16_t* comp,
                                            const uint16_t* rbuf, float inv_tx, int wm, int wn,
                                            int lane) {
  const int q = lane >> 4, lr = lane & 15;
  s16x4 ra[FI], rl[FI];
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const u32x2b w =
        *reinterpret_cast<const u32x2b*>(rbuf + (wm * 16 * FI + i * 16 + lr) * GB_CG + 4 * q);
    if (FMT == FP4Q_MXFP4) {
      ra[i] = __builtin_bit_cast(s16x4, w);
    } else {
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t wh = h ? w.y : w.x;
        const float r0 = __uint_as_float(wh << 16) * inv_tx;
        const float r1 = __uint_as_float(wh & 0xFFFF0000u) * inv_tx;
        const uint32_t h0 = f32_to_bf16_rne(r0), h1 = f32_to_bf16_rne(r1);
        const uint32_t l0 = f32_to_bf16_rne(r0 - __uint_as_float(h0 << 16));
        const uint32_t l1 = f32_to_bf16_rne(r1 - __uint_as_float(h1 << 16));
        hi[h] = h0 | (h1 << 16);
        lo[h] = l0 | (l1 << 16);
      }
      ra[i] = __builtin_bit_cast(s16x4, u32x2b{hi[0], hi[1]});
      rl[i] = __builtin_bit_cast(s16x4, u32x2b{lo[0], lo[1]});
    }
  }
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    const s16x4 rb = __builtin_bit_cast(
        s16x4, *reinterpret_cast<const u32x2b*>(comp + (q * 256 + wn * 16 * FJ + j * 16 + lr) * 4));
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ra[i], rb, acc[i][j], 0, 0, 0);
      if (FMT == FP4Q_NVFP4)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(rl[i], rb, acc[i][j], 0, 0, 0);
    }
  }
}

// W waves; DB: the next stage's fragments are read into a second register
// set during the current stage's MFMAs (three stages in flight), else the
// current stage is read after its barrier (two in flight).
template <int FMT, int W, bool DB, bool TL>
__global__ void __launch_bounds__(WaveLayout<W>::T, 1) k_gemm_big(BigArgs args) {
  using SL = StageLayout<FMT, W>;
  using WL = WaveLayout<W>;
  constexpr int FI = WL::FI, FJ = WL::FJ, NT = WL::T;
  __shared__ __attribute__((aligned(16))) uint8_t sStage[3 * SL::BYTES];
  __shared__ __attribute__((aligned(16))) uint16_t sComp[2][GB_COMP];
  __shared__ __attribute__((aligned(16))) uint16_t sR[2][GB_COMP];
  __shared__ int sS[GB_MAX_NS];
  // per stage: count, first channel index, descriptors of up to GB_XB channels
  __shared__ __attribute__((aligned(16))) int sRow[GB_MAX_NK][8];

  const BigArgs& p = args;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

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
  constexpr int L = SL::LOADS;
  float tx = 1.0f, tw = 1.0f, inv_tx = 1.0f;
  if (FMT == FP4Q_NVFP4) {
    tx = *p.ats;
    tw = *p.bts;
    inv_tx = 1.0f / tx;
  }
  auto stage = [&](int kt) __attribute__((always_inline)) { return sStage + (kt % 3) * SL::BYTES; };
  auto uni = [](int v) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(v); };

  // ---- prologue, before any stage is in flight (the fences of these
  // barriers then cost nothing): channel list, zeroed staging buffers, the
  // per-stage channel table
  if (nS > 0) {
    for (int j = t; j < nS; j += NT) sS[j] = p.chan[j];
    for (int i = t; i < 2 * GB_COMP / 8; i += NT)
      reinterpret_cast<u32x4*>(&sComp[0][0])[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    for (int kt = t; kt < nk; kt += NT) {
      // first channel at or past 128 kt, and at or past 128 (kt + 1)
      int lo = 0, hi = nS;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sS[mid] < 128 * kt) lo = mid + 1; else hi = mid;
      }
      int lo2 = lo, hi2 = nS;
      while (lo2 < hi2) {
        const int mid = (lo2 + hi2) >> 1;
        if (sS[mid] < 128 * kt + 128) lo2 = mid + 1; else hi2 = mid;
      }
      uint32_t d[GB_XB];
#pragma unroll
      for (int c = 0; c < GB_XB; ++c) d[c] = (lo + c < lo2) ? chan_desc<FMT>(sS[lo + c] & 127) : 0u;
      *reinterpret_cast<u32x4*>(&sRow[kt][0]) = u32x4{(uint32_t)(lo2 - lo), (uint32_t)lo, d[0], d[1]};
      *reinterpret_cast<u32x4*>(&sRow[kt][4]) = u32x4{d[2], d[3], 0u, 0u};
    }
  }
  asm volatile("" ::: "memory");
  if (nS > 0) issue_resid<W>(p, r0, wave, lane, 0, sR[0]);
  issue_stage<FMT, W, TL>(p, 0, wave, lane, r0, c0, stage(0));
  if (nk > 1) issue_stage<FMT, W, TL>(p, 1, wave, lane, r0, c0, stage(1));
  if (DB && nk > 2) issue_stage<FMT, W, TL>(p, 2, wave, lane, r0, c0, stage(2));

  v4f32 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = v4f32{0.f, 0.f, 0.f, 0.f};

  // Compensation bookkeeping is identical in every lane; readfirstlane keeps
  // it in scalar registers so the branches around the barriers below are
  // uniform branches the compiler can see as such.
  int jx = 0;        // channels extracted so far
  int gf = 0;        // compensation groups flushed so far
  int r_iter = -4;   // step that issued the residual loads of group gf

  // Flush group gf.  Its residual loads are older than the stage awaited at
  // the top of step r_iter + 3, so from then on they have landed; earlier,
  // wait for them explicitly.  Then prefetch the next group's residual into
  // the buffer just freed.
  auto flush = [&](int kt) __attribute__((always_inline)) {
    if (kt < r_iter + 3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    flush_group<FMT, FI, FJ>(acc, sComp[gf & 1], sR[gf & 1], inv_tx, wm, wn, lane);
    gf = uni(gf + 1);
    if (gf * GB_CG < nS) {
      lds_barrier();  // every wave is done with the buffer about to be refilled
      issue_resid<W>(p, r0, wave, lane, gf, sR[gf & 1]);
      r_iter = kt;
    }
  };

  // Channel extraction of stage kx in two halves around the MFMAs: the
  // first reads the table row and the code and scale bytes of up to GB_XB
  // channels (thread t < 256 = column t); the second decodes, writes the
  // staging buffers, extracts any further channels of the stage and
  // flushes groups as they complete.
  struct Pending {
    int cnt, jbase;
    uint32_t desc[GB_XB], cb[GB_XB], sb[GB_XB];
  };
  const int tcol = t & 255;
  const uint32_t toff_c = (uint32_t)(SL::B + (tcol >> 4) * GB_GRP + (tcol & 15) * 16);
  const uint32_t toff_s = (uint32_t)(SL::SB + tcol * 4);
  auto extract_begin = [&](int kx, Pending& pd) __attribute__((always_inline)) {
    const u32x4 r0v = *reinterpret_cast<const u32x4*>(&sRow[kx][0]);
    const u32x4 r1v = *reinterpret_cast<const u32x4*>(&sRow[kx][4]);
    pd.cnt = uni((int)r0v.x);
    pd.jbase = uni((int)r0v.y);
    const uint32_t d[GB_XB] = {r0v.z, r0v.w, r1v.x, r1v.y};
    const uint8_t* st = stage(kx);
#pragma unroll
    for (int c = 0; c < GB_XB; ++c) {
      pd.desc[c] = (uint32_t)uni((int)d[c]);
      pd.cb[c] = st[toff_c + (pd.desc[c] & 1023u)];
      pd.sb[c] = st[toff_s + (pd.desc[c] >> 11)];
    }
  };
  auto extract_end = [&](int kx, const Pending& pd, int kstep) __attribute__((always_inline)) {
    const int jend = pd.jbase + pd.cnt;
    for (int c = 0; jx < jend; ++c, jx = uni(jx + 1)) {
      const int g = jx / GB_CG;
      if (g >= gf + 2) flush(kstep);  // both staging buffers hold unflushed groups
      uint32_t desc, cb, sb;
      if (c < GB_XB) {
        desc = c == 0 ? pd.desc[0] : c == 1 ? pd.desc[1] : c == 2 ? pd.desc[2] : pd.desc[3];
        cb = c == 0 ? pd.cb[0] : c == 1 ? pd.cb[1] : c == 2 ? pd.cb[2] : pd.cb[3];
        sb = c == 0 ? pd.sb[0] : c == 1 ? pd.sb[1] : c == 2 ? pd.sb[2] : pd.sb[3];
      } else {  // more channels in this stage than the table row holds
        desc = (uint32_t)uni((int)chan_desc<FMT>(uni(sS[jx]) & 127));
        cb = stage(kx)[toff_c + (desc & 1023u)];
        sb = stage(kx)[toff_s + (desc >> 11)];
      }
      if (t < 256) {
        const int jj = jx % GB_CG;
        sComp[g & 1][((jj >> 2) * 256 + tcol) * 4 + (jj & 3)] = comp_bits<FMT>(cb, desc, sb);
      }
    }
    if (gf * GB_CG + GB_CG <= jx) flush(kstep);  // the oldest group is complete
  };

  if (DB) {
    // three stages in flight, fragments double-buffered in registers
    Frag<FI, FJ> f0, f1;
    Pending pd;
    if (nk > 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * L) : "memory");
    else if (nk > 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    read_frags<FMT, W>(stage(0), wm, wn, lane, f0);
    if (nS > 0) {
      extract_begin(0, pd);
      extract_end(0, pd, -1);
    }
    // stage kt's fragments are in `cur`; stage kt+1 is read into `nxt` and
    // its channels extracted; stage kt+3 goes into the LDS stage kt used
    auto step = [&](int kt, Frag<FI, FJ>& cur, Frag<FI, FJ>& nxt) __attribute__((always_inline)) {
      if (kt + 1 < nk) {
        if (kt + 2 < nk)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();  // stage kt+1 landed everywhere; stage kt's LDS is free
      if (kt + 3 < nk) issue_stage<FMT, W, TL>(p, kt + 3, wave, lane, r0, c0, stage(kt));
      if (kt + 1 < nk) read_frags<FMT, W>(stage(kt + 1), wm, wn, lane, nxt);
      const bool ex = nS > 0 && kt + 1 < nk;
      if (ex) extract_begin(kt + 1, pd);
      compute_frags<FMT, FI, FJ>(acc, cur, lane);
      if (ex) extract_end(kt + 1, pd, kt);
    };
    for (int kt = 0; kt < nk; kt += 2) {
      step(kt, f0, f1);
      if (kt + 1 >= nk) break;
      step(kt + 1, f1, f0);
    }
  } else {
    // two stages in flight; the current stage is read after its barrier
    Pending pd;
    auto step = [&](int kt) __attribute__((always_inline)) {
      if (kt + 1 < nk)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();  // stage kt landed everywhere; stage kt-1's LDS is free
      if (kt + 2 < nk) issue_stage<FMT, W, TL>(p, kt + 2, wave, lane, r0, c0, stage(kt + 2));
      Frag<FI, FJ> f;
      read_frags<FMT, W>(stage(kt), wm, wn, lane, f);
      if (nS > 0) extract_begin(kt, pd);
      compute_frags<FMT, FI, FJ>(acc, f, lane);
      if (nS > 0) extract_end(kt, pd, kt);
    };
    for (int kt = 0; kt < nk; ++kt) step(kt);
  }

  // remaining compensation groups (every channel is < K, so all extracted)
  while (gf * GB_CG < nS) flush(nk);

  // ---- epilogue: y = (t_x t_w) * acc; lane holds column lr, rows 4q..4q+3
  // of each 16x16 tile
  const float ys = (FMT == FP4Q_NVFP4) ? tx * tw : 1.0f;
  const int q = lane >> 4, lr = lane & 15;
  const bool interior = (r0 + GB_TILE <= p.M) && (c0 + GB_TILE <= p.N);
  const int64_t rw = r0 + wm * 16 * FI + 4 * q, cw = c0 + wn * 16 * FJ + lr;
  if (!p.y_bf16) {
    float* y = reinterpret_cast<float*>(p.y);
    if (interior) {
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_nontemporal_store(acc[i][j][e] * ys,
                                        y + (rw + i * 16 + e) * p.ldy + cw + j * 16);
    } else {
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
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
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t row = rw + i * 16 + e, col = cw + j * 16;
          if (interior || (row < p.M && col < p.N))
            y[row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][e] * ys);
        }
  }
}

bool big_gemm_eligible(int64_t M, int64_t N, int64_t K, int nS, const void* resid) {
  // residual rows are brought in as 16-byte pieces of 8 channels
  const bool resid_ok = nS == 0 || (reinterpret_cast<uintptr_t>(resid) & 15) == 0;
  return M >= 256 && N >= 256 && K % 128 == 0 && K / 128 <= GB_MAX_NK && nS <= GB_MAX_NS &&
         nS % GB_CG == 0 && resid_ok;
}

// Configuration per format: wave count and fragment double buffering.
template <int FMT> struct BigConfig;
template <> struct BigConfig<FP4Q_MXFP4> { static constexpr int W = 8; static constexpr bool DB = false; };
template <> struct BigConfig<FP4Q_NVFP4> { static constexpr int W = 8; static constexpr bool DB = false; };

template <int FMT>
static void launch_big(const BigArgs& a, bool tiled, hipStream_t stream) {
  using C = BigConfig<FMT>;
  dim3 grid((unsigned)(a.mt * a.nt));
  if (tiled)
    hipLaunchKernelGGL((k_gemm_big<FMT, C::W, C::DB, true>), grid, dim3(64 * C::W), 0, stream, a);
  else
    hipLaunchKernelGGL((k_gemm_big<FMT, C::W, C::DB, false>), grid, dim3(64 * C::W), 0, stream, a);
}

int launch_gemm_big(int fmt, bool tiled, int64_t M, int64_t N, int64_t K, const uint8_t* aq,
                    const uint8_t* as, const float* ats, const uint8_t* bq, const uint8_t* bs,
                    const float* bts, const int32_t* chan, int nS, const uint16_t* resid,
                    void* y, int y_bf16, int64_t ldy, hipStream_t stream) {
  BigArgs a{M, N, K, aq, as, ats, bq, bs, bts, chan, nS, resid, y, y_bf16, ldy,
            (int)((M + GB_TILE - 1) / GB_TILE), (int)((N + GB_TILE - 1) / GB_TILE)};
  if (fmt == FP4Q_NVFP4) launch_big<FP4Q_NVFP4>(a, tiled, stream);
  else launch_big<FP4Q_MXFP4>(a, tiled, stream);
  return 0;
}

}  // namespace fp4q
