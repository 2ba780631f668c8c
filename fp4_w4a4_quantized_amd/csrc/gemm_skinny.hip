// gemm_skinny.hip -- the decode-shaped (few activation rows) compensated
// W4A4 GEMM for gfx950.
//
// Same operation as gemm.hip (QUADS abstract: native W4A4 GEMM plus Residual
// Activation Compensation; explainer section 2.2 B; FourSight abstract:
// selected channels effectively BF16, with a separate decode datapath):
//   Y[m,n] = sum_k A[m,k] B[n,k] + sum_j R[m,j] B[n,S_j],   M <= 64.
// With at most 64 activation rows the cost is streaming the weights, so:
//  * a workgroup of 8 waves owns 48 output columns (3 groups of 16) and all
//    64 rows; the grid is about one workgroup per CU;
//  * the waves split K: wave w takes the 128-wide K steps w, w + 8, w + 16,
//    ... with two steps in flight.  Each lane loads its weight bytes and its
//    activation fragments (which stay in L2: every workgroup reads them)
//    straight into registers; the scale bytes of a step come with one
//    coalesced load per operand and are redistributed through a
//    wave-private LDS slot -- the main path has no barrier and waits only
//    for its own data (load issue, not bandwidth, bounds this shape, so the
//    load instruction count is kept low);
//  * NVFP4 decodes both operands in registers (v_cvt_scalef32_pk_f16_fp4,
//    then one v_pk_mul_f16 by the E4M3 block scale: exact in f16) for
//    v_mfma_f32_16x16x32_f16; MXFP4 feeds the packed codes and E8M0 scales
//    to v_mfma_scale_f32_16x16x128_f8f6f4 directly;
//  * the compensation weights B[n, S_j] come from the wave whose K step holds
//    channel S_j: it copies the step's weight bytes to a wave-private LDS
//    slot; then the 64 lanes decode four channels x 16 columns at a time
//    (to bf16, exact), with no branches; R[:, S] is staged in LDS at the
//    start (16-byte loads).
//    After the eight K-partial sums meet in LDS, waves 0-3 (16 rows each)
//    add R B_S with v_mfma_f32_16x16x16_bf16 and store
//    y = tw * (tx * main + comp).
// Rows past M use clamped (real) rows: a row of A only reaches the same row
// of the product, and those rows are not stored.  Columns past N likewise.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

typedef float v4f32s __attribute__((ext_vector_type(4)));
typedef float v2f32s __attribute__((ext_vector_type(2)));
typedef int i32x8s __attribute__((ext_vector_type(8)));
typedef _Float16 h8s __attribute__((ext_vector_type(8)));
typedef _Float16 h2s __attribute__((ext_vector_type(2)));
typedef short s4s __attribute__((ext_vector_type(4)));

constexpr int SK_COLS = 48;            // output columns per workgroup
constexpr int SK_CG = 3;               // 16-column groups
constexpr int SK_M = 64;               // activation rows handled
constexpr int SK_WAVES = 8;
constexpr int SK_T = 64 * SK_WAVES;
constexpr int SK_MAXS = 64;            // compensation channels
constexpr int SK_SRS = SK_MAXS + 4;    // LDS row stride (bf16) of R and B_S

struct SkinnyArgs {
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
  const float* cts;  // tensor scale of the compensation term, or null (1)
  const uint8_t* bsel;  // prepared compensation weights (tiled BF16), or null
  void* y;
  int y_bf16;
  int64_t ldy;
};

__device__ __forceinline__ h8s sk_decode8(uint32_t w, h2s s) {
  h2s p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  h2s p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  h2s p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  h2s p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  h8s r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// The two E4M3 scale bytes in the low half of `codes`, as f16 (exact: every
// E4M3 value, subnormals included, is an f16 value).
__device__ __forceinline__ h2s sk_scales2(uint32_t codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, false);
}

// Registers of one K step for one wave.  Lane (lr = lane % 16, q = lane / 16)
// holds:
//   x[a]  16 bytes of activation row 16a + lr, elements 32q .. 32q+31 of the
//         step; w[g] the same bytes of weight row col0 + 16g + lr
//   xsc   the step's scale bytes of activation row `lane` (8 NVFP4 blocks or
//         4 MXFP4 blocks), wsc those of weight row col0 + lane (lane < 48);
//         loaded with one coalesced load per operand and redistributed
//         through a wave-private LDS slot
struct Step {
  u32x4 x[4];
  u32x4 w[SK_CG];
  u32x2 xsc, wsc;
};

// Row-major operands: each lane computes its row addresses.  Tiled operands
// (TL): a fragment load of 16 rows x 64 bytes is one 1 KB block, lane l at
// byte 16 l, so only the block index (wave-uniform: the 16-row group,
// clamped to the last padded group) varies; `wso` is the lane's weight-row
// scale offset within a step (computed once per workgroup).
template <int FMT, bool TL>
__device__ __forceinline__ void load_step(const SkinnyArgs& p, int kt, int lane, int64_t col0,
                                          int64_t wso, Step& s) {
  constexpr int SPS = (FMT == FP4Q_NVFP4) ? 8 : 4;  // scale bytes per row per step
  const int64_t K = p.K;
  if (TL) {
    const int64_t KB = K >> 7;
    const int64_t gN = ((p.N + 15) >> 4) - 1, gM = ((p.M + 15) >> 4) - 1;
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) {
      int64_t grp = (col0 >> 4) + g;
      grp = grp < gN ? grp : gN;
      s.w[g] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(p.bq + ((grp * KB + kt) << 10) + lane * 16));
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t grp = a < gM ? a : gM;
      s.x[a] = *reinterpret_cast<const u32x4*>(p.aq + ((grp * KB + kt) << 10) + lane * 16);
    }
    // activation rows 0..63 are the first 64-row scale group
    const int64_t st = (int64_t)kt * (SPS * 64);
    const uint8_t* ws = p.bs + wso + st;
    const uint8_t* xs = p.as + st + lane * 4;
    if (FMT == FP4Q_NVFP4) {
      // the two scale dwords of a step sit in planes 256 bytes apart
      s.wsc = u32x2{*reinterpret_cast<const uint32_t*>(ws),
                    *reinterpret_cast<const uint32_t*>(ws + 256)};
      s.xsc = u32x2{*reinterpret_cast<const uint32_t*>(xs),
                    *reinterpret_cast<const uint32_t*>(xs + 256)};
    } else {
      s.wsc = u32x2{*reinterpret_cast<const uint32_t*>(ws), 0u};
      s.xsc = u32x2{*reinterpret_cast<const uint32_t*>(xs), 0u};
    }
    return;
  }
  const int64_t K2 = K >> 1, KS = K / (FMT == FP4Q_NVFP4 ? 16 : 32);
  const int q = lane >> 4, lr = lane & 15;
#pragma unroll
  for (int g = 0; g < SK_CG; ++g) {
    int64_t row = col0 + 16 * g + lr;
    row = row < p.N ? row : p.N - 1;
    s.w[g] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(p.bq + row * K2 + (int64_t)kt * 64 + q * 16));
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    int64_t row = 16 * a + lr;
    row = row < p.M ? row : p.M - 1;
    s.x[a] = *reinterpret_cast<const u32x4*>(p.aq + row * K2 + (int64_t)kt * 64 + q * 16);
  }
  int64_t wrow = col0 + (lane < SK_COLS ? lane : SK_COLS - 1);
  wrow = wrow < p.N ? wrow : p.N - 1;
  const int64_t xrow = lane < p.M ? lane : p.M - 1;
  if (FMT == FP4Q_NVFP4) {
    s.wsc = *reinterpret_cast<const u32x2*>(p.bs + wrow * KS + (int64_t)kt * 8);
    s.xsc = *reinterpret_cast<const u32x2*>(p.as + xrow * KS + (int64_t)kt * 8);
  } else {
    s.wsc = u32x2{*reinterpret_cast<const uint32_t*>(p.bs + wrow * KS + (int64_t)kt * 4), 0u};
    s.xsc = u32x2{*reinterpret_cast<const uint32_t*>(p.as + xrow * KS + (int64_t)kt * 4), 0u};
  }
}

// Bytes of one wave-private scale slot: weight rows then activation rows.
template <int FMT> struct SlotLayout {
  static constexpr int PER_ROW = (FMT == FP4Q_NVFP4) ? 8 : 4;  // scale bytes per row per step
  static constexpr int X_OFF = SK_COLS * PER_ROW;
  static constexpr int BYTES = X_OFF + SK_M * PER_ROW;
};

// Multiply one K step into the accumulators; take the compensation weights
// of the channels that fall in it.
template <int FMT, bool PB>
__device__ __forceinline__ void process_step(const Step& st, int kt, uint8_t* slot,
                                             uint8_t* cslot, int lane, int my_ch, int nS,
                                             uint16_t* sB, v4f32s (&acc)[4][SK_CG]) {
  using L = SlotLayout<FMT>;
  const int q = lane >> 4, lr = lane & 15;
  // redistribute the scale bytes: lane (lr, q) needs those of its rows for
  // elements 32q .. 32q+31 (NVFP4: blocks 2q, 2q+1; MXFP4: block q)
  if (FMT == FP4Q_NVFP4) {
    if (lane < SK_COLS) *reinterpret_cast<u32x2*>(slot + lane * 8) = st.wsc;
    *reinterpret_cast<u32x2*>(slot + L::X_OFF + lane * 8) = st.xsc;
  } else {
    if (lane < SK_COLS) *reinterpret_cast<uint32_t*>(slot + lane * 4) = st.wsc.x;
    *reinterpret_cast<uint32_t*>(slot + L::X_OFF + lane * 4) = st.xsc.x;
  }
  uint32_t ws[SK_CG], xs[4];
#pragma unroll
  for (int g = 0; g < SK_CG; ++g)
    ws[g] = (FMT == FP4Q_NVFP4)
                ? (uint32_t)*reinterpret_cast<const uint16_t*>(slot + (16 * g + lr) * 8 + 2 * q)
                : (uint32_t)slot[(16 * g + lr) * 4 + q];
#pragma unroll
  for (int a = 0; a < 4; ++a)
    xs[a] = (FMT == FP4Q_NVFP4)
                ? (uint32_t)*reinterpret_cast<const uint16_t*>(slot + L::X_OFF + (16 * a + lr) * 8 + 2 * q)
                : (uint32_t)slot[L::X_OFF + (16 * a + lr) * 4 + q];

  if (FMT == FP4Q_NVFP4) {
    // lane (lr, q): scales of blocks 2q (elements 32q .. +15) and 2q + 1
    h2s wsp[SK_CG], xsp[4];
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) wsp[g] = sk_scales2(ws[g]);
#pragma unroll
    for (int a = 0; a < 4; ++a) xsp[a] = sk_scales2(xs[a]);
    // sub-step s: lane (lr, q) holds elements 32q + 8s .. +7 of the step
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      h8s db[SK_CG];
#pragma unroll
      for (int g = 0; g < SK_CG; ++g) db[g] = sk_decode8(st.w[g][s], (s >> 1) ? wsp[g].yy : wsp[g].xx);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const h8s da = sk_decode8(st.x[a][s], (s >> 1) ? xsp[a].yy : xsp[a].xx);
#pragma unroll
        for (int g = 0; g < SK_CG; ++g)
          acc[a][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(da, db[g], acc[a][g], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const u32x4 xa = st.x[a];
      const i32x8s av = {(int)xa.x, (int)xa.y, (int)xa.z, (int)xa.w, 0, 0, 0, 0};
#pragma unroll
      for (int g = 0; g < SK_CG; ++g) {
        const u32x4 wb = st.w[g];
        const i32x8s bv = {(int)wb.x, (int)wb.y, (int)wb.z, (int)wb.w, 0, 0, 0, 0};
        acc[a][g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[a][g], 4, 4, 0,
                                                                     (int)xs[a], 0, (int)ws[g]);
      }
    }
  }
  // compensation weights of the channels in this step (unless prepared
  // ones were staged at the start): S is ascending, so
  // they are the entries [j0, j1) of the lanes of my_ch.  The step's weight
  // bytes go to the wave-private slot as rows of 64 bytes; lane (r, u) then
  // takes channel jb + u and the columns 16g + r.  One wave's LDS operations
  // complete in order, so the slot needs no barrier.  Lanes past j1 write
  // the unused padding column SK_MAXS of sB.
  if (!PB && nS > 0) {
    const uint64_t m = __ballot(my_ch >= 0 && (my_ch >> 7) == kt);
    if (m) {
      const int j0 = __builtin_ctzll(m), j1 = 64 - __builtin_clzll(m);
#pragma unroll
      for (int g = 0; g < SK_CG; ++g)
        *reinterpret_cast<u32x4*>(cslot + (16 * g + lr) * 64 + 16 * q) = st.w[g];
      for (int jb = j0; jb < j1; jb += 4) {
        const int j = jb + q;
        const bool ok = j < j1;
        const int pos = __builtin_amdgcn_ds_bpermute((ok ? j : j0) << 2, my_ch) & 127;
        const int jw = ok ? j : SK_MAXS;
#pragma unroll
        for (int g = 0; g < SK_CG; ++g) {
          const int n = 16 * g + lr;
          const uint32_t byte = cslot[n * 64 + (pos >> 1)];
          const uint32_t c8 = (FMT == FP4Q_NVFP4) ? slot[n * 8 + (pos >> 4)] : slot[n * 4 + (pos >> 5)];
          const v2f32s pr = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0);
          const float e = (pos & 1) ? pr[1] : pr[0];  // signed E2M1 value
          float sv;
          if (FMT == FP4Q_NVFP4)
            sv = e4m3_value(c8);
          else
            sv = c8 ? __uint_as_float(c8 << 23) : __uint_as_float(0x00400000u);
          // exact, and exact in bf16 (at most 6 significant bits)
          sB[n * SK_SRS + jw] = (uint16_t)(__float_as_uint(e * sv) >> 16);
        }
      }
    }
  }
}

template <int FMT, bool TL, bool PB>
__global__ void __launch_bounds__(SK_T, 1) k_gemm_skinny(SkinnyArgs p) {
  using L = SlotLayout<FMT>;
  __shared__ __attribute__((aligned(16))) v4f32s red[SK_WAVES * 4 * SK_CG * 64];   // 96 KB
  __shared__ __attribute__((aligned(16))) uint8_t sScale[SK_WAVES * 2 * L::BYTES];  // 2 slots per wave
  __shared__ __attribute__((aligned(16))) uint16_t sR[SK_M * SK_SRS];              // R[m][j]
  __shared__ __attribute__((aligned(16))) uint16_t sB[SK_COLS * SK_SRS];           // B_S[n][j]
  __shared__ __attribute__((aligned(16))) uint8_t sCode[SK_WAVES * SK_COLS * 64];    // 24 KB

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int q = lane >> 4, lr = lane & 15;
  const int64_t col0 = (int64_t)blockIdx.x * SK_COLS;
  const int nk = (int)(p.K / 128);
  const int nS = p.nS;

  // ---- prologue.  No barrier: everything here is per wave (the residual
  // rows are staged in LDS while the operand stream is in flight, and are
  // read after the reduction barrier).  Every load is unconditional (clamped
  // indices, or a valid stand-in address when there are no channels) so the
  // compiler can count the loads in flight and wait only for the data used.
  float tx = 1.0f, tw = 1.0f;
  if (FMT == FP4Q_NVFP4) {
    tx = *p.ats;
    tw = *p.bts;
  }
  // lane j holds channel S_j (valid for j < nS); this and the residual
  // load are issued first, so waiting for them never waits for the operand
  // stream.  R [M][nS] bf16, contiguous, 16-byte aligned, M nS a multiple of
  // 8: thread t takes elements 8t .. 8t+7 (of at most 4096).
  const int my_ch_raw = *(nS > 0 ? p.chan + (lane < nS ? lane : nS - 1)
                                 : reinterpret_cast<const int32_t*>(p.aq));
  const int rtot = (int)p.M * nS, e0 = 8 * t;
  const u32x4 rv = *reinterpret_cast<const u32x4*>(
      nS > 0 ? p.resid + (e0 < rtot ? e0 : rtot - 8) : reinterpret_cast<const uint16_t*>(p.aq));
  // prepared compensation weights: 1 KB blocks (16-column group, stage of
  // 32 channels), in each the 16-byte piece (channels 8u .. 8u+7 of the
  // stage, column r) at (16u + r) * 16; thread t < 3 * 64 nc takes piece
  // t % 64 of block t / 64 of this workgroup's column groups (clamped to the
  // last group; those columns are not stored)
  const int nc = (nS + 31) >> 5;
  const bool pb_on = PB && t < SK_CG * 64 * nc;
  int pb_g = 0, pb_c = 0;
  u32x4 pbv = u32x4{0u, 0u, 0u, 0u};
  if (PB) {
    const int blk = pb_on ? t >> 6 : 0;
    pb_g = blk / (nc > 0 ? nc : 1);
    pb_c = blk - pb_g * nc;
    const int64_t glast = ((p.N + 15) >> 4) - 1;
    int64_t gi = (col0 >> 4) + pb_g;
    gi = gi < glast ? gi : glast;
    if (pb_on)
      pbv = *reinterpret_cast<const u32x4*>(p.bsel + ((gi * nc + pb_c) << 10) + (t & 63) * 16);
  }
  // tiled layout: this lane's weight-row scale offset within a step (rows
  // exist up to the 64-row padding)
  int64_t wso = 0;
  if (TL) {
    constexpr int SPS = (FMT == FP4Q_NVFP4) ? 8 : 4;
    int64_t wrow = col0 + (lane < SK_COLS ? lane : SK_COLS - 1);
    const int64_t wlast = ((p.N + 63) & ~(int64_t)63) - 1;
    wrow = wrow < wlast ? wrow : wlast;
    wso = (wrow >> 6) * (p.K >> 7) * (SPS * 64) + (wrow & 63) * 4;
  }
  Step s0, s1;
  load_step<FMT, TL>(p, wave < nk ? wave : nk - 1, lane, col0, wso, s0);
  load_step<FMT, TL>(p, wave + SK_WAVES < nk ? wave + SK_WAVES : nk - 1, lane, col0, wso, s1);
  if (PB && pb_on) {
    const int u = (t & 63) >> 4, r = t & 15;
    uint16_t* dst = sB + (16 * pb_g + r) * SK_SRS + 32 * pb_c + 8 * u;  // 8-byte aligned
    reinterpret_cast<u32x2*>(dst)[0] = u32x2{pbv.x, pbv.y};
    reinterpret_cast<u32x2*>(dst)[1] = u32x2{pbv.z, pbv.w};
  }
  if (nS > 0 && e0 < rtot) {
    const uint32_t w4[4] = {rv.x, rv.y, rv.z, rv.w};
    int row = e0 / nS, j = e0 - row * nS;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sR[row * SK_SRS + j] = (uint16_t)(w4[k >> 1] >> (16 * (k & 1)));
      if (++j == nS) { j = 0; ++row; }
    }
  }

  v4f32s acc[4][SK_CG];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) acc[a][g] = v4f32s{0.f, 0.f, 0.f, 0.f};

  // ---- K steps wave, wave + 8, wave + 16, ...: two steps in flight
  uint8_t* slot0 = sScale + (wave * 2 + 0) * L::BYTES;
  uint8_t* slot1 = sScale + (wave * 2 + 1) * L::BYTES;
  uint8_t* cslot = sCode + wave * (SK_COLS * 64);
  const int my_ch = (nS > 0 && lane < nS) ? my_ch_raw : -1;
  if (nk <= 2 * SK_WAVES) {
    // K <= 2048: both steps are already in flight
    if (wave < nk) process_step<FMT, PB>(s0, wave, slot0, cslot, lane, my_ch, nS, sB, acc);
    if (wave + SK_WAVES < nk) process_step<FMT, PB>(s1, wave + SK_WAVES, slot1, cslot, lane, my_ch, nS, sB, acc);
  } else {
    for (int kt = wave; kt < nk; kt += 2 * SK_WAVES) {
      process_step<FMT, PB>(s0, kt, slot0, cslot, lane, my_ch, nS, sB, acc);
      if (kt + 2 * SK_WAVES < nk) load_step<FMT, TL>(p, kt + 2 * SK_WAVES, lane, col0, wso, s0);
      if (kt + SK_WAVES < nk) {
        process_step<FMT, PB>(s1, kt + SK_WAVES, slot1, cslot, lane, my_ch, nS, sB, acc);
        if (kt + 3 * SK_WAVES < nk) load_step<FMT, TL>(p, kt + 3 * SK_WAVES, lane, col0, wso, s1);
      }
    }
  }


  // ---- K-partial sums meet in LDS; wave a (< 4) then owns rows 16a .. 16a+15
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) red[((wave * 4 + a) * SK_CG + g) * 64 + lane] = acc[a][g];
  __syncthreads();
  if (wave >= 4) return;
  v4f32s out[SK_CG];
#pragma unroll
  for (int g = 0; g < SK_CG; ++g) {
    out[g] = red[((0 * 4 + wave) * SK_CG + g) * 64 + lane];
#pragma unroll
    for (int w2 = 1; w2 < SK_WAVES; ++w2) out[g] += red[((w2 * 4 + wave) * SK_CG + g) * 64 + lane];
  }

  // ---- compensation: y = tw * (tx * main + comp).  All SK_MAXS / 16
  // chunks run, with entries j >= nS of both operands masked to zero (the
  // LDS there is not written), so every LDS read is issued up front.
  if (nS > 0) {
    v4f32s comp[SK_CG];
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) comp[g] = v4f32s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < SK_MAXS / 16; ++c) {
      const int jq = 16 * c + 4 * q;
      const u32x2 m2 = u32x2{(jq + 0 < nS ? 0xFFFFu : 0u) | (jq + 1 < nS ? 0xFFFF0000u : 0u),
                             (jq + 2 < nS ? 0xFFFFu : 0u) | (jq + 3 < nS ? 0xFFFF0000u : 0u)};
      // A: R[16 wave + lr][jq .. jq+3]; B: B_S[16 g + lr][jq .. jq+3]
      const s4s ra = __builtin_bit_cast(
          s4s, *reinterpret_cast<const u32x2*>(sR + (16 * wave + lr) * SK_SRS + jq) & m2);
#pragma unroll
      for (int g = 0; g < SK_CG; ++g) {
        const s4s rb = __builtin_bit_cast(
            s4s, *reinterpret_cast<const u32x2*>(sB + (16 * g + lr) * SK_SRS + jq) & m2);
        comp[g] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ra, rb, comp[g], 0, 0, 0);
      }
    }
    const float cs = p.cts ? *p.cts : 1.0f;
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) out[g] = out[g] * tx + comp[g] * cs;
  } else if (FMT == FP4Q_NVFP4) {
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) out[g] *= tx;
  }

  // ---- store: lane holds rows 16 wave + 4q + e, column col0 + 16g + lr
#pragma unroll
  for (int g = 0; g < SK_CG; ++g) {
    const int64_t col = col0 + 16 * g + lr;
    if (col >= p.N) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = 16 * wave + 4 * q + e;
      if (row >= p.M) continue;
      const float v = out[g][e] * tw;
      if (p.y_bf16)
        reinterpret_cast<uint16_t*>(p.y)[row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
      else
        reinterpret_cast<float*>(p.y)[row * p.ldy + col] = v;
    }
  }
}

// ---- the fused decode datapath --------------------------------------------------
//
// FourSight abstract: a fused kernel with its own decode datapath.  For
// decode shapes the activation quantization is a separate launch of about
// the GEMM's own length, so here it moves into the GEMM: the activations
// arrive as BF16 and each workgroup quantizes them itself.  With K <= 2048
// (16 steps of 128) each of the 8 waves owns at most the two K steps it
// multiplies, wave and wave + 8; it loads their BF16 values (64 rows x 256
// columns, 32 KB per wave) straight into registers while the weight loads
// are in flight.  The 8 waves together hold the whole tensor, so the
// tensor amax is one LDS reduction -- no grid barrier, no second read.
// Each lane then holds whole 16-element blocks (rows 16a + lr, elements
// 32q .. 32q + 31 of a step: blocks 2q and 2q + 1), so it forms block
// scales, quotients and codes with the quantizer's own operations and
// leaves the codes in exactly the fragment registers the MFMAs take; the
// residual of the selected channels goes to LDS for the compensation term.
// Workgroup 0 can also write the quantized activations out (codes, scales,
// tensor scale, residual; row-major), for checking.  NVFP4, prepared
// compensation weights (or none).
struct FusedArgs {
  int64_t M, N, K;
  const uint16_t* x;
  int64_t ldx;
  const uint8_t* bq;
  const uint8_t* bs;
  const float* bts;
  const int32_t* chan;
  int nS;
  const uint8_t* bsel;
  void* y;
  int y_bf16;
  int64_t ldy;
  uint8_t* q_out;     // optional: [M, K/2] row-major
  uint8_t* s_out;     // optional: [M, K/16]
  float* ts_out;      // optional: [1]
  uint16_t* r_out;    // optional: [M, nS]
};

// The weights of one K step (load_step without the activations).
template <bool TL>
__device__ __forceinline__ void load_w_step(const FusedArgs& p, int kt, int lane, int64_t col0,
                                            int64_t wso, Step& s) {
  const int64_t K = p.K;
  if (TL) {
    const int64_t KB = K >> 7;
    const int64_t gN = ((p.N + 15) >> 4) - 1;
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) {
      int64_t grp = (col0 >> 4) + g;
      grp = grp < gN ? grp : gN;
      s.w[g] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(p.bq + ((grp * KB + kt) << 10) + lane * 16));
    }
    const uint8_t* ws = p.bs + wso + (int64_t)kt * (8 * 64);
    s.wsc = u32x2{*reinterpret_cast<const uint32_t*>(ws),
                  *reinterpret_cast<const uint32_t*>(ws + 256)};
    return;
  }
  const int64_t K2 = K >> 1, KS = K / 16;
  const int q = lane >> 4, lr = lane & 15;
#pragma unroll
  for (int g = 0; g < SK_CG; ++g) {
    int64_t row = col0 + 16 * g + lr;
    row = row < p.N ? row : p.N - 1;
    s.w[g] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(p.bq + row * K2 + (int64_t)kt * 64 + q * 16));
  }
  int64_t wrow = col0 + (lane < SK_COLS ? lane : SK_COLS - 1);
  wrow = wrow < p.N ? wrow : p.N - 1;
  s.wsc = *reinterpret_cast<const u32x2*>(p.bs + wrow * KS + (int64_t)kt * 8);
}

// One lane's activations of one K step: rows 16a + lr (a = 0..3, clamped to
// M - 1), elements 32q .. 32q + 31 of the step, as BF16 pairs.
struct XSlab {
  u32x4 v[4][4];  // [a][16-byte piece]
};

__device__ __forceinline__ void load_x_step(const FusedArgs& p, int kt, int lane, XSlab& x) {
  const int q = lane >> 4, lr = lane & 15;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    int64_t row = 16 * a + lr;
    row = row < p.M ? row : p.M - 1;
    // plain (cached) loads: every workgroup reads the same activations, and
    // the four loads of a lane revisit the same cache lines
    const u32x4* src = reinterpret_cast<const u32x4*>(p.x + row * p.ldx + (int64_t)kt * 128 + 32 * q);
#pragma unroll
    for (int c = 0; c < 4; ++c) x.v[a][c] = src[c];
  }
}

__device__ __forceinline__ uint32_t slab_absmax(const XSlab& x) {
  uint32_t m = 0;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 v = x.v[a][c];
      m = max(m, max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu)));
      m = max(m, max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu)));
    }
  return m;
}

// NVFP4 codes of one 16-element block held by one lane (two 16-byte pieces),
// with the quantizer's operations: block amax, (amax / 6) / t to E4M3
// (nearest even, saturating), d = sb t, the correctly rounded quotient x / d
// (reciprocal and two FMA corrections) and the hardware E2M1 conversion.
__device__ __forceinline__ void nv_block16(u32x4 p0, u32x4 p1, float t, uint32_t& c0,
                                           uint32_t& c1, uint32_t& sc, float& sb) {
  const uint32_t w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
  uint32_t am = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) am = max(am, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
  float xs[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    xs[2 * k] = __uint_as_float(w[k] << 16);
    xs[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
  }
  const float amax = bf16_to_f32(am);
  const float vs = (amax / 6.0f) / t;
  sc = e4m3_encode(vs);
  sb = e4m3_value(sc);
  const float d = sb * t;
  float qv[16];
  if (d >= 0x1p-96f) {
    const float yr = 1.0f / d;
#pragma unroll
    for (int k = 0; k < 16; ++k) qv[k] = div_rn(xs[k], d, yr);
  } else if (d > 0.0f) {
#pragma unroll
    for (int k = 0; k < 16; ++k) qv[k] = xs[k] / d;
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) qv[k] = xs[k] * 0.0f;  // signed zero: magnitude code 0
  }
  float lo[8], hi[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    lo[k] = qv[k];
    hi[k] = qv[8 + k];
  }
  c0 = e2m1_pack8(lo);
  c1 = e2m1_pack8(hi);
}

template <bool TL>
__global__ void __launch_bounds__(SK_T, 1) k_gemm_decode_fused(FusedArgs p) {
  using L = SlotLayout<FP4Q_NVFP4>;
  __shared__ __attribute__((aligned(16))) v4f32s red[SK_WAVES * 4 * SK_CG * 64];   // 96 KB
  __shared__ __attribute__((aligned(16))) uint8_t sScale[SK_WAVES * 2 * L::BYTES];
  __shared__ __attribute__((aligned(16))) uint16_t sR[SK_M * SK_SRS];
  __shared__ __attribute__((aligned(16))) uint16_t sB[SK_COLS * SK_SRS];
  __shared__ uint32_t sMax[SK_WAVES];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int q = lane >> 4, lr = lane & 15;
  const int64_t col0 = (int64_t)blockIdx.x * SK_COLS;
  const int nk = (int)(p.K / 128);
  const int nS = p.nS;
  const float tw = *p.bts;
  const int my_ch_raw = *(nS > 0 ? p.chan + (lane < nS ? lane : nS - 1)
                                 : reinterpret_cast<const int32_t*>(p.bts));
  const int my_ch = (nS > 0 && lane < nS) ? my_ch_raw : -1;

  // prepared compensation weights into sB (as k_gemm_skinny with PB)
  const int nc = (nS + 31) >> 5;
  const bool pb_on = nS > 0 && t < SK_CG * 64 * nc;
  int pb_g = 0, pb_c = 0;
  u32x4 pbv = u32x4{0u, 0u, 0u, 0u};
  {
    const int blk = pb_on ? t >> 6 : 0;
    pb_g = blk / (nc > 0 ? nc : 1);
    pb_c = blk - pb_g * nc;
    const int64_t glast = ((p.N + 15) >> 4) - 1;
    int64_t gi = (col0 >> 4) + pb_g;
    gi = gi < glast ? gi : glast;
    if (pb_on)
      pbv = *reinterpret_cast<const u32x4*>(p.bsel + ((gi * nc + pb_c) << 10) + (t & 63) * 16);
  }
  int64_t wso = 0;
  if (TL) {
    int64_t wrow = col0 + (lane < SK_COLS ? lane : SK_COLS - 1);
    const int64_t wlast = ((p.N + 63) & ~(int64_t)63) - 1;
    wrow = wrow < wlast ? wrow : wlast;
    wso = (wrow >> 6) * (p.K >> 7) * (8 * 64) + (wrow & 63) * 4;
  }
  // the first step's weights, then this wave's activations (steps wave and
  // wave + 8); the second step's weights follow once the first step's
  // activations are quantized (their registers are then free)
  const int k0 = wave < nk ? wave : nk - 1;
  const int k1 = wave + SK_WAVES < nk ? wave + SK_WAVES : nk - 1;
  Step s0, s1;
  load_w_step<TL>(p, k0, lane, col0, wso, s0);
  XSlab x0, x1;
  load_x_step(p, k0, lane, x0);
  load_x_step(p, k1, lane, x1);
  if (pb_on) {
    const int u = (t & 63) >> 4, r = t & 15;
    uint16_t* dst = sB + (16 * pb_g + r) * SK_SRS + 32 * pb_c + 8 * u;
    reinterpret_cast<u32x2*>(dst)[0] = u32x2{pbv.x, pbv.y};
    reinterpret_cast<u32x2*>(dst)[1] = u32x2{pbv.z, pbv.w};
  }

  // tensor amax: the 8 waves together hold every step of every row
  uint32_t m = max(slab_absmax(x0), slab_absmax(x1));
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if (lane == 0) sMax[wave] = m;
  __syncthreads();
  m = 0;
#pragma unroll
  for (int w2 = 0; w2 < SK_WAVES; ++w2) m = max(m, sMax[w2]);
  const float tx = nv_tensor_scale(bf16_to_f32(m));
  const bool writer = blockIdx.x == 0 && p.q_out != nullptr;
  if (writer && t == 0) *p.ts_out = tx;

  // quantize this wave's steps into the fragment registers; the residual of
  // the selected channels (R = bf16(x - (e2m1 sb) t), as the quantizer)
  // goes to sR, and workgroup 0 may write codes and scales out
  uint32_t xsc[2][4];
  auto quant_step = [&](const XSlab& x, int kt, bool valid, Step& s, uint32_t (&xs)[4])
      __attribute__((always_inline)) {
    const uint64_t mch = __ballot(my_ch >= 0 && (my_ch >> 7) == kt);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      uint32_t c[4], sc[2];
      float sbv[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
        nv_block16(x.v[a][2 * b], x.v[a][2 * b + 1], tx, c[2 * b], c[2 * b + 1], sc[b], sbv[b]);
      s.x[a] = u32x4{c[0], c[1], c[2], c[3]};
      xs[a] = sc[0] | (sc[1] << 8);
      const int64_t row = 16 * a + lr;
      if (writer && valid && row < p.M) {
        *reinterpret_cast<u32x4*>(p.q_out + row * (p.K >> 1) + (int64_t)kt * 64 + 16 * q) = s.x[a];
        *reinterpret_cast<uint16_t*>(p.s_out + row * (p.K >> 4) + (int64_t)kt * 8 + 2 * q) =
            (uint16_t)xs[a];
      }
      if (valid && mch) {
        // channels of this step in the lane's 32 columns
        for (uint64_t mm = mch; mm; mm &= mm - 1) {
          const int j = __builtin_ctzll(mm);
          const int cc = __builtin_amdgcn_ds_bpermute(j << 2, my_ch) & 127;
          if ((cc >> 5) != q) continue;
          const int e = cc & 31, b = e >> 4, k = e & 15;
          const uint32_t code = (c[2 * b + (k >> 3)] >> (4 * (k & 7))) & 15u;
          float pv = (e2m1_mag_value(code) * sbv[b]) * tx;
          if (code & 8u) pv = -pv;
          // element e of the lane's 32: piece e / 8, dword (e % 8) / 2, half e % 2
          const u32x4 pc = x.v[a][e >> 3];
          const int wi = (e & 7) >> 1;
          const uint32_t wd = wi == 0 ? pc.x : wi == 1 ? pc.y : wi == 2 ? pc.z : pc.w;
          const float xe = __uint_as_float((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
          if (row < p.M) sR[row * SK_SRS + j] = (uint16_t)f32_to_bf16_rne(xe - pv);
        }
      }
    }
  };
  quant_step(x0, k0, wave < nk, s0, xsc[0]);
  load_w_step<TL>(p, k1, lane, col0, wso, s1);
  quant_step(x1, k1, wave + SK_WAVES < nk, s1, xsc[1]);

  v4f32s acc[4][SK_CG];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) acc[a][g] = v4f32s{0.f, 0.f, 0.f, 0.f};

  // multiply: as process_step (NVFP4), the activation scales already in the
  // lane's own registers
  uint8_t* slot0 = sScale + (wave * 2 + 0) * L::BYTES;
  uint8_t* slot1 = sScale + (wave * 2 + 1) * L::BYTES;
  auto mult = [&](const Step& st, const uint32_t (&xs)[4], uint8_t* slot)
      __attribute__((always_inline)) {
    if (lane < SK_COLS) *reinterpret_cast<u32x2*>(slot + lane * 8) = st.wsc;
    h2s wsp[SK_CG], xsp[4];
#pragma unroll
    for (int g = 0; g < SK_CG; ++g)
      wsp[g] = sk_scales2((uint32_t)*reinterpret_cast<const uint16_t*>(slot + (16 * g + lr) * 8 + 2 * q));
#pragma unroll
    for (int a = 0; a < 4; ++a) xsp[a] = sk_scales2(xs[a]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      h8s db[SK_CG];
#pragma unroll
      for (int g = 0; g < SK_CG; ++g) db[g] = sk_decode8(st.w[g][s], (s >> 1) ? wsp[g].yy : wsp[g].xx);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const h8s da = sk_decode8(st.x[a][s], (s >> 1) ? xsp[a].yy : xsp[a].xx);
#pragma unroll
        for (int g = 0; g < SK_CG; ++g)
          acc[a][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(da, db[g], acc[a][g], 0, 0, 0);
      }
    }
  };
  if (wave < nk) mult(s0, xsc[0], slot0);
  if (wave + SK_WAVES < nk) mult(s1, xsc[1], slot1);

  // ---- K-partial sums meet in LDS (sR, sB complete too); wave a (< 4) then
  // owns rows 16a .. 16a+15
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) red[((wave * 4 + a) * SK_CG + g) * 64 + lane] = acc[a][g];
  __syncthreads();
  if (writer && nS > 0) {
    for (int i = t; i < (int)p.M * nS; i += SK_T) {
      const int row = i / nS, j = i - row * nS;
      p.r_out[i] = sR[row * SK_SRS + j];
    }
  }
  if (wave >= 4) return;
  v4f32s out[SK_CG];
#pragma unroll
  for (int g = 0; g < SK_CG; ++g) {
    out[g] = red[((0 * 4 + wave) * SK_CG + g) * 64 + lane];
#pragma unroll
    for (int w2 = 1; w2 < SK_WAVES; ++w2) out[g] += red[((w2 * 4 + wave) * SK_CG + g) * 64 + lane];
  }
  if (nS > 0) {
    v4f32s comp[SK_CG];
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) comp[g] = v4f32s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < SK_MAXS / 16; ++c) {
      const int jq = 16 * c + 4 * q;
      const u32x2 m2 = u32x2{(jq + 0 < nS ? 0xFFFFu : 0u) | (jq + 1 < nS ? 0xFFFF0000u : 0u),
                             (jq + 2 < nS ? 0xFFFFu : 0u) | (jq + 3 < nS ? 0xFFFF0000u : 0u)};
      const s4s ra = __builtin_bit_cast(
          s4s, *reinterpret_cast<const u32x2*>(sR + (16 * wave + lr) * SK_SRS + jq) & m2);
#pragma unroll
      for (int g = 0; g < SK_CG; ++g) {
        const s4s rb = __builtin_bit_cast(
            s4s, *reinterpret_cast<const u32x2*>(sB + (16 * g + lr) * SK_SRS + jq) & m2);
        comp[g] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ra, rb, comp[g], 0, 0, 0);
      }
    }
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) out[g] = out[g] * tx + comp[g];
  } else {
#pragma unroll
    for (int g = 0; g < SK_CG; ++g) out[g] *= tx;
  }
#pragma unroll
  for (int g = 0; g < SK_CG; ++g) {
    const int64_t col = col0 + 16 * g + lr;
    if (col >= p.N) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = 16 * wave + 4 * q + e;
      if (row >= p.M) continue;
      const float v = out[g][e] * tw;
      if (p.y_bf16)
        reinterpret_cast<uint16_t*>(p.y)[row * p.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
      else
        reinterpret_cast<float*>(p.y)[row * p.ldy + col] = v;
    }
  }
}

bool decode_fused_eligible(int64_t M, int64_t K, int nS) {
  return M >= 1 && M <= SK_M && K >= 128 && K % 128 == 0 && K <= 128 * 2 * SK_WAVES &&
         nS >= 0 && nS <= SK_MAXS;
}

int launch_gemm_decode_fused(bool tiled, int64_t M, int64_t N, int64_t K, const uint16_t* x,
                             int64_t ldx, const uint8_t* bq, const uint8_t* bs, const float* bts,
                             const int32_t* chan, int nS, const uint8_t* bsel, void* y, int y_bf16,
                             int64_t ldy, uint8_t* q_out, uint8_t* s_out, float* ts_out,
                             uint16_t* r_out, hipStream_t stream) {
  FusedArgs a{M, N, K, x, ldx, bq, bs, bts, chan, nS, bsel, y, y_bf16, ldy, q_out, s_out, ts_out,
              r_out};
  dim3 grid((unsigned)((N + SK_COLS - 1) / SK_COLS));
  if (tiled)
    hipLaunchKernelGGL((k_gemm_decode_fused<true>), grid, dim3(SK_T), 0, stream, a);
  else
    hipLaunchKernelGGL((k_gemm_decode_fused<false>), grid, dim3(SK_T), 0, stream, a);
  return 0;
}

bool skinny_gemm_eligible(int64_t M, int64_t N, int64_t K, int nS) {
  // the residual rows are read as 16-byte pieces of 8 entries (R itself is
  // 16-byte aligned)
  return M >= 1 && M <= SK_M && N >= 1 && K % 128 == 0 && nS <= SK_MAXS && (M * nS) % 8 == 0;
}

int launch_gemm_skinny(int fmt, bool tiled, int64_t M, int64_t N, int64_t K, const uint8_t* aq,
                       const uint8_t* as, const float* ats, const uint8_t* bq, const uint8_t* bs,
                       const float* bts, const int32_t* chan, int nS, const uint16_t* resid,
                       const float* cts, const uint8_t* bsel, void* y, int y_bf16, int64_t ldy,
                       hipStream_t stream) {
  SkinnyArgs a{M, N, K, aq, as, ats, bq, bs, bts, chan, nS, resid, cts, bsel, y, y_bf16, ldy};
  dim3 grid((unsigned)((N + SK_COLS - 1) / SK_COLS));
  const bool pb = bsel != nullptr && nS > 0;
#define FP4Q_SKINNY(F, T, P) hipLaunchKernelGGL((k_gemm_skinny<F, T, P>), grid, dim3(SK_T), 0, stream, a)
#define FP4Q_SKINNY_P(F, T) \
  if (pb) FP4Q_SKINNY(F, T, true); else FP4Q_SKINNY(F, T, false)
  if (fmt == FP4Q_NVFP4 && tiled) { FP4Q_SKINNY_P(FP4Q_NVFP4, true); }
  else if (fmt == FP4Q_NVFP4) { FP4Q_SKINNY_P(FP4Q_NVFP4, false); }
  else if (tiled) { FP4Q_SKINNY_P(FP4Q_MXFP4, true); }
  else { FP4Q_SKINNY_P(FP4Q_MXFP4, false); }
#undef FP4Q_SKINNY_P
#undef FP4Q_SKINNY
  return 0;
}

}  // namespace fp4q
