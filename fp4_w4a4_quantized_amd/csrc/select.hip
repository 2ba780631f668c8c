// select.hip -- online selection of the residual channels.
//
// The explainer of the QUADS paper (gist.science), section 2.2 B, keeps the
// channels with the largest residual through a binary top-k mask.  Read here
// as: the magnitude of channel c is the largest |R(m, c)| over the rows, R
// the BF16 residual bf16(x - deq(code)) that the quantizer emits for a
// selected channel; the k largest channels win, ties going to the lower
// index; the list comes out ascending, together with R on those channels.
//
// Four launches, none of them with atomics on global memory:
//  1. k_chan_score: a workgroup owns 512 columns and a block of rows; each
//     lane walks one 8-column chunk down its wave's rows (one contiguous
//     1 KB load of x per wave and row), keeps max |x - p| in FP32 and the
//     four waves meet in LDS.  Nearest-even rounding to BF16 is monotone, so
//     rounding that maximum once equals the maximum of the rounded residuals.
//     Each row block writes its partial maxima as BF16 magnitude bits.
//  2. k_chan_reduce (many row blocks only): maximum over the row blocks,
//     16 waves per 128 columns.  With few partial maxima the pick kernel
//     reduces them itself while it loads the scores.
//  3. k_chan_pick: one workgroup, the scores in LDS.  A BF16 magnitude is a
//     15-bit integer whose order is the order of the values, so the k-th
//     largest score T comes out of two histogram passes (high 8 bits, then
//     low 7 bits), no sort; a wave adds the lanes that share a bin with one
//     LDS atomic, since scores crowd into few exponents.  Then every thread
//     owns a contiguous column range, and two block-wide prefix sums place
//     the columns above T and the first k - #(> T) columns equal to T, in
//     index order: the ascending list.
//  4. k_chan_resid: R on the chosen channels, one thread per (8 rows, j),
//     with the quantizer's own FP32 operations; the eight rows' gathers are
//     in flight together.
//
// Grouped (the MoE form: each expert's rows choose their own channels, with
// the expert's tensor scale): the score tiles are (group, row block) in
// group order, each workgroup finding its tile by a block-wide scan over the
// groups' block counts; the pick runs one workgroup per group, reducing the
// group's partial maxima while it loads them into LDS (an empty group scores
// zero everywhere and takes the first k channels, the tie rule); each
// residual row takes its group's list and tensor scale.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

namespace {

constexpr int SC_THREADS = 256;   // 4 waves
constexpr int SC_CHUNKS = 64;     // 8-column chunks per score workgroup (one per lane)
constexpr int SC_TARGET_WG = 1024;
constexpr int RD_THREADS = 1024;  // 16 waves
constexpr int PK_THREADS = 1024;
constexpr int RS_THREADS = 256;
constexpr int RS_ROWS = 8;             // rows per residual thread
constexpr int PK_LDS_COLS = 30720;     // scores held in LDS up to this many columns (60 KB)
constexpr int64_t PK_FUSE_ENTRIES = 65536;  // partial maxima the pick kernel reduces itself

typedef float v2f32 __attribute__((ext_vector_type(2)));

inline size_t round256(size_t b) { return (b + 255) / 256 * 256; }

struct ScorePlan {
  int64_t rb;     // rows per score workgroup (a multiple of 4)
  int64_t parts;  // row blocks
};

// Enough workgroups to cover the chip about once; at least 16 rows each.
ScorePlan score_plan(int64_t rows, int64_t cols) {
  const int64_t gx = (cols / 8 + SC_CHUNKS - 1) / SC_CHUNKS;
  const int64_t want = (SC_TARGET_WG + gx - 1) / gx;
  int64_t rb = (rows + want - 1) / want;
  rb = (rb + 3) / 4 * 4;
  if (rb < 16) rb = 16;
  const int64_t parts = rows > 0 ? (rows + rb - 1) / rb : 1;
  return {rb, parts};
}

// The partial maxima get their own reduction launch unless the pick kernel
// can take them while it loads the scores into LDS.
bool reduce_launch(int64_t parts, int64_t cols) {
  return parts > 1 && (cols > PK_LDS_COLS || parts * cols > PK_FUSE_ENTRIES);
}

// Signed dequantized value of a code as the quantizer forms it for the
// residual: (e2m1 * E4M3 scale) * t for NVFP4, e2m1 * 2^e for MXFP4.
template <int FMT>
__device__ __forceinline__ float deq_code(uint32_t code, float s, float t) {
  float p = (FMT == FP4Q_NVFP4) ? (e2m1_mag_value(code) * s) * t : e2m1_mag_value(code) * s;
  return (code & 8u) ? -p : p;
}

template <int FMT>
__device__ __forceinline__ float block_scale(uint32_t sc) {
  return (FMT == FP4Q_NVFP4) ? e4m3_value(sc) : exp2i((int)sc - 127);
}

// Grouped score tiles: group g has ceil(rows_g / rb) row blocks, tiles in
// group order.  Finds tile `tile`'s group and row range (thread t counts
// groups 8t .. 8t + 7, G <= 2048); false past the last tile (uniform).
__device__ bool grouped_tile(const int32_t* __restrict__ off, int G, int64_t rb, int tile,
                             int* s_wsum, int* s_res, int& g, int64_t& r0, int64_t& r1) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int gg = t * 8 + i;
    if (gg < G) cnt += (int)((off[gg + 1] - off[gg] + rb - 1) / rb);
  }
  int incl = cnt;
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == 63) s_wsum[wave] = incl;
  if (t == 0) s_res[0] = -1;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wsum[w];
  const int excl = before + incl - cnt;
  if (tile >= excl && tile < excl + cnt) {
    int acc = excl;
    for (int i = 0; i < 8; ++i) {
      const int gg = t * 8 + i;
      const int c = (gg < G) ? (int)((off[gg + 1] - off[gg] + rb - 1) / rb) : 0;
      if (tile < acc + c) {
        s_res[0] = gg;
        s_res[1] = tile - acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  if (s_res[0] < 0) return false;
  g = s_res[0];
  r0 = off[g] + (int64_t)s_res[1] * rb;
  r1 = min((int64_t)off[g + 1], r0 + rb);
  return true;
}

template <int FMT, bool GROUPED>
__global__ __launch_bounds__(SC_THREADS) void k_chan_score(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, bool tiled,
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ scales,
    const float* __restrict__ tscale, int64_t rb, const int32_t* __restrict__ off, int G,
    uint16_t* __restrict__ part) {
  constexpr int CPB = (FMT == FP4Q_NVFP4) ? 2 : 4;  // chunks per scale block
  __shared__ uint32_t red[4 * SC_CHUNKS * 8];
  __shared__ int s_wsum[4];
  __shared__ int s_res[2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t cc = (int64_t)blockIdx.x * SC_CHUNKS + lane;
  int64_t r0 = (int64_t)blockIdx.y * rb;
  int64_t r1 = min(rows, r0 + rb);
  int grp = 0;
  if (GROUPED && !grouped_tile(off, G, rb, (int)blockIdx.y, s_wsum, s_res, grp, r0, r1)) return;
  const float t = (FMT == FP4Q_NVFP4) ? tscale[grp] : 1.0f;

  float m[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) m[k] = 0.0f;

  if (cc < (cols >> 3)) {
    // four rows of this wave per step, issued together; a row past the
    // block repeats the step's first row, which leaves the maximum unchanged
    for (int64_t r = r0 + wave; r < r1; r += 16) {
      u32x4 v[4];
      uint32_t cw[4], sc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t rr = (r + 4 * u < r1) ? r + 4 * u : r;
        v[u] = *reinterpret_cast<const u32x4*>(x + rr * ldx + 8 * cc);
        cw[u] = *reinterpret_cast<const uint32_t*>(q + code_off(tiled, rr, 4 * cc, cols));
        sc[u] = scales[scale_off<FMT>(tiled, rr, cc / CPB, cols)];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float s = block_scale<FMT>(sc[u]);
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        // signed E2M1 values of the eight codes (exact; code 8 may give
        // either zero, which |x - p| does not see)
        const v2f32 e[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], 1.0f, 0),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], 1.0f, 1),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], 1.0f, 2),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], 1.0f, 3)};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float xk = __uint_as_float(h ? (w[b] & 0xFFFF0000u) : (w[b] << 16));
            const float p = (FMT == FP4Q_NVFP4) ? (e[b][h] * s) * t : e[b][h] * s;
            m[2 * b + h] = fmaxf(m[2 * b + h], fabsf(xk - p));
          }
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) red[(wave * SC_CHUNKS + lane) * 8 + k] = __float_as_uint(m[k]);
  __syncthreads();

  // thread t: columns 2t and 2t+1 of the workgroup's 512 (chunk t/4)
  const int t2 = threadIdx.x;
  const int64_t col = (int64_t)blockIdx.x * SC_CHUNKS * 8 + 2 * t2;
  if (col < cols) {
    const int l = t2 >> 2, k0 = (t2 & 3) * 2;
    uint32_t a = 0, b = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      a = max(a, red[(w * SC_CHUNKS + l) * 8 + k0]);
      b = max(b, red[(w * SC_CHUNKS + l) * 8 + k0 + 1]);
    }
    const uint32_t lo = f32_to_bf16_rne(__uint_as_float(a));
    const uint32_t hi = f32_to_bf16_rne(__uint_as_float(b));
    *reinterpret_cast<uint32_t*>(part + (int64_t)blockIdx.y * cols + col) = lo | (hi << 16);
  }
}

__global__ __launch_bounds__(RD_THREADS) void k_chan_reduce(const uint16_t* __restrict__ part,
                                                            int64_t parts, int64_t cols,
                                                            uint16_t* __restrict__ score) {
  __shared__ uint32_t red[16][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 128 + 2 * lane;
  uint32_t lo = 0, hi = 0;
  if (c < cols) {
    // eight row blocks per wave and step, loads issued together (a block
    // past the end repeats the wave's first, which leaves the maximum alone)
    for (int64_t p = wave; p < parts; p += 16 * 8) {
      uint32_t w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t pp = (p + 16 * u < parts) ? p + 16 * u : p;
        w[u] = *reinterpret_cast<const uint32_t*>(part + pp * cols + c);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        lo = max(lo, w[u] & 0xFFFFu);
        hi = max(hi, w[u] >> 16);
      }
    }
  }
  red[wave][lane] = lo | (hi << 16);
  __syncthreads();
  if (wave == 0 && c < cols) {
#pragma unroll
    for (int w = 1; w < 16; ++w) {
      const uint32_t v = red[w][lane];
      lo = max(lo, v & 0xFFFFu);
      hi = max(hi, v >> 16);
    }
    *reinterpret_cast<uint32_t*>(score + c) = lo | (hi << 16);
  }
}

// Exclusive prefix sum of v over the 1024 threads of the workgroup.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  __syncthreads();
  return pre + x - v;
}

// Run by the 64 lanes of wave 0.  hist[NB] counts; 1 <= need <= the total.
// Finds the bin b with above(b) < need <= above(b) + hist[b], where above(b)
// counts the entries of the bins above b, and stores b and above(b).
template <int NB>
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t need, uint32_t* out) {
  constexpr int Q = NB / 64;
  const int lane = threadIdx.x;
  uint32_t loc = 0;
#pragma unroll
  for (int i = 0; i < Q; ++i) loc += hist[lane * Q + i];
  uint32_t suf = loc;  // sum over lanes >= this one
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(suf, off);
    if (lane + off < 64) suf += y;
  }
  uint32_t acc = suf - loc;
  if (acc < need && need <= suf) {
#pragma unroll
    for (int i = Q - 1; i >= 0; --i) {
      const uint32_t h = hist[lane * Q + i];
      if (acc + h >= need) {
        out[0] = (uint32_t)(lane * Q + i);
        out[1] = acc;
        break;
      }
      acc += h;
    }
  }
}

// Histogram add from the whole wave: lanes whose bin equals the first
// pending lane's bin add once, for two rounds; the rest add one by one.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool valid) {
  const int lane = threadIdx.x & 63;
  uint64_t pend = __ballot(valid);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    if (pend == 0) break;
    const int first = __builtin_ctzll(pend);
    const uint32_t b = __shfl(bin, first);
    const uint64_t same = __ballot(bin == b) & pend;
    if (lane == first) atomicAdd(&hist[b], (uint32_t)__popcll(same));
    pend &= ~same;
  }
  if ((pend >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
}

// LDS: scores kept in LDS (cols <= PK_LDS_COLS), each the maximum
// of `parts` partial rows of `part`; otherwise parts == 1 and the scores
// are read from `part` itself.  GROUPED (LDS only): workgroup g picks for
// group g, whose partial rows are its score tiles (ceil(rows_g / rb) of them,
// after those of the groups before it); chan is [G, k].
template <bool LDS, bool GROUPED>
__global__ __launch_bounds__(PK_THREADS) void k_chan_pick(const uint16_t* __restrict__ part,
                                                          int parts, int cols, int k,
                                                          int32_t* __restrict__ chan,
                                                          const int32_t* __restrict__ off,
                                                          int64_t rb) {
  __shared__ uint16_t s_score[LDS ? PK_LDS_COLS : 2];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel[4];
  __shared__ int wsum[16];
  const int t = threadIdx.x;
  if (GROUPED) {
    // this group's first tile: the sum of the block counts of the groups
    // before it (a block-wide sum)
    const int g = blockIdx.x;
    int sum = 0;
    for (int gg = t; gg < g; gg += PK_THREADS)
      sum += (int)((off[gg + 1] - off[gg] + rb - 1) / rb);
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_down(sum, o);
    if ((t & 63) == 0) wsum[t >> 6] = sum;
    __syncthreads();
    int first = 0;
    for (int w = 0; w < PK_THREADS / 64; ++w) first += wsum[w];
    __syncthreads();  // wsum is reused by the scans below
    parts = (int)((off[g + 1] - off[g] + rb - 1) / rb);
    part += (int64_t)first * cols;
    chan += (int64_t)g * k;
  }

  if (t < 256) hist[t] = 0;
  // the scores were written by other workgroups, so every load goes out to
  // memory: loads are issued eight at a time rather than one after another
  if (LDS && parts == 1) {
    for (int c0 = t; c0 < cols; c0 += 8 * PK_THREADS) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * PK_THREADS;
        v[u] = c < cols ? part[c] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * PK_THREADS;
        if (c < cols) s_score[c] = (uint16_t)v[u];
      }
    }
  } else if (LDS) {
    for (int c = t; c < cols; c += PK_THREADS) {
      uint32_t m = 0;
      for (int p0 = 0; p0 < parts; p0 += 8) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = p0 + u < parts ? part[(int64_t)(p0 + u) * cols + c] : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) m = max(m, v[u]);
      }
      s_score[c] = (uint16_t)m;
    }
  }
  const uint16_t* score = LDS ? s_score : part;
  __syncthreads();
  for (int base = 0; base < cols; base += PK_THREADS) {
    const int c = base + t;
    const uint32_t s = c < cols ? score[c] : 0u;
    hist_add(hist, s >> 7, c < cols);
  }
  __syncthreads();
  if (t < 64) find_bin<256>(hist, (uint32_t)k, sel);
  __syncthreads();
  const uint32_t b1 = sel[0], above1 = sel[1];
  if (t < 128) hist[t] = 0;
  __syncthreads();
  for (int base = 0; base < cols; base += PK_THREADS) {
    const int c = base + t;
    const uint32_t s = c < cols ? score[c] : 0u;
    hist_add(hist, s & 0x7Fu, c < cols && (s >> 7) == b1);
  }
  __syncthreads();
  if (t < 64) find_bin<128>(hist, (uint32_t)k - above1, sel + 2);
  __syncthreads();
  const uint32_t T = (b1 << 7) | sel[2];
  const int need_eq = k - (int)(above1 + sel[3]);  // columns equal to T to take, >= 1

  const int cpt = (cols + PK_THREADS - 1) / PK_THREADS;
  const int c0 = min(cols, t * cpt), c1 = min(cols, c0 + cpt);
  int gt = 0, eq = 0;
  for (int c = c0; c < c1; ++c) {
    const uint32_t s = score[c];
    gt += s > T;
    eq += s == T;
  }
  const int eq_before = block_excl_scan(eq, wsum);
  int take = min(max(need_eq - eq_before, 0), eq);
  int o = block_excl_scan(gt + take, wsum);
  // o stays below k by construction; the bound keeps the stores inside
  // chan[k] whatever the scores hold
  for (int c = c0; c < c1 && o < k; ++c) {
    const uint32_t s = score[c];
    if (s > T) {
      chan[o++] = c;
    } else if (s == T && take > 0) {
      chan[o++] = c;
      --take;
    }
  }
}

// GROUPED: row r takes the list and tensor scale of its group (chan [G, k]).
template <int FMT, bool GROUPED>
__global__ __launch_bounds__(RS_THREADS) void k_chan_resid(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, bool tiled,
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ scales,
    const float* __restrict__ tscale, const int32_t* __restrict__ chan, uint32_t k,
    uint32_t total, uint16_t* __restrict__ resid, const int32_t* __restrict__ off, int G) {
  constexpr int BLK = (FMT == FP4Q_NVFP4) ? 16 : 32;
  const uint32_t i = blockIdx.x * RS_THREADS + threadIdx.x;
  if (i >= total) return;
  const uint32_t rg = i / k, j = i - rg * k;
  const int64_t r0 = (int64_t)rg * RS_ROWS;
  const int nr = (int)min((int64_t)RS_ROWS, rows - r0);
  // the group of each row (GROUPED): the last group starting at or before r0,
  // then forward over the rows (empty groups skipped)
  int gr[RS_ROWS];
  if (GROUPED) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= r0) lo = mid; else hi = mid - 1;
    }
    int g = lo;
#pragma unroll
    for (int u = 0; u < RS_ROWS; ++u) {
      const int64_t r = r0 + (u < nr ? u : nr - 1);
      while (g < G - 1 && off[g + 1] <= r) ++g;
      gr[u] = g;
    }
  } else {
#pragma unroll
    for (int u = 0; u < RS_ROWS; ++u) gr[u] = 0;
  }
  uint32_t xv[RS_ROWS], cb[RS_ROWS], sc[RS_ROWS];
  int64_t cu[RS_ROWS];
#pragma unroll
  for (int u = 0; u < RS_ROWS; ++u) {
    const int64_t r = r0 + (u < nr ? u : nr - 1);  // past the end: repeat the last row
    // in range by construction
    const int64_t c = min(max((int64_t)chan[(int64_t)gr[u] * k + j], (int64_t)0), cols - 1);
    cu[u] = c;
    xv[u] = x[r * ldx + c];
    cb[u] = q[code_off(tiled, r, c >> 1, cols)];
    sc[u] = scales[scale_off<FMT>(tiled, r, c / BLK, cols)];
  }
#pragma unroll
  for (int u = 0; u < RS_ROWS; ++u) {
    if (u < nr) {
      const int64_t c = cu[u];
      const float t = (FMT == FP4Q_NVFP4) ? tscale[gr[u]] : 1.0f;
      const uint32_t code = (c & 1) ? (cb[u] >> 4) : (cb[u] & 15u);
      const float p = deq_code<FMT>(code, block_scale<FMT>(sc[u]), t);
      resid[(r0 + u) * k + j] = (uint16_t)f32_to_bf16_rne(bf16_to_f32(xv[u]) - p);
    }
  }
}

// Steps 2-4 from the partial maxima part [nparts, cols]; sbuf: cols entries
// for the reduction's output (used when it gets its own launch).
template <int FMT>
void select_from_parts(bool tiled, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                       const uint8_t* q, const uint8_t* scales, const float* tscale, int k,
                       int32_t* chan, uint16_t* resid, const uint16_t* part, int64_t nparts,
                       uint16_t* sbuf, hipStream_t stream) {
  const uint16_t* score = part;
  int parts = (int)nparts;
  if (reduce_launch(nparts, cols)) {
    hipLaunchKernelGGL(k_chan_reduce, dim3((unsigned)((cols + 127) / 128)), dim3(RD_THREADS), 0,
                       stream, part, nparts, cols, sbuf);
    score = sbuf;
    parts = 1;
  }
  if (cols <= PK_LDS_COLS)
    hipLaunchKernelGGL((k_chan_pick<true, false>), dim3(1), dim3(PK_THREADS), 0, stream, score,
                       parts, (int)cols, k, chan, nullptr, (int64_t)1);
  else
    hipLaunchKernelGGL((k_chan_pick<false, false>), dim3(1), dim3(PK_THREADS), 0, stream, score,
                       1, (int)cols, k, chan, nullptr, (int64_t)1);
  const int64_t groups = (rows + RS_ROWS - 1) / RS_ROWS;
  const uint32_t total = (uint32_t)(groups * k);
  if (total > 0)
    hipLaunchKernelGGL((k_chan_resid<FMT, false>), dim3((total + RS_THREADS - 1) / RS_THREADS),
                       dim3(RS_THREADS), 0, stream, x, rows, cols, ldx, tiled, q, scales, tscale,
                       chan, (uint32_t)k, total, resid, nullptr, 1);
}

template <int FMT>
void launch_select_fmt(bool tiled, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                       const uint8_t* q, const uint8_t* scales, const float* tscale, int k,
                       int32_t* chan, uint16_t* resid, void* ws, hipStream_t stream) {
  const ScorePlan pl = score_plan(rows, cols);
  uint16_t* part = static_cast<uint16_t*>(ws);
  const dim3 sg((unsigned)((cols / 8 + SC_CHUNKS - 1) / SC_CHUNKS), (unsigned)pl.parts);
  hipLaunchKernelGGL((k_chan_score<FMT, false>), sg, dim3(SC_THREADS), 0, stream, x, rows, cols,
                     ldx, tiled, q, scales, tscale, pl.rb, nullptr, 1, part);
  uint16_t* sbuf =
      reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + round256((size_t)pl.parts * cols * 2));
  select_from_parts<FMT>(tiled, x, rows, cols, ldx, q, scales, tscale, k, chan, resid, part,
                         pl.parts, sbuf, stream);
}

// Grouped: score tiles (group, row block) bounded by ceil(rows / rb) + G.
template <int FMT>
void launch_select_grouped_fmt(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                               const uint8_t* q, const uint8_t* scales, const float* tscale,
                               const int32_t* off, int G, int k, int32_t* chan, uint16_t* resid,
                               void* ws, hipStream_t stream) {
  const ScorePlan pl = score_plan(rows, cols);
  const int64_t tiles = (rows + pl.rb - 1) / pl.rb + G;
  uint16_t* part = static_cast<uint16_t*>(ws);
  const dim3 sg((unsigned)((cols / 8 + SC_CHUNKS - 1) / SC_CHUNKS), (unsigned)tiles);
  hipLaunchKernelGGL((k_chan_score<FMT, true>), sg, dim3(SC_THREADS), 0, stream, x, rows, cols,
                     ldx, false, q, scales, tscale, pl.rb, off, G, part);
  hipLaunchKernelGGL((k_chan_pick<true, true>), dim3((unsigned)G), dim3(PK_THREADS), 0, stream,
                     part, 0, (int)cols, k, chan, off, pl.rb);
  const int64_t groups = (rows + RS_ROWS - 1) / RS_ROWS;
  const uint32_t total = (uint32_t)(groups * k);
  if (total > 0)
    hipLaunchKernelGGL((k_chan_resid<FMT, true>), dim3((total + RS_THREADS - 1) / RS_THREADS),
                       dim3(RS_THREADS), 0, stream, x, rows, cols, ldx, false, q, scales, tscale,
                       chan, (uint32_t)k, total, resid, off, G);
}

}  // namespace

size_t select_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0) return 0;
  const ScorePlan pl = score_plan(rows, cols);
  size_t b = round256((size_t)pl.parts * (size_t)cols * 2);
  if (reduce_launch(pl.parts, cols)) b += round256((size_t)cols * 2);
  return b;
}

size_t select_grouped_workspace_bytes(int64_t rows, int64_t cols, int G) {
  if (rows < 0 || cols <= 0 || G < 1) return 0;
  const ScorePlan pl = score_plan(rows, cols);
  const int64_t tiles = (rows + pl.rb - 1) / pl.rb + G;
  return round256((size_t)tiles * (size_t)cols * 2);
}

bool select_grouped_cols_ok(int64_t cols) { return cols <= PK_LDS_COLS; }

// The scored quantizer's partial maxima (bands x cols), then the reduction's
// output when it gets a launch of its own.
size_t select_scored_workspace_bytes(int64_t bands, int64_t cols) {
  if (bands < 1 || cols <= 0) return 0;
  size_t b = round256((size_t)bands * (size_t)cols * 2);
  if (reduce_launch(bands, cols)) b += round256((size_t)cols * 2);
  return b;
}

void launch_select_scored(int fmt, bool tiled, const uint16_t* x, int64_t rows, int64_t cols,
                          int64_t ldx, const uint8_t* q, const uint8_t* scales,
                          const float* tscale, int k, int32_t* chan, uint16_t* resid,
                          const uint16_t* part, int64_t bands, void* ws, hipStream_t stream) {
  uint16_t* sbuf =
      reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + round256((size_t)bands * cols * 2));
  if (fmt == FP4Q_NVFP4)
    select_from_parts<FP4Q_NVFP4>(tiled, x, rows, cols, ldx, q, scales, tscale, k, chan, resid,
                                  part, bands, sbuf, stream);
  else
    select_from_parts<FP4Q_MXFP4>(tiled, x, rows, cols, ldx, q, scales, tscale, k, chan, resid,
                                  part, bands, sbuf, stream);
}

void launch_select_grouped(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                           const uint8_t* q, const uint8_t* scales, const float* tscale,
                           const int32_t* off, int G, int k, int32_t* chan, uint16_t* resid,
                           void* ws, hipStream_t stream) {
  if (fmt == FP4Q_NVFP4)
    launch_select_grouped_fmt<FP4Q_NVFP4>(x, rows, cols, ldx, q, scales, tscale, off, G, k, chan,
                                          resid, ws, stream);
  else
    launch_select_grouped_fmt<FP4Q_MXFP4>(x, rows, cols, ldx, q, scales, tscale, off, G, k, chan,
                                          resid, ws, stream);
}

void launch_select(int fmt, bool tiled, const uint16_t* x, int64_t rows, int64_t cols,
                   int64_t ldx, const uint8_t* q, const uint8_t* scales, const float* tscale,
                   int k, int32_t* chan, uint16_t* resid, void* ws, hipStream_t stream) {
  if (fmt == FP4Q_NVFP4)
    launch_select_fmt<FP4Q_NVFP4>(tiled, x, rows, cols, ldx, q, scales, tscale, k, chan, resid,
                                  ws, stream);
  else
    launch_select_fmt<FP4Q_MXFP4>(tiled, x, rows, cols, ldx, q, scales, tscale, k, chan, resid,
                                  ws, stream);
}

}  // namespace fp4q
