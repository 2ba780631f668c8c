// quantize.hip -- online activation (and weight) quantization to NVFP4 /
// MXFP4 with residual emission on selected channels.
//
// QUADS abstract: activations are quantized online every forward pass and
// suffer the coarse E2M1 grid; the explainer's section 2.2 B and the
// FourSight abstract keep a residual for a few selected channels.
//
// Work unit: one lane owns one 16-byte chunk (8 BF16 elements), so a wave's
// loads and code stores are fully contiguous.  A scale block is 2 (NVFP4) or
// 4 (MXFP4) neighbouring lanes; they combine their maxima with DPP lane moves
// and compute the scale redundantly; the block's first lane stores the scale
// byte.  Element quotients use a per-block reciprocal with exact FMA
// corrections (bit-identical to IEEE division); E2M1 rounding and packing use
// the hardware FP4 conversion.  Each lane writes its 8 codes with one 32-bit
// store.  The residual
// channels of a chunk come from a per-workgroup table in LDS (first channel
// index and an 8-bit mask per column chunk), built once from the channel
// list.
//
// NVFP4 needs the tensor (or per-expert group) amax before any block scale:
//  * small dense tensors (the decode regime): one launch; each workgroup
//    takes the maximum of the chunks it holds, the workgroups combine them
//    through a grid-wide maximum made of agent-scope atomics (grid_max
//    below), then quantize their chunks -- no second launch and no
//    workspace;
//  * large dense tensors: a partial-amax pass writes one maximum per
//    workgroup to the workspace; each quantize workgroup reduces those
//    first;
//  * expert groups: atomic max of the FP32 bit pattern per group (exact and
//    order-free for non-negative values) after a fill kernel clears the
//    words.
// MXFP4 is a single pass.
#include <algorithm>
#include <atomic>

#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

constexpr int QT = 256;              // threads per workgroup, general path
constexpr int QU = 4;                // chunks per thread, general path
constexpr int FT = 512;              // threads per workgroup, fused small path
constexpr int64_t FUSED_MAX_CHUNKS = 32 * FT;  // small-tensor path up to 128K elements
constexpr bool SMALL_FUSED = true;   // small tensors: one launch (else two short passes)
constexpr int AMAX_PARTS = 1024;     // partial maxima of the dense large path
constexpr int AMAX_BATCH = 16;       // loads in flight per thread in amax scans
constexpr int TAB_MAX = 2048;        // column chunks covered by the LDS channel table

typedef float f32x4q __attribute__((ext_vector_type(4)));

// Group of a row: the g with off[g] <= row < off[g+1] (binary search).
__device__ __forceinline__ int group_of_row(const int32_t* __restrict__ off, int G, int64_t row) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Largest BF16 magnitude pattern of 8 packed elements.
__device__ __forceinline__ uint32_t absmax8(u32x4 v) {
  uint32_t m = max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu);
  m = max(m, max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  m = max(m, max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu));
  return max(m, max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu));
}

// Row and column chunk of flat chunk index c (< 2^31): quotient estimated in
// FP64 (exact operands, error far below one) and corrected by one step.
struct ChunkGrid {
  const uint16_t* x;
  uint32_t cpr;      // 16-byte chunks per row
  int64_t ldx;       // row stride in elements
  double rcp;        // 1 / cpr
  bool contig;       // ldx == cols: chunk c sits at x + 8c
};

__device__ __forceinline__ void chunk_rc(const ChunkGrid& gr, uint32_t c, uint32_t& r, uint32_t& cc) {
  uint32_t q = (uint32_t)((double)c * gr.rcp);
  int32_t rem = (int32_t)(c - q * gr.cpr);
  if (rem < 0) { --q; rem += (int32_t)gr.cpr; }
  else if (rem >= (int32_t)gr.cpr) { ++q; rem -= (int32_t)gr.cpr; }
  r = q;
  cc = (uint32_t)rem;
}

__device__ __forceinline__ u32x4 load_chunk(const ChunkGrid& gr, uint32_t c) {
  const uint16_t* p;
  if (gr.contig) {
    p = gr.x + (int64_t)c * 8;
  } else {
    uint32_t r, cc;
    chunk_rc(gr, c, r, cc);
    p = gr.x + (int64_t)r * gr.ldx + (int64_t)cc * 8;
  }
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Max |x| (BF16 magnitude pattern) over the chunks first, first + stride, ...
// below `end`, AMAX_BATCH independent loads in flight per thread; the rest
// in batches of eight, where a chunk past the end re-reads `first` (which
// leaves the maximum alone) instead of waiting for one load at a time.
__device__ __forceinline__ uint32_t strided_amax(const ChunkGrid& gr, uint32_t first, uint32_t end,
                                                 uint32_t stride) {
  constexpr int TAIL = 8;
  uint32_t m = 0;
  int64_t i = first;
  for (; i + (int64_t)(AMAX_BATCH - 1) * stride < end; i += (int64_t)AMAX_BATCH * stride) {
    u32x4 v[AMAX_BATCH];
#pragma unroll
    for (int u = 0; u < AMAX_BATCH; ++u) v[u] = load_chunk(gr, (uint32_t)(i + u * stride));
#pragma unroll
    for (int u = 0; u < AMAX_BATCH; ++u) m = max(m, absmax8(v[u]));
  }
  for (; i < end; i += (int64_t)TAIL * stride) {
    u32x4 v[TAIL];
#pragma unroll
    for (int u = 0; u < TAIL; ++u) {
      const int64_t c = i + (int64_t)u * stride;
      v[u] = load_chunk(gr, (uint32_t)(c < end ? c : first));
    }
#pragma unroll
    for (int u = 0; u < TAIL; ++u) m = max(m, absmax8(v[u]));
  }
  return m;
}

// Reduce a per-thread maximum across the workgroup; every thread gets it.
template <int NT>
__device__ __forceinline__ uint32_t wg_max(uint32_t m, uint32_t* red) {
  for (int s = 32; s > 0; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) m = max(m, red[i]);
  __syncthreads();
  return m;
}

// ---- NVFP4 tensor amax passes ---------------------------------------------

// Clear the amax words and pre-set every tensor scale to 1 (empty groups
// keep it).  A fill kernel rather than a memset so the sequence can be
// captured in a HIP graph.
__global__ void k_quant_init(uint32_t* __restrict__ amax_bits, float* __restrict__ tscale, int G,
                             int nwords) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nwords) amax_bits[i] = 0u;
  if (i < G) tscale[i] = 1.0f;
}

// Per-group amax.  Each workgroup owns a flat run of AMAX_WG_CHUNKS chunks
// (one batch of AMAX_BATCH loads per thread, all in flight together), which
// may start and end inside rows.  A run inside one group (most runs) is
// reduced across the workgroup and issues one atomic.  A run that crosses
// group boundaries keeps per-row maxima in LDS, and each row's maximum then
// goes to its group.
constexpr int AMAX_WG_CHUNKS = QT * AMAX_BATCH;
constexpr int AMAX_WG_ROWS = AMAX_WG_CHUNKS / 2 + 2;  // rows a run can touch (cpr >= 2)

__global__ void __launch_bounds__(QT) k_group_amax(ChunkGrid gr, int64_t rows,
                                                   const int32_t* __restrict__ off, int G,
                                                   uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t red[QT / 64];
  __shared__ uint32_t rmax[AMAX_WG_ROWS];
  const uint32_t cpr = gr.cpr, total = (uint32_t)(rows * cpr);
  const uint32_t c0 = blockIdx.x * (uint32_t)AMAX_WG_CHUNKS;
  const uint32_t c1 = c0 + AMAX_WG_CHUNKS < total ? c0 + AMAX_WG_CHUNKS : total;
  uint32_t r0, cc0, rl, ccl;
  chunk_rc(gr, c0, r0, cc0);
  chunk_rc(gr, c1 - 1, rl, ccl);
  const int g0 = group_of_row(off, G, r0);
  const int g1 = group_of_row(off, G, rl);
  if (g0 == g1) {
    uint32_t m = strided_amax(gr, c0 + threadIdx.x, c1, QT);
    m = wg_max<QT>(m, red);
    if (threadIdx.x == 0 && m) atomicMax(&amax_bits[g0], m << 16);
    return;
  }
  const uint32_t nrows = rl - r0 + 1;
  for (uint32_t i = threadIdx.x; i < nrows; i += QT) rmax[i] = 0u;
  __syncthreads();
  // chunk c0 + t + QT u: its row relative to r0 steps by QT / cpr rows and
  // QT % cpr chunks per u
  const uint32_t drow = (uint32_t)QT / cpr, dcc = (uint32_t)QT - drow * cpr;
  uint32_t rr, cc;
  chunk_rc(gr, c0 + threadIdx.x, rr, cc);
  rr -= r0;
  u32x4 v[AMAX_BATCH];
  uint32_t row[AMAX_BATCH];
#pragma unroll
  for (int u = 0; u < AMAX_BATCH; ++u) {
    const uint32_t cu = c0 + threadIdx.x + u * QT;
    v[u] = load_chunk(gr, cu < c1 ? cu : c0);
    row[u] = cu < c1 ? rr : (uint32_t)AMAX_WG_ROWS;
    rr += drow;
    cc += dcc;
    if (cc >= cpr) { cc -= cpr; ++rr; }
  }
#pragma unroll
  for (int u = 0; u < AMAX_BATCH; ++u)
    if (row[u] < nrows) atomicMax(&rmax[row[u]], absmax8(v[u]));
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < nrows; i += QT) {
    const uint32_t m = rmax[i];
    if (m) atomicMax(&amax_bits[group_of_row(off, G, r0 + i)], m << 16);
  }
}

// Tensor maximum across the workgroups of one launch (the small-tensor NVFP4
// path), through state kept at the front of the caller's workspace (zero
// before its first use): a launch counter, a status word and one 64-bit
// slot per workgroup.  Every access is an atomic at agent scope, performed
// where all XCDs see it, and no release fence is needed (one would write
// back the per-XCD L2).  A launch tags its slots with counter + 1 in the
// high 32 bits: each workgroup stores its maximum under the tag in its own
// slot (workgroup 0 also stores the tag with a zero maximum in the slots
// past the grid, so every slot always carries an earlier launch's tag,
// never the current one, before it is written), then the first wave loads
// the launch's slots, lane i slot i, until all carry the tag, and takes
// their maximum: one store and one load on the critical path.  Workgroup 0
// then advances the counter; every workgroup has read it by then (their
// slots carry the tag derived from it).  Every workgroup of the launch is
// resident at once (at most 32 workgroups of 512 threads).  Calls with
// different workspaces are independent; calls that share one must not
// overlap.
//
// The spins are bounded.  A workgroup whose spin runs out has no valid
// tensor maximum: it sets bit 0 of the status word and poisons what it
// writes (E4M3 NaN block scales, BF16 NaN residuals, and a NaN tensor scale
// from workgroup 0), so a GEMM on the result gives NaN instead of a silent
// wrong value; fp4q_quantize_status() reads and clears the word.
constexpr uint32_t GRID_SPIN_LIMIT = 1u << 22;
constexpr uint32_t GRID_SLOTS = 32;
constexpr int WS_STATUS = 1;           // u32 index of the status word
constexpr int WS_SLOT_BYTES = 256;     // byte offset of the slots
constexpr size_t WS_HEADER = 512;      // bytes before the amax words
constexpr uint32_t STATUS_GRID_EXPIRED = 1u;

// Test controls of the exchange (kernel arguments): the spin limit, and a
// workgroup that skips its slot store (-1: none).
struct GridCtl {
  uint32_t* state;   // workspace front: [0] counter, [1] status, slots at byte 256
  uint32_t spin;
  int skip;
};

// Host-side test hooks (fp4q_test_hook); zero / -1 in normal operation.
static std::atomic<uint32_t> g_hook_spin{0};
static std::atomic<int> g_hook_skip{-1};

void set_grid_hooks(uint32_t spin, int skip) {
  g_hook_spin.store(spin);
  g_hook_skip.store(skip);
}
uint32_t grid_hook_spin() { return g_hook_spin.load(); }
int grid_hook_skip() { return g_hook_skip.load(); }

// Opaque copy of `v` that can only be formed once `dep` is available.
__device__ __forceinline__ uint32_t after(uint32_t v, uint32_t dep) {
  asm volatile("" : "+v"(v) : "v"(dep));
  return v;
}

// The launch counter; read early, before the chunk loads are used.
__device__ __forceinline__ uint32_t grid_gen(const GridCtl& gc) {
  return __hip_atomic_load(gc.state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by all 64 lanes of the first wave of every workgroup with the
// workgroup's maximum (a BF16 magnitude pattern, below 2^15) and the
// counter; returns the launch's maximum in every lane, and in `expired`
// whether any of this workgroup's spins ran out.
__device__ __forceinline__ uint32_t grid_max(uint32_t m, uint32_t nwg, uint32_t gen,
                                             const GridCtl& gc, bool& expired) {
  const int lane = threadIdx.x & 63;
  uint64_t* slot = reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(gc.state) +
                                               WS_SLOT_BYTES);
  const uint32_t tag = gen + 1u;
  const uint64_t tagw = (uint64_t)tag << 32;
  if (lane == 0 && (int)blockIdx.x != gc.skip)
    __hip_atomic_store(&slot[blockIdx.x], tagw | m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (blockIdx.x == 0 && (uint32_t)lane >= nwg && (uint32_t)lane < GRID_SLOTS)
    __hip_atomic_store(&slot[lane], tagw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t v = tagw;
  bool ok = true;
  if ((uint32_t)lane < nwg) {
    ok = false;
    for (uint32_t i = 0; i < gc.spin; ++i) {
      v = __hip_atomic_load(&slot[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((uint32_t)(v >> 32) == tag) {
        ok = true;
        break;
      }
    }
  }
  uint32_t r = ok ? (uint32_t)v & 0x7FFFu : 0u;
  for (int s = 32; s > 0; s >>= 1) r = max(r, (uint32_t)__shfl_xor((int)r, s));
  expired = __ballot(!ok) != 0;
  if (expired && lane == 0)
    __hip_atomic_fetch_or(gc.state + WS_STATUS, STATUS_GRID_EXPIRED, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  if (blockIdx.x == 0 && lane == 0)
    __hip_atomic_store(gc.state, after(gen + 1u, r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return r;
}

// Dense, large: one partial maximum per workgroup.
__global__ void __launch_bounds__(QT) k_amax_partial(ChunkGrid gr, uint32_t total,
                                                     uint32_t* __restrict__ part) {
  __shared__ uint32_t red[QT / 64];
  uint32_t m = strided_amax(gr, blockIdx.x * QT + threadIdx.x, total, gridDim.x * QT);
  m = wg_max<QT>(m, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// ---- residual channel table --------------------------------------------------

// Entry for column chunk cc (columns 8cc .. 8cc+7): bits 0-7 mark the
// selected columns, bits 8-31 hold the index j of the first of them in S.
__device__ __forceinline__ void build_chan_table(const int32_t* __restrict__ S, int nS,
                                                 int64_t cpr, uint32_t* tab, int nt) {
  for (int i = threadIdx.x; i < cpr; i += nt) tab[i] = 0u;
  __syncthreads();
  for (int j = threadIdx.x; j < nS; j += nt) {
    const int c = S[j], cc = c >> 3;
    uint32_t v = 1u << (c & 7);
    if (j == 0 || (S[j - 1] >> 3) != cc) v |= (uint32_t)j << 8;
    atomicOr(&tab[cc], v);
  }
  __syncthreads();
}

// The same entry found by binary search in S (table too small, or a chunk
// of another group than the one the table was built for).
__device__ __forceinline__ uint32_t chan_entry_search(const int32_t* __restrict__ S, int nS,
                                                      int64_t cc) {
  const int c0 = (int)(cc * 8);
  int lo = 0, hi = nS;  // first j with S[j] >= c0
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (S[mid] < c0) lo = mid + 1; else hi = mid;
  }
  uint32_t mask = 0;
  for (int j = lo; j < nS && j < lo + 8; ++j) {
    const int c = S[j];
    if (c >= c0 + 8) break;
    mask |= 1u << (c - c0);
  }
  return mask | ((uint32_t)lo << 8);
}

// ---- one chunk ---------------------------------------------------------------

struct ChunkCodes {
  float xs[8];     // the chunk's values
  uint32_t packed; // its 8 codes, low nibble first
  uint32_t sc;     // block scale code
  float sb;        // NVFP4 block scale value
  float d;         // the divisor that maps x onto the grid (sb t, or 2^e)
};

// Codes and block scale of one 8-element chunk as the quantizer forms them.
// All lanes of the wave call this (the block max moves between lanes).
template <int FMT>
__device__ __forceinline__ ChunkCodes chunk_codes(u32x4 v, float t) {
  constexpr int CPB = (FMT == FP4Q_NVFP4) ? 2 : 4;  // chunks per scale block
  // block max over the 2 or 4 lanes of the block: DPP quad permutations
  // [1,0,3,2] (lane ^ 1) and [2,3,0,1] (lane ^ 2)
  uint32_t am = absmax8(v);
  am = max(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0xB1, 0xF, 0xF, false));
  if (CPB == 4) am = max(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0x4E, 0xF, 0xF, false));
  const float amax = bf16_to_f32(am);

  ChunkCodes r;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 8; ++k)
    r.xs[k] = __uint_as_float((k & 1) ? (w[k >> 1] & 0xFFFF0000u) : (w[k >> 1] << 16));

  float qv[8];
  r.sb = 0.0f;
  if (FMT == FP4Q_NVFP4) {
    const float vs = (amax / 6.0f) / t;
    r.sc = e4m3_encode(vs);
    r.sb = e4m3_value(r.sc);
    r.d = r.sb * t;
    if (r.d >= 0x1p-96f) {
      const float y = 1.0f / r.d;
#pragma unroll
      for (int k = 0; k < 8; ++k) qv[k] = div_rn(r.xs[k], r.d, y);
    } else if (r.d > 0.0f) {
#pragma unroll
      for (int k = 0; k < 8; ++k) qv[k] = r.xs[k] / r.d;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) qv[k] = r.xs[k] * 0.0f;  // signed zero: magnitude code 0
    }
    r.packed = e2m1_pack8(qv);
  } else {
    const int e = mx_exponent(amax);
    r.sc = (uint32_t)(e + 127);
    r.d = exp2i(e);
    r.packed = e2m1_pack8(r.xs, __uint_as_float(r.sc << 23));  // x / 2^e, exact
  }
  return r;
}

// Dequantized value of code `code` of a chunk: (e2m1 * sb) * t (NVFP4; the
// first product exact) or e2m1 * 2^e (MXFP4, exact) -- the value the
// residual subtracts.
template <int FMT>
__device__ __forceinline__ float chunk_deq(const ChunkCodes& r, uint32_t code, float t) {
  float p;
  if (FMT == FP4Q_NVFP4)
    p = (e2m1_mag_value(code) * r.sb) * t;
  else
    p = e2m1_mag_value(code) * r.d;
  return (code & 8u) ? -p : p;
}

// Quantize chunk cc of row `row` held in v.  All lanes of the wave call this
// (the block max moves between lanes); `active` gates the stores.
template <int FMT>
__device__ __forceinline__ void quantize_chunk(u32x4 v, bool active, bool poison, bool tiled,
                                               int64_t row, int64_t cc, int64_t cols, float t,
                                               uint32_t chan_ent, int nS,
                                               uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
                                               uint16_t* __restrict__ resid) {
  constexpr int CPB = (FMT == FP4Q_NVFP4) ? 2 : 4;  // chunks per scale block
  const ChunkCodes r = chunk_codes<FMT>(v, t);
  uint32_t sc = r.sc;
  const uint32_t packed = r.packed;
  if (!active) return;
  if (poison) sc = 0x7Fu;  // E4M3 NaN: no valid tensor scale (see grid_max)
  if ((cc & (CPB - 1)) == 0) scales[scale_off<FMT>(tiled, row, cc / CPB, cols)] = (uint8_t)sc;

  *reinterpret_cast<uint32_t*>(q + code_off(tiled, row, 4 * cc, cols)) = packed;

  // residual on the selected channels of this chunk
  uint32_t mask = chan_ent & 0xFFu;
  if (nS > 0 && mask) {
    int j = (int)(chan_ent >> 8);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (mask & (1u << k)) {
        const uint32_t code = (packed >> (4 * k)) & 15u;
        const float p = chunk_deq<FMT>(r, code, t);
        resid[row * nS + j] = poison ? (uint16_t)0x7FC0u : (uint16_t)f32_to_bf16_rne(r.xs[k] - p);
        ++j;
      }
    }
  }
}

// ---- the quantize kernel -------------------------------------------------------

// How NVFP4 finds its tensor scale.
enum { AMAX_NONE = 0, AMAX_GROUP_WORDS = 1, AMAX_PARTIALS = 2, AMAX_FUSED = 3 };

// TO (tiled order, for the tiled packed layout): chunk c covers block
// c / 256 of 16 rows x 16 chunks (one 1 KB block of codes), row-group major,
// row (c % 256) / 16 and chunk c % 16 inside it, so a wave's stores fill
// contiguous 64-byte runs of the tiled blocks while its loads still read
// 256-byte row segments.  Otherwise chunks run in row-major order.
template <int FMT, int MODE, int NT, int U, bool TO>
__global__ void __launch_bounds__(NT) k_quantize(
    ChunkGrid gr, int64_t rows, int64_t cols, bool tiled, const int32_t* __restrict__ off, int G,
    const int32_t* __restrict__ chan, int nS, uint8_t* __restrict__ q,
    uint8_t* __restrict__ scales, float* __restrict__ tscale, uint16_t* __restrict__ resid,
    const uint32_t* __restrict__ amax_words, int nparts, GridCtl gc) {
  __shared__ uint32_t red[NT / 64];
  __shared__ uint32_t tab[TAB_MAX];
  const uint32_t cpr = gr.cpr, total_rm = (uint32_t)(rows * cpr);
  const uint32_t nbk = cpr >> 4;  // (TO) 16-chunk blocks per row group
  const uint32_t total = TO ? (uint32_t)(((rows + 15) >> 4) * 16 * cpr) : total_rm;
  const uint32_t base = blockIdx.x * (uint32_t)(NT * U);
  const bool grouped = (G > 1);
  auto rc_of = [&](uint32_t c, uint32_t& row, uint32_t& cc) __attribute__((always_inline)) {
    if (TO) {
      const uint32_t blk = c >> 8, w = c & 255u, rg = blk / nbk;
      row = rg * 16 + (w >> 4);
      cc = (blk - rg * nbk) * 16 + (w & 15u);
    } else {
      chunk_rc(gr, c, row, cc);
    }
  };

  // Row and column chunk of this thread's U chunks: one division for the
  // first, then steps of NT chunks (a chunk past the end gets a row past the
  // last one, so it stays inactive).
  uint32_t rowu[U], ccu[U];
  rc_of(base + threadIdx.x, rowu[0], ccu[0]);
  if (TO && NT == 256) {
    // tiled order: NT = 256 chunks is one 1 KB block further
    const uint32_t w = threadIdx.x;
    uint32_t rg = rowu[0] >> 4, bk = ccu[0] >> 4;
#pragma unroll
    for (int u = 1; u < U; ++u) {
      if (++bk == nbk) { bk = 0; ++rg; }
      rowu[u] = rg * 16 + (w >> 4);
      ccu[u] = bk * 16 + (w & 15u);
    }
  } else if (!TO) {
    const uint32_t drow = (uint32_t)NT / cpr, dcc = (uint32_t)NT - drow * cpr;
#pragma unroll
    for (int u = 1; u < U; ++u) {
      rowu[u] = rowu[u - 1] + drow;
      ccu[u] = ccu[u - 1] + dcc;
      if (ccu[u] >= cpr) { ccu[u] -= cpr; ++rowu[u]; }
    }
  } else {
#pragma unroll
    for (int u = 1; u < U; ++u) rc_of(base + u * NT + threadIdx.x, rowu[u], ccu[u]);
  }

  // this thread's chunks go out first (a clamped in-range address past the
  // end, so no branch separates the loads)
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t c = base + u * NT + threadIdx.x;
    if (TO) {
      const uint32_t row = rowu[u] < (uint32_t)rows ? rowu[u] : (uint32_t)rows - 1;
      v[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(gr.x + (int64_t)row * gr.ldx + (int64_t)ccu[u] * 8));
    } else {
      v[u] = load_chunk(gr, c < total ? c : total - 1);
    }
  }

  // group of the workgroup's first row; its channel table (built while the
  // chunk loads are in flight)
  uint32_t row_first, cc_first;
  rc_of(base, row_first, cc_first);
  const int gA = grouped ? group_of_row(off, G, row_first) : 0;
  const int64_t gA_end = grouped ? (int64_t)off[gA + 1] : rows;
  const bool use_tab = nS > 0 && cpr <= TAB_MAX;
  if (use_tab) build_chan_table(chan + (int64_t)gA * nS, nS, cpr, tab, NT);

  // tensor scale of the dense paths (one group)
  float tdense = 1.0f;
  bool poison = false;
  if (MODE == AMAX_PARTIALS) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += NT) m = max(m, amax_words[i]);
    tdense = nv_tensor_scale(bf16_to_f32(wg_max<NT>(m, red)));
  } else if (MODE == AMAX_FUSED) {
    // the maximum of this workgroup's own chunks (already loaded), then
    // across the launch
    __shared__ uint32_t s_amax, s_bad;
    const uint32_t gen = threadIdx.x < 64 ? grid_gen(gc) : 0u;
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = base + u * NT + threadIdx.x;
      if (c < total && rowu[u] < (uint32_t)rows) m = max(m, absmax8(v[u]));
    }
    m = wg_max<NT>(m, red);
    if (threadIdx.x < 64) {
      bool expired;
      const uint32_t g = grid_max(m, gridDim.x, gen, gc, expired);
      if (threadIdx.x == 0) {
        s_amax = g;
        s_bad = expired ? 1u : 0u;
      }
    }
    __syncthreads();
    tdense = nv_tensor_scale(bf16_to_f32(s_amax));
    poison = s_bad != 0u;
  }
  if ((MODE == AMAX_PARTIALS || MODE == AMAX_FUSED) && blockIdx.x == 0 && threadIdx.x == 0)
    tscale[0] = poison ? __uint_as_float(0x7FC00000u) : tdense;

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t c = base + u * NT + threadIdx.x;
    uint32_t row = rowu[u], cc = ccu[u];
    const bool active = c < total && row < (uint32_t)rows;
    if (!active) row = cc = 0;
    int g = gA;
    if (grouped && active && row >= gA_end) g = group_of_row(off, G, row);
    float t = tdense;
    if (MODE == AMAX_GROUP_WORDS) {
      t = nv_tensor_scale(__uint_as_float(amax_words[g]));
      if (active && cc == 0 && row == (uint32_t)off[g]) tscale[g] = t;
    }
    uint32_t ent = 0;
    if (nS > 0 && active)
      ent = (use_tab && g == gA) ? tab[cc] : chan_entry_search(chan + (int64_t)g * nS, nS, cc);
    quantize_chunk<FMT>(v[u], active, poison, tiled, row, cc, cols, t, ent, nS, q, scales,
                        resid);
  }
}

// ---- the dense tile quantizer ------------------------------------------------
//
// One group: the large NVFP4 tensors (after the partial-amax pass) and
// MXFP4 at every size.  One lane owns a 32-element unit of one row (64
// bytes of BF16 in, 16 bytes of codes out: two NVFP4 blocks or one MXFP4
// block), so the per-block work (maximum, scale code, divisor) is done once
// per block instead of once per lane holding part of it, and the main path
// moves no data between lanes.  A wave owns a tile of R rows x WC units
// (R WC = 64); with WC = 4 the tile is 16 rows x 128 columns and its 64 code
// pieces are one 1 KB block of the tiled layout, written contiguously
// (lane = piece).  The residual of the selected channels of a tile is
// formed afterwards by lanes indexed by (row, channel): the lane holding a
// channel's unit passes its BF16 value through a small per-wave LDS slot
// (x is not read again) and the block scale codes come from the wave's LDS
// copy, so the cost follows the number of selected entries rather than the
// tile's width.  A workgroup whose tiles' channels fit RES_W columns
// collects its residual rows in LDS and writes them as contiguous runs.
//
// NVFP4 arithmetic, equal to the IEEE single operations the definitions
// name:
//  * amax / 6 is amax * RN(1/6) with one FMA correction; that this equals
//    the correctly rounded quotient was checked exhaustively over every
//    non-negative finite BF16 amax;
//  * (amax / 6) / t and x / d use RN(1/t) and RN(1/d) (a per-workgroup table
//    over the 127 block-scale codes) with two FMA corrections, which is the
//    correctly rounded quotient by Markstein's theorem while t >= 2^-87:
//    then d >= 2^-96 or d = 0, and a dividend too small for the residual
//    to be exact gives a quotient far below the first rounding threshold
//    of its format (code 0 either way).  Below that tensor scale the
//    dividends, divisors and t are multiplied by 2^64 first (exact, and no
//    quotient changes).  The remainder is formed negated, which keeps the
//    sign of a zero quotient.
// MXFP4 converts the BF16 pairs directly (v_cvt_scalef32_pk_fp4_bf16 with
// the power-of-two block scale: x / 2^e is exact, so this is the
// nearest-even E2M1 code of x / 2^e as in the FP32 form; checked on the GPU
// against the FP32 form for every finite BF16 value in both places of a
// pair and every E8M0 scale).
constexpr int TT = 256;           // threads per workgroup
constexpr int TW = TT / 64;       // waves per workgroup
constexpr int TDU = 2;            // tiles per wave
constexpr int TILE_PARTS = 256;   // partial maxima of the NVFP4 amax pass
constexpr uint32_t CTAB_MAX = 1024;  // column tiles covered by the LDS channel table
constexpr int SCHAN_MAX = 1024;      // channels staged in LDS (longer lists are read from memory)
constexpr int RES_W = 128;           // residual entries per row a workgroup collects in LDS

typedef __bf16 bf16x2t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8t __attribute__((ext_vector_type(8)));
typedef float f32x2t __attribute__((ext_vector_type(2)));
typedef float f32x4t __attribute__((ext_vector_type(4)));

struct TileArgs {
  const uint16_t* x;
  int64_t ldx;
  int64_t cols;
  uint32_t rows, upr, nct, ntiles;  // units per row, column tiles, tiles
  const int32_t* chan;
  int nS;
  uint8_t* q;
  uint8_t* scales;
  float* tscale;
  uint16_t* resid;
  const uint32_t* parts;   // one group: NVFP4 partial maxima
  int nparts;
  const int32_t* off;      // groups: row offsets [G + 1]
  int G;
  const uint32_t* gwords;  // groups: NVFP4 amax words (FP32 bits of max |x|), gslots per group
  int gslots;
  uint16_t* score;  // score mode: column maxima of |x - p| per band of row tiles, BF16 bits
  uint32_t nrt;     // score mode: row tiles
};

// NVFP4 tensor scale of group g: the maximum of its amax words.
__device__ __forceinline__ float group_tscale(const TileArgs& p, int g) {
  uint32_t m = 0;
  for (int i = 0; i < p.gslots; ++i) m = max(m, p.gwords[(int64_t)g * p.gslots + i]);
  return nv_tensor_scale(__uint_as_float(m));
}

// E2M1 magnitude of a code's 3 low bits, without a branch: 0.5 m for
// exponent 0, else 2^(e-1) (1 + m/2).
__device__ __forceinline__ float e2m1_mag_bf(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float nrm = __uint_as_float((126u + e) << 23 | (m << 22));
  return e ? nrm : (m ? 0.5f : 0.0f);
}


// RN(a / 6) for a non-negative BF16 value a (exhaustively checked).
__device__ __forceinline__ float div6_rn(float a) {
  constexpr float c6 = 0x1.555556p-3f;  // RN(1/6)
  const float q = a * c6;
  return __builtin_fmaf(__builtin_fmaf(-q, 6.0f, a), c6, q);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
  for (int s = 32; s > 0; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s));
  return m;
}

// First j with S[j] >= v (S ascending, nS entries).
__device__ __forceinline__ int chan_lower_bound(const int32_t* __restrict__ S, int nS, int64_t v) {
  int lo = 0, hi = nS;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)S[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Largest BF16 magnitude pattern of 16 packed elements (packed u16 maxima).
__device__ __forceinline__ uint32_t absmax16_bits(u32x4 a, u32x4 b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, a.x & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 8; ++i)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, (i < 4 ? a[i] : b[i - 4]) & 0x7FFF7FFFu));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// Largest BF16 magnitude pattern of 32 packed elements (packed u16 maxima).
__device__ __forceinline__ uint32_t absmax32_bits(const u32x4 (&w)[4]) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, w[0].x & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 16; ++i)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i >> 2][i & 3] & 0x7FFF7FFFu));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// Codes and the two block scale codes (low byte first) of one NVFP4 unit:
// both blocks' scale codes and divisors first, from the packed maxima, then
// each block unpacked, divided and packed (few values live at once).
// TABLE: {d, RN(1/d)} of the block-scale codes come from the workgroup's
// table; else RN(1/d) is one IEEE division per block (per-group tensor
// scales).  sx: 2^64 when the tensor scale is below 2^-87, else 1.
// Dividends and divisors are multiplied by sx, which is exact for them
// (then all far below 1) and leaves every quotient unchanged while it
// brings the operands into the range where the reciprocal-and-FMA
// division is correctly rounded; d itself is RN(sb t) unscaled, as defined.
// ts = t sx and yts = RN(1/ts); the table holds {d sx, RN(1/(d sx))}.
// PS: sx may differ from 1 (a wave-uniform choice; with PS false sx is 1
// and the products by it are left out).
template <bool TABLE, bool PS>
__device__ __forceinline__ void nv_unit(const u32x4 (&w)[4], float t, float sx, float ts,
                                        float yts, const float2* dytab, u32x4& codes,
                                        uint32_t& scw) {
  if (!PS) sx = 1.0f;
  float dr[2], yr[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float v6 = div6_rn(bf16_to_f32(absmax16_bits(w[2 * b], w[2 * b + 1])));
    const uint32_t sc = e4m3_encode(quot_rn(PS ? v6 * sx : v6, ts, yts));
    scw = b == 0 ? sc : (scw | sc << 8);
    if (TABLE) {
      const float2 dy = dytab[sc];
      dr[b] = dy.x;
      yr[b] = dy.y;
    } else {
      dr[b] = PS ? e4m3_value(sc) * t * sx : e4m3_value(sc) * t;
      yr[b] = dr[b] > 0.0f ? 1.0f / dr[b] : 0.0f;
    }
  }
  uint32_t cw[4];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float d = dr[b], y = yr[b];
    auto qt = [&](uint32_t bits) __attribute__((always_inline)) {
      return quot_rn(PS ? __uint_as_float(bits) * sx : __uint_as_float(bits), d, y);
    };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 u = w[2 * b + h];
      uint32_t pk = 0;
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, qt(u.x << 16), qt(u.x & 0xFFFF0000u), 1.0f, 0);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, qt(u.y << 16), qt(u.y & 0xFFFF0000u), 1.0f, 1);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, qt(u.z << 16), qt(u.z & 0xFFFF0000u), 1.0f, 2);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, qt(u.w << 16), qt(u.w & 0xFFFF0000u), 1.0f, 3);
      cw[2 * b + h] = pk;
    }
  }
  codes = u32x4{cw[0], cw[1], cw[2], cw[3]};
}

// The operand scale of the division for tensor scale t (see nv_unit).
__device__ __forceinline__ float div_prescale(float t) { return t >= 0x1p-87f ? 1.0f : 0x1p64f; }

constexpr int RG_MAX = TDU * TW * 64;  // rows the tiles of one workgroup cover at most
constexpr int SOFF_MAX = 2048;         // group offsets staged in LDS (G + 1 at most)
constexpr int GT_MAX = 4;              // groups of a workgroup with their divisor tables in LDS

// rgrp[i] = group of row rbase + i, for the rows of this workgroup's tiles:
// the offsets are staged in LDS (soff, when G < SOFF_MAX) and searched
// there, one row per thread.  Contains a barrier; returns rbase.
template <int R, int DU>
__device__ __forceinline__ uint32_t build_row_groups(const TileArgs& p, int32_t* rgrp,
                                                     int32_t* soff, uint32_t* nrows = nullptr) {
  const uint32_t T0 = blockIdx.x * DU * TW;
  const uint32_t T1 = (T0 + DU * TW < p.ntiles ? T0 + DU * TW : p.ntiles) - 1;
  const uint32_t rbase = (T0 / p.nct) * R;
  const uint32_t rlim0 = (T1 / p.nct + 1) * R, rlim = rlim0 < p.rows ? rlim0 : p.rows;
  const int G = p.G;
  if (G < SOFF_MAX) {
    for (int i = threadIdx.x; i <= G; i += TT) soff[i] = p.off[i];
    __syncthreads();
    for (uint32_t i = threadIdx.x; rbase + i < rlim; i += TT) {
      const int64_t row = rbase + i;
      int lo = 0, hi = G - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)soff[mid] <= row) lo = mid; else hi = mid - 1;
      }
      rgrp[i] = lo;
    }
  } else {
    for (uint32_t i = threadIdx.x; rbase + i < rlim; i += TT)
      rgrp[i] = group_of_row(p.off, G, rbase + i);
  }
  __syncthreads();
  if (nrows) *nrows = rlim - rbase;
  return rbase;
}

// Dword d (wave-uniform) of a lane's 64-byte unit.
__device__ __forceinline__ uint32_t unit_dword(const u32x4 (&w)[4], uint32_t d) {
  switch (d) {
    case 0: return w[0].x;  case 1: return w[0].y;  case 2: return w[0].z;  case 3: return w[0].w;
    case 4: return w[1].x;  case 5: return w[1].y;  case 6: return w[1].z;  case 7: return w[1].w;
    case 8: return w[2].x;  case 9: return w[2].y;  case 10: return w[2].z; case 11: return w[2].w;
    case 12: return w[3].x; case 13: return w[3].y; case 14: return w[3].z; default: return w[3].w;
  }
}

// Entries of an ascending channel list S below c0 and below c1: by ballot
// over one load per lane when nS <= 64 (sl: this lane's entry, or INT_MAX),
// else by binary search.  Wave-uniform results.
__device__ __forceinline__ void chan_range(const int32_t* __restrict__ S, int nS, int64_t c0,
                                           int64_t c1, int& jl, int& jh, int32_t& sl) {
  const int lane = threadIdx.x & 63;
  if (nS <= 64) {
    sl = lane < nS ? S[lane] : 0x7FFFFFFF;
    jl = __popcll(__ballot((int64_t)sl < c0));
    jh = __popcll(__ballot((int64_t)sl < c1));
  } else {
    sl = 0x7FFFFFFF;
    jl = chan_lower_bound(S, nS, c0);
    jh = chan_lower_bound(S, nS, c1);
  }
  jl = __builtin_amdgcn_readfirstlane(jl);
  jh = __builtin_amdgcn_readfirstlane(jh);
}

// Tiles of R rows x WC units.  GRP: the rows belong to groups (expert
// ranges off[g] <= row < off[g+1]) with their own NVFP4 tensor scale (from
// the group amax words) and channel list (chan + g nS); a tile that spans
// groups takes each lane's group by search and forms the residual group by
// group.  SL: the one channel list (nS <= SCHAN_MAX) is staged in LDS.
// SCORE (one group, no channels yet): the scores of online channel
// selection come out of the same pass over x, so that x is read once: a
// workgroup takes one column tile and a band of DU TW row tiles, and writes
// for each of its columns the largest |x - p| over the band's rows (p the
// dequantized code, formed as the selection's residual forms it), rounded
// once to BF16 (nearest-even rounding is monotone, so this is the largest
// rounded residual).
template <int FMT, bool TILED, int WC, int DU, bool SL, bool GRP, bool SCORE = false>
__global__ void __launch_bounds__(TT) k_quant_tile(TileArgs p) {
  constexpr int R = 64 / WC;
  constexpr int SPU = (FMT == FP4Q_NVFP4) ? 2 : 1;  // scale blocks per unit
  constexpr int SCW = 8 * WC + 4;                   // score mode: a row of a piece in LDS (padded)
  static_assert(!TILED || WC == 4, "the tiled layout's code block is 16 rows x 128 columns");
  static_assert(!(SL && GRP), "one staged channel list");
  static_assert(!(SCORE && (GRP || SL)), "scores: one group, no channel list");
  __shared__ uint32_t ctab[GRP || SCORE ? 1 : CTAB_MAX];
  __shared__ int32_t schan[SL ? SCHAN_MAX : 1];
  __shared__ float2 dytab[GRP ? 1 : 128];
  __shared__ uint8_t scx[TW][64 * SPU];
  __shared__ int32_t rgrp[GRP ? RG_MAX : 1];
  __shared__ int32_t soff[GRP ? SOFF_MAX : 1];
  __shared__ uint16_t sres[SCORE ? 1 : 16][SCORE ? 1 : RES_W];  // the workgroup's residual rows (see agg)
  __shared__ uint16_t xres[TW][64 / R][R];  // a residual pass's x values, per wave
  __shared__ __attribute__((aligned(16))) float ssc[SCORE ? TW : 1][SCORE ? R : 1][SCORE ? SCW : 1];  // a piece's x - p, per wave
  __shared__ float swc[SCORE ? TW : 1][SCORE ? 32 * WC : 1];             // the waves' column maxima
  // grouped NVFP4: the tensor scales {t, sx, t sx, RN(1/(t sx))} and divisor
  // tables {d sx, RN(1/(d sx))} of the workgroup's groups, when it spans at
  // most GT_MAX of them (the usual case: its tiles cover 16 or 32 rows)
  constexpr bool GTAB = GRP && FMT == FP4Q_NVFP4;
  __shared__ float4 gts[GTAB ? GT_MAX : 1];
  __shared__ float2 gdy[GTAB ? GT_MAX : 1][GTAB ? 128 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane % R, c = lane / R;
  const uint32_t nct = p.nct;
  const int nS = p.nS;

  // this wave's tiles and their loads, before anything else
  u32x4 v[DU][4];
  uint32_t tile[DU];
  // score mode: column tile bct and row tiles band DU TW .. of it; a tile
  // past the last row tile is marked ntiles (none)
  const uint32_t bct = SCORE ? blockIdx.x % nct : 0u, band = SCORE ? blockIdx.x / nct : 0u;
#pragma unroll
  for (int k = 0; k < DU; ++k) {
    if (SCORE) {
      const uint32_t rt = band * (DU * TW) + k * TW + wave;
      tile[k] = rt < p.nrt ? rt * nct + bct : p.ntiles;
    } else {
      tile[k] = (blockIdx.x * DU + k) * TW + wave;
    }
    const uint32_t T = tile[k] < p.ntiles ? tile[k] : p.ntiles - 1;
    const uint32_t rt = T / nct, ct = T - rt * nct;
    uint32_t row = rt * R + r, uc = ct * WC + c;
    row = row < p.rows ? row : p.rows - 1;
    uc = uc < p.upr ? uc : p.upr - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(p.x + (int64_t)row * p.ldx + (int64_t)uc * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[k][i] = src[i];  // plain loads: the amax pass left x in the caches
  }

  // one group: NVFP4 tensor scale from the partial maxima (every wave), the
  // divisor table {d, RN(1/d)} of the block-scale codes, the channel table
  // ctab[ct] = first j with S[j] >= 32 WC ct (ct <= nct) and the staged list
  float t = 1.0f, sx = 1.0f, ts = 1.0f, yts = 1.0f;
  bool use_ctab = false;
  if constexpr (!GRP) {
    if (FMT == FP4Q_NVFP4) {
      uint32_t m = 0;
      for (int i = lane; i < p.nparts; i += 64) m = max(m, p.parts[i]);
      t = nv_tensor_scale(bf16_to_f32(wave_max_u32(m)));
      sx = div_prescale(t);
      ts = t * sx;
      yts = 1.0f / ts;
      if (threadIdx.x < 128) {
        const float d = e4m3_value(threadIdx.x) * t * sx;
        dytab[threadIdx.x] = float2{d, d > 0.0f ? 1.0f / d : 0.0f};
      }
      if (blockIdx.x == 0 && threadIdx.x == 0) p.tscale[0] = t;
    }
    use_ctab = nS > 0 && nct + 1 <= CTAB_MAX;
    if (nS > 0) {
      constexpr uint32_t W = 32 * WC;
      for (int j = threadIdx.x; j <= nS; j += TT) {
        const int32_t sj = j < nS ? p.chan[j] : 0;
        if (SL && j < nS) schan[j] = sj;
        if (use_ctab) {
          const uint32_t lo = j == 0 ? 0u : (uint32_t)p.chan[j - 1] / W + 1u;
          const uint32_t hi = j == nS ? nct : (uint32_t)sj / W;
          for (uint32_t ct = lo; ct <= hi; ++ct) ctab[ct] = (uint32_t)j;
        }
      }
    }
    __syncthreads();
  }
  uint32_t rbase = 0;
  int gA = 0;
  bool use_gt = false;
  if constexpr (GRP) {
    uint32_t nrow = 0;
    rbase = build_row_groups<R, DU>(p, rgrp, soff, &nrow);
    if (GTAB && nrow > 0) {
      gA = rgrp[0];
      const int ng = rgrp[nrow - 1] - gA + 1;
      use_gt = ng <= GT_MAX;  // uniform
      if (use_gt) {
        if ((int)threadIdx.x < ng) {
          const float tg = group_tscale(p, gA + (int)threadIdx.x);
          const float sg = div_prescale(tg);
          gts[threadIdx.x] = float4{tg, sg, tg * sg, 1.0f / (tg * sg)};
        }
        __syncthreads();
        for (int i = threadIdx.x; i < ng * 128; i += TT) {
          const float4 T = gts[i >> 7];
          const float d = e4m3_value((uint32_t)(i & 127)) * T.x * T.y;
          gdy[i >> 7][i & 127] = float2{d, d > 0.0f ? 1.0f / d : 0.0f};
        }
        __syncthreads();
      }
    }
  }
  // entry j of the channel list of group g
  auto chan_at = [&](int g, int j) __attribute__((always_inline)) -> int64_t {
    if (SL) return (int64_t)schan[j];
    return (int64_t)p.chan[(GRP ? (int64_t)g * nS : 0) + j];
  };

  // agg: the workgroup's residual entries are collected in LDS and written
  // row by row in contiguous runs at the end (scattered 2-byte stores fetch
  // their lines), when its tiles share one 16-row band and one group and
  // cover at most RES_W channels of it: rows wr0 .. wr0+15, entries
  // wjl .. wjl+wn-1 of the group's list
  bool agg = false;
  uint32_t wr0 = 0;
  int wjl = 0, wn = 0;
  if (R == 16 && nS > 0) {
    const uint32_t T0 = blockIdx.x * DU * TW;
    const uint32_t T1 = (T0 + DU * TW < p.ntiles ? T0 + DU * TW : p.ntiles) - 1;
    const uint32_t rt = T0 / nct;
    if (T1 / nct == rt) {
      wr0 = rt * R;
      const uint32_t wrl = (wr0 + R < p.rows ? wr0 + R : p.rows) - 1;
      const int g = GRP ? rgrp[wr0 - rbase] : 0;
      if (!GRP || rgrp[wrl - rbase] == g) {
        const int64_t C0 = (int64_t)(T0 - rt * nct) * (32 * WC);
        const int64_t C1 = (int64_t)(T1 - rt * nct + 1) * (32 * WC);
        int jl, jh;
        if (!GRP && use_ctab) {
          jl = (int)ctab[T0 - rt * nct];
          jh = (int)ctab[T1 - rt * nct + 1];
        } else {
          const int32_t* S = p.chan + (GRP ? (int64_t)g * nS : 0);
          jl = chan_lower_bound(S, nS, C0);
          jh = chan_lower_bound(S, nS, C1);
        }
        jl = __builtin_amdgcn_readfirstlane(jl);
        jh = __builtin_amdgcn_readfirstlane(jh);
        agg = jh - jl <= RES_W;
        wjl = jl;
        wn = jh - jl;
      }
    }
  }

  // each tile's groups, and the channel range of its first group
  int g0[DU], g1[DU], jlo[DU], nres[DU];
#pragma unroll
  for (int k = 0; k < DU; ++k) {
    g0[k] = g1[k] = jlo[k] = nres[k] = 0;
    if (tile[k] >= p.ntiles) continue;
    const uint32_t rt = tile[k] / nct, ct = tile[k] - rt * nct;
    const uint32_t r0 = rt * R, rlast = (r0 + R < p.rows ? r0 + R : p.rows) - 1;
    if (GRP) {
      g0[k] = __builtin_amdgcn_readfirstlane(rgrp[r0 - rbase]);
      g1[k] = __builtin_amdgcn_readfirstlane(rgrp[rlast - rbase]);
    }
    if (nS == 0) continue;
    const int64_t c0 = (int64_t)ct * (32 * WC);
    int jl, jh;
    int32_t sl = 0x7FFFFFFF;
    if (!GRP && use_ctab) {
      jl = __builtin_amdgcn_readfirstlane((int)ctab[ct]);
      jh = __builtin_amdgcn_readfirstlane((int)ctab[ct + 1]);
    } else {
      chan_range(p.chan + (GRP ? (int64_t)g0[k] * nS : 0), nS, c0, c0 + 32 * WC, jl, jh, sl);
    }
    jlo[k] = jl;
    nres[k] = (jh - jl) * R;
  }

  // score mode: lane l reduces column l % (8 WC) of each 8-column piece over
  // eight rows (row group l / (8 WC)); cm[i] keeps piece i's maximum
  float cm[4] = {0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int k = 0; k < DU; ++k) {
    if (tile[k] >= p.ntiles) break;
    const uint32_t rt = tile[k] / nct, ct = tile[k] - rt * nct;
    const uint32_t r0 = rt * R;
    const uint32_t row = r0 + r, uc = ct * WC + c;
    const bool active = row < p.rows && uc < p.upr;
    // this lane's group and its NVFP4 tensor scale
    float tk = t, sxk = sx, tsk = ts, ytsk = yts;
    const float2* dyk = dytab;
    if (GTAB) {
      const int g = g0[k] == g1[k] ? g0[k] : rgrp[(row < p.rows ? row : p.rows - 1) - rbase];
      if (use_gt) {
        const float4 T = gts[g - gA];
        tk = T.x;
        sxk = T.y;
        tsk = T.z;
        ytsk = T.w;
        dyk = gdy[g - gA];
      } else {
        tk = group_tscale(p, g);
        sxk = div_prescale(tk);
        tsk = tk * sxk;
        ytsk = 1.0f / tsk;
      }
      if (active && uc == 0 && row == (uint32_t)p.off[g]) p.tscale[g] = tk;
    }
    u32x4 codes;
    uint32_t scw;  // this unit's block scale codes (NVFP4: two bytes, low first)
    if (FMT == FP4Q_NVFP4) {
      const bool ps = __builtin_amdgcn_ballot_w64(sxk != 1.0f) != 0;
      if (!GRP || use_gt) {
        if (ps) nv_unit<true, true>(v[k], tk, sxk, tsk, ytsk, dyk, codes, scw);
        else nv_unit<true, false>(v[k], tk, sxk, tsk, ytsk, dyk, codes, scw);
      } else {
        if (ps) nv_unit<false, true>(v[k], tk, sxk, tsk, ytsk, dyk, codes, scw);
        else nv_unit<false, false>(v[k], tk, sxk, tsk, ytsk, dyk, codes, scw);
      }
    } else {
      const int e = mx_exponent(bf16_to_f32(absmax32_bits(v[k])));
      scw = (uint32_t)(e + 127);
      const float s = __uint_as_float(scw << 23);
      // the pairs taken from a bf16x8 view of each 16-byte piece (a bit cast
      // of one 32-bit element of the u32x4 to a BF16 pair is folded wrongly
      // by this compiler: it reads element 0 for all four)
      uint32_t cw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8t w = __builtin_bit_cast(bf16x8t, v[k][i]);
        uint32_t pk = 0;
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, bf16x2t{w[0], w[1]}, s, 0);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, bf16x2t{w[2], w[3]}, s, 1);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, bf16x2t{w[4], w[5]}, s, 2);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, bf16x2t{w[6], w[7]}, s, 3);
        cw[i] = pk;
      }
      codes = u32x4{cw[0], cw[1], cw[2], cw[3]};
    }
    if (active) {
      const int64_t K = p.cols;
      int64_t co, so;
      if (TILED) {
        co = ((((int64_t)(row >> 4) * (K >> 7) + (uc >> 2)) << 10) + (int64_t)(lane << 4));
        const int64_t sb = ((int64_t)(row >> 6) * (K >> 7) + (uc >> 2)) * (SPU * 256);
        so = (FMT == FP4Q_NVFP4) ? sb + (((((uc & 3) >> 1) << 6) + (row & 63)) << 2) + 2 * (uc & 1)
                                 : sb + ((row & 63) << 2) + (uc & 3);
      } else {
        co = (int64_t)row * (K >> 1) + (int64_t)uc * 16;
        so = (int64_t)row * (K / (16 * (3 - SPU))) + (int64_t)uc * SPU;
      }
      __builtin_nontemporal_store(codes, reinterpret_cast<u32x4*>(p.q + co));
      if (FMT == FP4Q_NVFP4)
        *reinterpret_cast<uint16_t*>(p.scales + so) = (uint16_t)scw;
      else
        p.scales[so] = (uint8_t)scw;
    }

    if (SCORE) {
      // |x - p| of the unit's elements, one 8-element piece at a time, and
      // its maximum over the tile's rows (rows past the end repeat the
      // last row, units past the end a real unit whose columns are not
      // stored; neither changes a stored maximum)
      float sv[SPU];
#pragma unroll
      for (int b = 0; b < SPU; ++b)
        sv[b] = FMT == FP4Q_NVFP4 ? e4m3_value((scw >> (8 * b)) & 0xFFu) : exp2i((int)scw - 127);
      const int cc = lane % (8 * WC), rg = lane / (8 * WC);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = sv[FMT == FP4Q_NVFP4 ? (i >> 1) : 0];
        const uint32_t cw = codes[i];
        const u32x4 w = v[k][i];
        const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
        // signed E2M1 values (exact; code 8 gives a zero of either sign,
        // which |x - p| does not see)
        const f32x2t ev[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0),
                              __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1),
                              __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2),
                              __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3)};
        float dv[8];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const f32x2t e = ev[h];
          const float p0 = FMT == FP4Q_NVFP4 ? (e.x * s) * tk : e.x * s;
          const float p1 = FMT == FP4Q_NVFP4 ? (e.y * s) * tk : e.y * s;
          dv[2 * h] = __uint_as_float(wd[h] << 16) - p0;
          dv[2 * h + 1] = __uint_as_float(wd[h] & 0xFFFF0000u) - p1;
        }
        *reinterpret_cast<f32x4t*>(&ssc[wave][r][8 * c]) = f32x4t{dv[0], dv[1], dv[2], dv[3]};
        *reinterpret_cast<f32x4t*>(&ssc[wave][r][8 * c + 4]) = f32x4t{dv[4], dv[5], dv[6], dv[7]};
        __builtin_amdgcn_wave_barrier();
        float m = cm[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(ssc[wave][8 * rg + j][cc]));
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int o = 8 * WC; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        cm[i] = m;
      }
    }

    // residual of the selected channels in this tile's columns, group by
    // group: lane i of a pass takes row i % R and channel jlo + i / R
    if (!SCORE && nS > 0) {
      if (SPU == 2)
        *reinterpret_cast<uint16_t*>(&scx[wave][2 * lane]) = (uint16_t)scw;
      else
        scx[wave][lane] = (uint8_t)scw;
      const int64_t c0 = (int64_t)ct * (32 * WC);
      for (int g = g0[k]; g <= g1[k]; ++g) {
        const bool first = g == g0[k];
        int jl = jlo[k], n = nres[k];  // (first group: found before the loop)
        uint32_t rlo = r0, rhi = p.rows;
        float tg = t;
        if (GRP) {
          rlo = max(r0, (uint32_t)p.off[g]);
          rhi = min(rhi, (uint32_t)p.off[g + 1]);
          if (!first) {
            int jh;
            int32_t sl;
            chan_range(p.chan + (int64_t)g * nS, nS, c0, c0 + 32 * WC, jl, jh, sl);
            n = (jh - jl) * R;
          }
          if (FMT == FP4Q_NVFP4) tg = use_gt ? gts[g - gA].x : group_tscale(p, g);
        }
        const float sxg = div_prescale(tg);
        for (int i0 = 0; i0 < n; i0 += 64) {
          // the pass's x values come from the registers of the lanes that
          // own them: channel q of the pass (column col, the same for the
          // wave) sits in the lanes of unit (col - c0) / 32, at one dword
          // index; they put it in the wave's LDS slot for the item lanes
#pragma unroll
          for (int q = 0; q < 64 / R; ++q) {
            if (i0 + q * R >= n) break;
            const uint32_t cq = (uint32_t)__builtin_amdgcn_readfirstlane(
                                    (int)(chan_at(g, jl + i0 / R + q) - c0));
            const uint32_t wd = unit_dword(v[k], (cq & 31u) >> 1);
            if ((uint32_t)c == (cq >> 5)) xres[wave][q][r] = (uint16_t)((cq & 1u) ? (wd >> 16) : wd);
          }
          const int i = i0 + lane;
          const uint32_t rr = (uint32_t)i % R, jj = (uint32_t)i / R;
          const uint32_t rw = r0 + rr;
          if (i < n && rw >= rlo && rw < rhi) {
            const int j = jl + (int)jj;
            const int64_t col = chan_at(g, j);
            const uint32_t cl = (uint32_t)(col - c0);
            const uint32_t h = xres[wave][lane / R][rr];
            const float xv = bf16_to_f32(h);
            const uint32_t sc = scx[wave][((cl >> 5) * R + rr) * SPU + (SPU == 2 ? ((cl >> 4) & 1) : 0)];
            float deq;
            if (FMT == FP4Q_NVFP4) {
              const float sb = e4m3_value(sc);
              float d, y;
              if (!GRP || use_gt) {
                const float2 dy = GRP ? gdy[g - gA][sc] : dytab[sc];
                d = dy.x;
                y = dy.y;
              } else {
                d = sb * tg * sxg;
                y = d > 0.0f ? 1.0f / d : 0.0f;
              }
              const float qv = quot_rn(xv * sxg, d, y);
              const uint32_t code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, qv, 0.0f, 1.0f, 0) & 15u;
              deq = (e2m1_mag_bf(code) * sb) * tg;
              if (code & 8u) deq = -deq;
            } else {
              const uint32_t code = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                                        0u, __builtin_bit_cast(bf16x2t, h), __uint_as_float(sc << 23), 0) & 15u;
              deq = e2m1_mag_bf(code) * exp2i((int)sc - 127);
              if (code & 8u) deq = -deq;
            }
            const uint16_t rv = (uint16_t)f32_to_bf16_rne(xv - deq);
            if (agg) sres[rw - wr0][j - wjl] = rv;
            else p.resid[(int64_t)rw * nS + j] = rv;
          }
        }
      }
    }
  }
  if (SCORE) {
    // the waves meet in LDS: lane l < 8 WC holds column (l / 8) 32 + 8 i + l % 8
    // of the tile for piece i
    if (lane < 8 * WC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) swc[wave][(lane >> 3) * 32 + 8 * i + (lane & 7)] = cm[i];
    }
    __syncthreads();
    if (threadIdx.x < 32 * WC) {
      float m = 0.0f;
#pragma unroll
      for (int w = 0; w < TW; ++w) m = fmaxf(m, swc[w][threadIdx.x]);
      const int64_t col = (int64_t)bct * (32 * WC) + threadIdx.x;
      if (col < p.cols) p.score[(int64_t)band * p.cols + col] = (uint16_t)f32_to_bf16_rne(m);
    }
  }
  if (agg) {  // uniform over the workgroup
    __syncthreads();
    const int n = 16 * wn;
    for (int i = threadIdx.x; i < n; i += TT) {
      const int rr = i / wn, jj = i - rr * wn;
      const uint32_t rw = wr0 + (uint32_t)rr;
      if (rw < p.rows) p.resid[(int64_t)rw * nS + wjl + jj] = sres[rr][jj];
    }
  }
}

// Per-group amax over the tile quantizer's tiles: each lane's unit maximum
// (packed BF16 magnitudes), then each row's (its WC lanes), then each
// tile's.  A workgroup combines its single-group tiles in LDS and issues
// one atomic maximum per run of equal groups; a tile that spans groups
// issues one per group.  Atomics on one word are serialised, so each group
// has p.gslots words (as many as the workspace's amax area allows, at most
// 8) and a workgroup takes word blockIdx % gslots; the group's maximum is
// the maximum of its words.  The words hold FP32 bit patterns of max |x|
// (exact and order-free for non-negative values) and are cleared first.
template <int WC, int DU>
__global__ void __launch_bounds__(TT) k_group_amax_tile(TileArgs p, uint32_t* __restrict__ words) {
  constexpr int R = 64 / WC;
  __shared__ int32_t rgrp[RG_MAX];
  __shared__ int32_t soff[SOFF_MAX];
  __shared__ int32_t sg[TW * DU];   // a tile's group, or -1 (none or several)
  __shared__ uint32_t sm[TW * DU];  // its maximum
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane % R, c = lane / R;
  const uint32_t nct = p.nct;
  u32x4 v[DU][4];
  uint32_t tile[DU];
#pragma unroll
  for (int k = 0; k < DU; ++k) {
    tile[k] = (blockIdx.x * DU + k) * TW + wave;
    const uint32_t T = tile[k] < p.ntiles ? tile[k] : p.ntiles - 1;
    const uint32_t rt = T / nct, ct = T - rt * nct;
    uint32_t row = rt * R + r, uc = ct * WC + c;
    row = row < p.rows ? row : p.rows - 1;
    uc = uc < p.upr ? uc : p.upr - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(p.x + (int64_t)row * p.ldx + (int64_t)uc * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[k][i] = src[i];
  }
  const uint32_t rbase = build_row_groups<R, DU>(p, rgrp, soff);
  const int S = p.gslots, slot_w = (int)(blockIdx.x % (uint32_t)S);
#pragma unroll
  for (int k = 0; k < DU; ++k) {
    const int slot = k * TW + wave;  // tile order
    if (tile[k] >= p.ntiles) {
      if (lane == 0) sg[slot] = -1;
      continue;
    }
    const uint32_t rt = tile[k] / nct, ct = tile[k] - rt * nct;
    const uint32_t r0 = rt * R, rlast = (r0 + R < p.rows ? r0 + R : p.rows) - 1;
    const uint32_t row = r0 + r, uc = ct * WC + c;
    uint32_t m = (row < p.rows && uc < p.upr) ? absmax32_bits(v[k]) : 0u;
    if (WC >= 2) m = max(m, (uint32_t)__shfl_xor((int)m, R * (WC / 2)));
    if (WC == 4) m = max(m, (uint32_t)__shfl_xor((int)m, R));
    const int g0 = __builtin_amdgcn_readfirstlane(rgrp[r0 - rbase]);
    const int g1 = __builtin_amdgcn_readfirstlane(rgrp[rlast - rbase]);
    if (g0 == g1) {
      m = wave_max_u32(m);
      if (lane == 0) {
        sg[slot] = g0;
        sm[slot] = m;
      }
    } else {
      if (lane == 0) sg[slot] = -1;
      const int gl = rgrp[(row < p.rows ? row : p.rows - 1) - rbase];
      for (int g = g0; g <= g1; ++g) {
        const uint32_t mg = wave_max_u32(gl == g ? m : 0u);
        if (lane == 0 && mg) atomicMax(&words[g * S + slot_w], mg << 16);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int gc = -1;
    uint32_t mc = 0;
    for (int i = 0; i < TW * DU; ++i) {
      if (sg[i] == gc && gc >= 0) {
        mc = max(mc, sm[i]);
        continue;
      }
      if (gc >= 0 && mc) atomicMax(&words[gc * S + slot_w], mc << 16);
      gc = sg[i];
      mc = gc >= 0 ? sm[i] : 0u;
    }
    if (gc >= 0 && mc) atomicMax(&words[gc * S + slot_w], mc << 16);
  }
}

template <int FMT, bool TILED, int WC, bool GRP>
static void launch_tile_wc(const TileArgs& a, hipStream_t stream) {
  const uint32_t per = TDU * TW;
  const dim3 grid((a.ntiles + per - 1) / per);
  if (!GRP && a.nS <= SCHAN_MAX)
    hipLaunchKernelGGL((k_quant_tile<FMT, TILED, WC, TDU, !GRP, GRP>), grid, dim3(TT), 0, stream, a);
  else
    hipLaunchKernelGGL((k_quant_tile<FMT, TILED, WC, TDU, false, GRP>), grid, dim3(TT), 0, stream, a);
}

template <int FMT, bool GRP>
static void launch_tile_g(bool tiled, const TileArgs& a, int wc, hipStream_t stream) {
  if (tiled) launch_tile_wc<FMT, true, 4, GRP>(a, stream);
  else if (wc == 4) launch_tile_wc<FMT, false, 4, GRP>(a, stream);
  else if (wc == 2) launch_tile_wc<FMT, false, 2, GRP>(a, stream);
  else launch_tile_wc<FMT, false, 1, GRP>(a, stream);
}

// The tile quantizer over x [rows, cols]; one group (parts: the NVFP4
// partial maxima) or G groups (off, and gwords: the NVFP4 group amax words).
template <int FMT>
static void launch_tile(bool tiled, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                        const int32_t* off, int G, const int32_t* chan, int nS, uint8_t* q,
                        uint8_t* scales, float* tscale, uint16_t* resid, const uint32_t* parts,
                        int nparts, const uint32_t* gwords, hipStream_t stream,
                        uint32_t* amax_words = nullptr, int gslots = 1) {
  TileArgs a{};
  a.gslots = gslots;
  a.x = x; a.ldx = ldx; a.cols = cols;
  a.rows = (uint32_t)rows;
  a.upr = (uint32_t)(cols / 32);
  a.off = off; a.G = G; a.gwords = gwords;
  a.chan = chan; a.nS = nS; a.q = q; a.scales = scales; a.tscale = tscale; a.resid = resid;
  a.parts = parts; a.nparts = nparts;
  const int wc = tiled || a.upr >= 3 ? 4 : (int)a.upr;  // 1, 2 or 4 units across a tile
  const uint32_t R = 64u / (uint32_t)wc;
  a.nct = (a.upr + wc - 1) / wc;
  a.ntiles = (uint32_t)((rows + R - 1) / R) * a.nct;
  if (amax_words != nullptr) {  // the groups' amax pass over the same tiles first
    const dim3 grid((a.ntiles + TDU * TW - 1) / (TDU * TW));
    if (wc == 4) hipLaunchKernelGGL((k_group_amax_tile<4, TDU>), grid, dim3(TT), 0, stream, a, amax_words);
    else if (wc == 2) hipLaunchKernelGGL((k_group_amax_tile<2, TDU>), grid, dim3(TT), 0, stream, a, amax_words);
    else hipLaunchKernelGGL((k_group_amax_tile<1, TDU>), grid, dim3(TT), 0, stream, a, amax_words);
  }
  if (off != nullptr && G > 1) launch_tile_g<FMT, true>(tiled, a, wc, stream);
  else launch_tile_g<FMT, false>(tiled, a, wc, stream);
}

// Score mode of the tile quantizer (one group, no channels): codes, scales
// and tensor scale as launch_tile, plus score [bands, cols] (BF16 bits),
// bands = ceil(row tiles / (TDU TW)); returns bands.
template <int FMT>
static int64_t launch_tile_score(bool tiled, const uint16_t* x, int64_t rows, int64_t cols,
                                 int64_t ldx, uint8_t* q, uint8_t* scales, float* tscale,
                                 const uint32_t* parts, int nparts, uint16_t* score,
                                 hipStream_t stream) {
  TileArgs a{};
  a.gslots = 1;
  a.x = x; a.ldx = ldx; a.cols = cols;
  a.rows = (uint32_t)rows;
  a.upr = (uint32_t)(cols / 32);
  a.G = 1;
  a.q = q; a.scales = scales; a.tscale = tscale;
  a.parts = parts; a.nparts = nparts;
  a.score = score;
  const int wc = tiled || a.upr >= 3 ? 4 : (int)a.upr;
  const uint32_t R = 64u / (uint32_t)wc;
  a.nct = (a.upr + wc - 1) / wc;
  a.nrt = (uint32_t)((rows + R - 1) / R);
  a.ntiles = a.nrt * a.nct;
  const int64_t bands = ((int64_t)a.nrt + TDU * TW - 1) / (TDU * TW);
  const dim3 grid((unsigned)(bands * a.nct));
  if (tiled)
    hipLaunchKernelGGL((k_quant_tile<FMT, true, 4, TDU, false, false, true>), grid, dim3(TT), 0, stream, a);
  else if (wc == 4)
    hipLaunchKernelGGL((k_quant_tile<FMT, false, 4, TDU, false, false, true>), grid, dim3(TT), 0, stream, a);
  else if (wc == 2)
    hipLaunchKernelGGL((k_quant_tile<FMT, false, 2, TDU, false, false, true>), grid, dim3(TT), 0, stream, a);
  else
    hipLaunchKernelGGL((k_quant_tile<FMT, false, 1, TDU, false, false, true>), grid, dim3(TT), 0, stream, a);
  return bands;
}

template <int FMT, int MODE, int NT, int U>
static void launch_q(const ChunkGrid& gr, int64_t rows, int64_t cols, bool tiled,
                     hipStream_t stream, const int32_t* off, int G, const int32_t* chan, int nS,
                     uint8_t* q, uint8_t* scales, float* tscale, uint16_t* resid,
                     const uint32_t* words, int nparts, GridCtl gc = GridCtl{nullptr, 0, -1}) {
  const int64_t per = (int64_t)NT * U;
  const int64_t total = (tiled ? (rows + 15) / 16 * 16 : rows) * (int64_t)gr.cpr;
  dim3 grid((unsigned)((total + per - 1) / per));
  if (tiled)
    hipLaunchKernelGGL((k_quantize<FMT, MODE, NT, U, true>), grid, dim3(NT), 0, stream, gr, rows,
                       cols, true, off, G, chan, nS, q, scales, tscale, resid, words, nparts, gc);
  else
    hipLaunchKernelGGL((k_quantize<FMT, MODE, NT, U, false>), grid, dim3(NT), 0, stream, gr, rows,
                       cols, false, off, G, chan, nS, q, scales, tscale, resid, words, nparts, gc);
}

int launch_quantize(int fmt, bool tiled, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                    const int32_t* off, int G, const int32_t* chan, int nS, uint8_t* q,
                    uint8_t* scales, float* tscale, uint16_t* resid, void* ws,
                    hipStream_t stream) {
  const int64_t chunks = rows * (cols >> 3);
  const ChunkGrid gr{x, (uint32_t)(cols >> 3), ldx, 1.0 / (double)(cols >> 3), ldx == cols};
  // NVFP4 workspace: the exchange state of the small-tensor path, then the
  // amax words of the other paths
  uint32_t* state = static_cast<uint32_t*>(ws);
  uint32_t* words = ws ? reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + WS_HEADER)
                       : nullptr;
  const bool grouped = (off != nullptr && G > 1);
  const int Gk = grouped ? G : 1;
  if (fmt == FP4Q_MXFP4) {
    if (chunks == 0) return 0;
    // no tensor scale: groups matter only for their channel lists
    launch_tile<FP4Q_MXFP4>(tiled, x, rows, cols, ldx, grouped && nS > 0 ? off : nullptr, Gk, chan,
                            nS, q, scales, tscale, resid, nullptr, 0, nullptr, stream);
    return 0;
  }
  if (grouped) {
    // the tile path spreads each group's amax over gslots words of the
    // workspace's amax area (AMAX_PARTS words, or G when larger)
    const bool tile = cols % 32 == 0;
    const int gslots = tile ? std::max(1, std::min(8, AMAX_PARTS / G)) : 1;
    const int nwords = G * gslots;
    hipLaunchKernelGGL(k_quant_init, dim3((nwords + QT - 1) / QT), dim3(QT), 0, stream, words, tscale,
                       G, nwords);
    if (rows > 0) {
      if (tile) {  // amax and quantize passes over the same tiles
        launch_tile<FP4Q_NVFP4>(tiled, x, rows, cols, ldx, off, G, chan, nS, q, scales, tscale,
                                resid, nullptr, 0, words, stream, words, gslots);
      } else {
        const int64_t nwg = (chunks + AMAX_WG_CHUNKS - 1) / AMAX_WG_CHUNKS;
        hipLaunchKernelGGL(k_group_amax, dim3((unsigned)nwg), dim3(QT), 0, stream, gr, rows, off,
                           G, words);
        launch_q<FP4Q_NVFP4, AMAX_GROUP_WORDS, QT, QU>(gr, rows, cols, tiled, stream, off, G, chan,
                                                        nS, q, scales, tscale, resid, words, 0);
      }
    }
    return 0;
  }
  if (rows == 0) {  // empty tensor: tensor scale 1
    hipLaunchKernelGGL(k_quant_init, dim3(1), dim3(QT), 0, stream, words, tscale, 1, 1);
    return 0;
  }
  // the fused path's grid (tiled: rows padded to 16) is at most 32
  // workgroups: one slot each in the grid maximum, all resident at once
  const int64_t launch_chunks = (tiled ? (rows + 15) / 16 * 16 : rows) * (cols >> 3);
  if (launch_chunks <= FUSED_MAX_CHUNKS) {
    static_assert(FUSED_MAX_CHUNKS / FT <= GRID_SLOTS, "one grid slot per workgroup");
    if (SMALL_FUSED) {
      const uint32_t spin = g_hook_spin.load();
      const GridCtl gc{state, spin ? spin : GRID_SPIN_LIMIT, g_hook_skip.load()};
      launch_q<FP4Q_NVFP4, AMAX_FUSED, FT, 1>(gr, rows, cols, tiled, stream, off, 1, chan, nS, q, scales,
                                              tscale, resid, words, 0, gc);
    } else {
      // two short passes spread over many workgroups
      const int64_t parts = (chunks + QT - 1) / QT;
      hipLaunchKernelGGL(k_amax_partial, dim3((unsigned)parts), dim3(QT), 0, stream, gr,
                         (uint32_t)chunks, words);
      launch_q<FP4Q_NVFP4, AMAX_PARTIALS, QT, 1>(gr, rows, cols, tiled, stream, off, 1, chan, nS, q,
                                                  scales, tscale, resid, words, (int)parts);
    }
    return 0;
  }
  const bool tile = cols % 32 == 0;
  const int64_t pmax = tile ? TILE_PARTS : AMAX_PARTS;
  int64_t parts = (chunks + (int64_t)QT * AMAX_BATCH - 1) / ((int64_t)QT * AMAX_BATCH);
  parts = parts < pmax ? parts : pmax;
  hipLaunchKernelGGL(k_amax_partial, dim3((unsigned)parts), dim3(QT), 0, stream, gr,
                     (uint32_t)chunks, words);
  if (tile)
    launch_tile<FP4Q_NVFP4>(tiled, x, rows, cols, ldx, nullptr, 1, chan, nS, q, scales, tscale,
                            resid, words, (int)parts, nullptr, stream);
  else
    launch_q<FP4Q_NVFP4, AMAX_PARTIALS, QT, QU>(gr, rows, cols, tiled, stream, off, 1, chan, nS, q,
                                                 scales, tscale, resid, words, (int)parts);
  return 0;
}

// The quantizer's pass that also scores the columns for online channel
// selection (one group, no channels, rows > 0, cols % 32 == 0): score
// [bands, cols] BF16 bits; returns bands.  NVFP4 takes the partial-amax pass
// first, into the workspace's amax words.
int64_t launch_quantize_scored(int fmt, bool tiled, const uint16_t* x, int64_t rows, int64_t cols,
                               int64_t ldx, uint8_t* q, uint8_t* scales, float* tscale, void* ws,
                               uint16_t* score, hipStream_t stream) {
  if (fmt == FP4Q_MXFP4)
    return launch_tile_score<FP4Q_MXFP4>(tiled, x, rows, cols, ldx, q, scales, tscale, nullptr, 0,
                                         score, stream);
  uint32_t* words = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + WS_HEADER);
  const int64_t chunks = rows * (cols >> 3);
  const ChunkGrid gr{x, (uint32_t)(cols >> 3), ldx, 1.0 / (double)(cols >> 3), ldx == cols};
  int64_t parts = (chunks + (int64_t)QT * AMAX_BATCH - 1) / ((int64_t)QT * AMAX_BATCH);
  parts = parts < TILE_PARTS ? parts : TILE_PARTS;
  hipLaunchKernelGGL(k_amax_partial, dim3((unsigned)parts), dim3(QT), 0, stream, gr,
                     (uint32_t)chunks, words);
  return launch_tile_score<FP4Q_NVFP4>(tiled, x, rows, cols, ldx, q, scales, tscale, words,
                                       (int)parts, score, stream);
}

// Bands of the scored pass (the score buffer holds bands x cols entries).
int64_t quantize_score_bands(bool tiled, int64_t rows, int64_t cols) {
  const int64_t upr = cols / 32;
  const int64_t wc = tiled || upr >= 3 ? 4 : upr;
  const int64_t nrt = (rows + 64 / wc - 1) / (64 / wc);
  return (nrt + TDU * TW - 1) / (TDU * TW);
}

// ---- Outlier Fallback: quantize-dequantize with the deadzone entries kept ----
//
// Decomposition page, abstract: the fallback recovers the deadzone entries.
// One lane per 16-byte chunk (row-major, one group), the quantizer's own
// block scale and codes (chunk_codes); the FP32 output is x itself where the
// code magnitude is 0 and the dequantized value elsewhere (chunk_deq).  Each
// workgroup adds its count of non-zero fallback entries to one 64-bit
// counter, cleared by a fill kernel earlier in the stream.
__global__ void k_clear_u64(unsigned long long* __restrict__ p) {
  if (threadIdx.x == 0) *p = 0ull;
}

template <int FMT>
__global__ void __launch_bounds__(QT) k_qdq_fallback(ChunkGrid gr, int64_t rows,
                                                     float* __restrict__ y, int64_t ldy,
                                                     const uint32_t* __restrict__ amax_words,
                                                     int nparts,
                                                     unsigned long long* __restrict__ count) {
  __shared__ uint32_t red[QT / 64];
  const uint32_t total = (uint32_t)(rows * gr.cpr);
  const uint32_t base = blockIdx.x * (uint32_t)(QT * QU);
  u32x4 v[QU];
#pragma unroll
  for (int u = 0; u < QU; ++u) {
    const uint32_t c = base + u * QT + threadIdx.x;
    v[u] = load_chunk(gr, c < total ? c : total - 1);
  }
  float t = 1.0f;
  if (FMT == FP4Q_NVFP4) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += QT) m = max(m, amax_words[i]);
    t = nv_tensor_scale(bf16_to_f32(wg_max<QT>(m, red)));
  }
  uint32_t nfb = 0;
#pragma unroll
  for (int u = 0; u < QU; ++u) {
    const uint32_t c = base + u * QT + threadIdx.x;
    const ChunkCodes r = chunk_codes<FMT>(v[u], t);
    if (c >= total) continue;
    uint32_t row, cc;
    chunk_rc(gr, c, row, cc);
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t code = (r.packed >> (4 * k)) & 15u;
      const bool fb = (code & 7u) == 0u;
      o[k] = fb ? r.xs[k] : chunk_deq<FMT>(r, code, t);
      nfb += (fb && r.xs[k] != 0.0f) ? 1u : 0u;
    }
    f32x4q* dst = reinterpret_cast<f32x4q*>(y + (int64_t)row * ldy + (int64_t)cc * 8);
    __builtin_nontemporal_store(f32x4q{o[0], o[1], o[2], o[3]}, dst);
    __builtin_nontemporal_store(f32x4q{o[4], o[5], o[6], o[7]}, dst + 1);
  }
  if (count) {
    for (int s = 32; s > 0; s >>= 1) nfb += (uint32_t)__shfl_xor((int)nfb, s);
    __syncthreads();  // red is reused
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = nfb;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t n = 0;
#pragma unroll
      for (int i = 0; i < QT / 64; ++i) n += red[i];
      if (n) atomicAdd(count, (unsigned long long)n);
    }
  }
}

// Outlier Fallback on the tile quantizer's tiles (one group, row-major,
// cols % 32 == 0): each lane forms its unit's codes and block scales exactly
// as the quantizer does, then writes its 32 FP32 outputs: x itself where the
// code magnitude is 0, else the dequantized value -- the E2M1 value (signed,
// exact from the hardware conversion) times the block scale, then (NVFP4)
// times the tensor scale, the residual's rounding.  Workgroups add their
// count of non-zero fallback entries to one counter, cleared earlier.
template <int FMT, int WC, int DU>
__global__ void __launch_bounds__(TT) k_qdq_tile(TileArgs p, float* __restrict__ y, int64_t ldy,
                                                 unsigned long long* __restrict__ count) {
  typedef float v2f32t __attribute__((ext_vector_type(2)));
  constexpr int R = 64 / WC;
  constexpr int OW = WC * 32 + 4;  // an output row of the tile in LDS (padded)
  __shared__ float2 dytab[128];
  __shared__ uint32_t red[TW];
  __shared__ float ob[TW][R][OW];  // a tile's outputs, for row-contiguous stores
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane % R, c = lane / R;
  const uint32_t nct = p.nct;
  u32x4 v[DU][4];
  uint32_t tile[DU];
#pragma unroll
  for (int k = 0; k < DU; ++k) {
    tile[k] = (blockIdx.x * DU + k) * TW + wave;
    const uint32_t T = tile[k] < p.ntiles ? tile[k] : p.ntiles - 1;
    const uint32_t rt = T / nct, ct = T - rt * nct;
    uint32_t row = rt * R + r, uc = ct * WC + c;
    row = row < p.rows ? row : p.rows - 1;
    uc = uc < p.upr ? uc : p.upr - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(p.x + (int64_t)row * p.ldx + (int64_t)uc * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[k][i] = src[i];
  }
  float t = 1.0f, sx = 1.0f, ts = 1.0f, yts = 1.0f;
  if (FMT == FP4Q_NVFP4) {
    uint32_t m = 0;
    for (int i = lane; i < p.nparts; i += 64) m = max(m, p.parts[i]);
    t = nv_tensor_scale(bf16_to_f32(wave_max_u32(m)));
    sx = div_prescale(t);
    ts = t * sx;
    yts = 1.0f / ts;
    if (threadIdx.x < 128) {
      const float d = e4m3_value(threadIdx.x) * t * sx;
      dytab[threadIdx.x] = float2{d, d > 0.0f ? 1.0f / d : 0.0f};
    }
    __syncthreads();
  }
  uint32_t nfb = 0;
#pragma unroll
  for (int k = 0; k < DU; ++k) {
    if (tile[k] >= p.ntiles) break;
    const uint32_t rt = tile[k] / nct, ct = tile[k] - rt * nct;
    const uint32_t row = rt * R + r, uc = ct * WC + c;
    u32x4 codes;
    uint32_t scw;
    if (FMT == FP4Q_NVFP4) {
      if (sx != 1.0f)  // uniform: one tensor scale
        nv_unit<true, true>(v[k], t, sx, ts, yts, dytab, codes, scw);
      else
        nv_unit<true, false>(v[k], t, sx, ts, yts, dytab, codes, scw);
    } else {
      scw = (uint32_t)(mx_exponent(bf16_to_f32(absmax32_bits(v[k]))) + 127);
      const float s = __uint_as_float(scw << 23);
      uint32_t cw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8t w = __builtin_bit_cast(bf16x8t, v[k][i]);
        uint32_t pk = 0;
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, bf16x2t{w[0], w[1]}, s, 0);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, bf16x2t{w[2], w[3]}, s, 1);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, bf16x2t{w[4], w[5]}, s, 2);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, bf16x2t{w[6], w[7]}, s, 3);
        cw[i] = pk;
      }
      codes = u32x4{cw[0], cw[1], cw[2], cw[3]};
    }
    const bool active = row < p.rows && uc < p.upr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // elements 8i .. 8i+7
      const float sb = FMT == FP4Q_NVFP4 ? e4m3_value((scw >> (8 * (i >> 1))) & 0xFFu)
                                         : exp2i((int)scw - 127);
      const v2f32t e[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[i], 1.0f, 0),
                           __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[i], 1.0f, 1),
                           __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[i], 1.0f, 2),
                           __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[i], 1.0f, 3)};
      float o[8];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t xw = v[k][i][h];
        const float x0 = __uint_as_float(xw << 16), x1 = __uint_as_float(xw & 0xFFFF0000u);
        const float d0 = FMT == FP4Q_NVFP4 ? (e[h].x * sb) * t : e[h].x * sb;
        const float d1 = FMT == FP4Q_NVFP4 ? (e[h].y * sb) * t : e[h].y * sb;
        o[2 * h] = e[h].x == 0.0f ? x0 : d0;
        o[2 * h + 1] = e[h].y == 0.0f ? x1 : d1;
        nfb += (active && e[h].x == 0.0f && x0 != 0.0f) ? 1u : 0u;
        nfb += (active && e[h].y == 0.0f && x1 != 0.0f) ? 1u : 0u;
      }
      f32x4q* d4 = reinterpret_cast<f32x4q*>(&ob[wave][r][c * 32 + 8 * i]);
      d4[0] = f32x4q{o[0], o[1], o[2], o[3]};
      d4[1] = f32x4q{o[4], o[5], o[6], o[7]};
    }
    // the tile's rows leave in contiguous runs: 16 bytes per lane, WC * 8
    // lanes per row (one wave's LDS operations complete in order)
    const int64_t col0 = (int64_t)ct * (WC * 32);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int idx = m * 64 + lane, rr = idx / (WC * 8), c16 = idx - rr * (WC * 8);
      const uint32_t orow = rt * R + (uint32_t)rr;
      if (orow < p.rows && ct * WC + (uint32_t)(c16 >> 3) < p.upr) {
        const f32x4q val = *reinterpret_cast<const f32x4q*>(&ob[wave][rr][4 * c16]);
        __builtin_nontemporal_store(val, reinterpret_cast<f32x4q*>(y + (int64_t)orow * ldy + col0 + 4 * c16));
      }
    }
  }
  if (count) {
    for (int s2 = 32; s2 > 0; s2 >>= 1) nfb += (uint32_t)__shfl_xor((int)nfb, s2);
    if (lane == 0) red[wave] = nfb;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t n = 0;
#pragma unroll
      for (int i = 0; i < TW; ++i) n += red[i];
      if (n) atomicAdd(count, (unsigned long long)n);
    }
  }
}

template <int FMT>
static void launch_qdq_tile(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, float* y,
                            int64_t ldy, unsigned long long* cnt, const uint32_t* parts, int nparts,
                            hipStream_t stream) {
  TileArgs a{};
  a.x = x; a.ldx = ldx; a.cols = cols;
  a.rows = (uint32_t)rows;
  a.upr = (uint32_t)(cols / 32);
  a.parts = parts; a.nparts = nparts;
  const int wc = a.upr >= 3 ? 4 : (int)a.upr;
  const uint32_t R = 64u / (uint32_t)wc;
  a.nct = (a.upr + wc - 1) / wc;
  a.ntiles = (uint32_t)((rows + R - 1) / R) * a.nct;
  const dim3 grid((a.ntiles + TDU * TW - 1) / (TDU * TW));
  if (wc == 4) hipLaunchKernelGGL((k_qdq_tile<FMT, 4, TDU>), grid, dim3(TT), 0, stream, a, y, ldy, cnt);
  else if (wc == 2) hipLaunchKernelGGL((k_qdq_tile<FMT, 2, TDU>), grid, dim3(TT), 0, stream, a, y, ldy, cnt);
  else hipLaunchKernelGGL((k_qdq_tile<FMT, 1, TDU>), grid, dim3(TT), 0, stream, a, y, ldy, cnt);
}

int launch_qdq_fallback(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                        float* y, int64_t ldy, int64_t* count, void* ws, hipStream_t stream) {
  unsigned long long* cnt = reinterpret_cast<unsigned long long*>(count);
  if (cnt) hipLaunchKernelGGL(k_clear_u64, dim3(1), dim3(64), 0, stream, cnt);
  if (rows == 0) return 0;
  const int64_t chunks = rows * (cols >> 3);
  const ChunkGrid gr{x, (uint32_t)(cols >> 3), ldx, 1.0 / (double)(cols >> 3), ldx == cols};
  const dim3 grid((unsigned)((chunks + QT * QU - 1) / (QT * QU)));
  const bool tile = cols % 32 == 0;  // the tile form; else one lane per 8-element chunk
  if (fmt == FP4Q_MXFP4) {
    launch_qdq_tile<FP4Q_MXFP4>(x, rows, cols, ldx, y, ldy, cnt, nullptr, 0, stream);
    return 0;
  }
  uint32_t* words = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + WS_HEADER);
  const int64_t pmax = tile ? TILE_PARTS : AMAX_PARTS;
  int64_t parts = (chunks + (int64_t)QT * AMAX_BATCH - 1) / ((int64_t)QT * AMAX_BATCH);
  parts = parts < pmax ? parts : pmax;
  hipLaunchKernelGGL(k_amax_partial, dim3((unsigned)parts), dim3(QT), 0, stream, gr,
                     (uint32_t)chunks, words);
  if (tile)
    launch_qdq_tile<FP4Q_NVFP4>(x, rows, cols, ldx, y, ldy, cnt, words, (int)parts, stream);
  else
    hipLaunchKernelGGL(k_qdq_fallback<FP4Q_NVFP4>, grid, dim3(QT), 0, stream, gr, rows, y, ldy,
                       words, (int)parts, cnt);
  return 0;
}

size_t quantize_workspace_bytes(int fmt, int G) {
  if (fmt != FP4Q_NVFP4) return 0;
  const int n = G > AMAX_PARTS ? G : AMAX_PARTS;
  return WS_HEADER + (size_t)n * sizeof(uint32_t);
}

int quantize_status(const void* ws, hipStream_t stream, uint32_t* status) {
  uint32_t* word = static_cast<uint32_t*>(const_cast<void*>(ws)) + WS_STATUS;
  uint32_t v = 0;
  if (hipStreamSynchronize(stream) != hipSuccess) return -1;
  if (hipMemcpyAsync(&v, word, sizeof v, hipMemcpyDeviceToHost, stream) != hipSuccess) return -1;
  if (hipStreamSynchronize(stream) != hipSuccess) return -1;
  if (v != 0u) {
    if (hipMemsetAsync(word, 0, sizeof v, stream) != hipSuccess) return -1;
    if (hipStreamSynchronize(stream) != hipSuccess) return -1;
  }
  *status = v;
  return 0;
}

}  // namespace fp4q
