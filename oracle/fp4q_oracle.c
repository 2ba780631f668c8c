/*
 * fp4q_oracle.c -- plain CPU oracle for block-scaled FP4 (NVFP4 / MXFP4)
 * activation quantization, the W4A4 GEMM with sparse residual compensation,
 * its expert-grouped form, and the exact three-way MXFP4 error decomposition.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no source with the HIP
 * path: every codec here is written as its definition (nearest value out of an
 * enumerated set, ties broken by the stated rule), not as the bit tricks the
 * GPU kernels use.
 *
 * Sources (titles of the pages this follows):
 *  - "QUADS: Stabilizing NVFP4 Reinforcement Learning for MoE via
 *    QUantization-error Alignment across Dual Sides", abstract: NVFP4 joins
 *    fine-grained scaling with native W4A4 FP4 GEMMs; activations are
 *    re-quantized online and their error is amplified by the coarse E2M1 grid;
 *    Residual Activation Compensation corrects high-error activation channels
 *    while the W4A4 GEMM stays native.
 *  - The German explainer of the same paper (gist.science), section 2.2 B:
 *    a residual correction term Delta X_q on selected channels is added to
 *    the quantized output; section 1: E2M1 has 8 levels per sign.
 *  - "FourSight: Stable FP4 RL Post-Training via Sequence Filtering and Sparse
 *    Channel Compensation", abstract: the top-variance activation channels are
 *    kept in BF16 while the rest stays NVFP4.
 *  - "Decomposing MXFP4 quantization error for LLM reinforcement learning",
 *    abstract: the MXFP4 error splits exactly into three additive parts --
 *    scale bias (power-of-two rounding of the scale), deadzone truncation
 *    (small values zeroed) and grid noise (rounding to the 4-bit grid).
 *
 * The pages do not fix block sizes, scale encodings, rounding or packing; the
 * readings used here (each stated where it is used) are:
 *  - E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; round to nearest, ties to
 *    the even mantissa bit; saturate at 6; sign bit = sign bit of the input.
 *  - NVFP4: 16-element blocks along K, E4M3 (bias 7, max 448, no inf) block
 *    scale from amax/6 divided by an FP32 tensor scale t = amax_tensor/2688.
 *  - MXFP4: 32-element blocks, scale 2^e with the smallest e such that
 *    6*2^e >= block amax (nothing clips), stored as E8M0 code e+127.
 *  - Two codes per byte, even element in the low nibble.
 *  - Residual R = bf16(x - deq(code)) on the chosen channels only.
 *  - GEMM: Y = deq(Xq) * deq(Wq)^T + R[:,S] * deq(Wq)[:,S]^T, in FP64.
 *  - Online channel selection (the explainer's section 2.2 B: a binary mask
 *    keeps the top-k% channels by residual magnitude): the magnitude of
 *    channel c is max over rows of |R(m, c)|, R the BF16 residual the
 *    quantizer would emit for c; the k largest win, ties to the lower index;
 *    the list is returned ascending.
 *  - Quantize-before-permute for the expert-grouped layer (the QUADS
 *    abstract's NVFP4 rollout for MoE; the pages do not say where in the
 *    routing the activations are quantized): the token matrix is quantized
 *    once, one tensor scale for all tokens, and row m of the expert-ordered
 *    operand is a copy of the codes and block scales of its token; the
 *    residual of expert g's channels is R(token, S_g[j]) by the rule above.
 *  - Second-pass residual (the explainer's section 2.2 B: the high-residual
 *    channels are quantized a second time and the correction term is added
 *    to the quantized output): R[:,S] itself quantized by the same rule, as
 *    an M x |S| tensor with blocks along the selected-channel index j and,
 *    for NVFP4, its own tensor scale; the compensation term is then
 *    deq(Q(R)) * deq(Wq)[:,S]^T.
 *
 * Every FP32 step of the quantizer is one IEEE binary32 operation with
 * round-to-nearest-even; build with -O2 -ffp-contract=off, no fast-math.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_NVFP4 0
#define ORC_MXFP4 1

/* Thread count of the parallel loops (timing of the CPU baseline only; no
 * result depends on it). */
void orc_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes indexed by the 3 low bits of a code (sign is bit 3). */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(uint8_t code) {
    double m = E2M1_GRID[code & 7];
    return (code & 8) ? -m : m;
}

/* Nearest E2M1 magnitude to |q|; on an exact tie the code whose mantissa bit
 * (bit 0) is 0 wins.  Anything at or above the largest level 6 is nearest to
 * 6 (saturation); it is decided first because for huge |q| the FP64
 * distances below would no longer be exact.  Below 6 every distance is exact
 * (a float and a grid value under 8 differ by at most ~30 significant bits,
 * and a tiny float's distance to 0 is the float itself). */
uint8_t orc_e2m1_encode_mag(float q) {
    double a = fabs((double)q);
    if (a >= 6.0) return 7;
    int best = 0;
    double best_d = fabs(a - E2M1_GRID[0]);
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - E2M1_GRID[c]);   /* exact: few significant bits */
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)best;
}

/* E4M3 (FN variant): sign 1, exponent 4 (bias 7), mantissa 3.  Exponent
 * field 0 is subnormal: m/8 * 2^-6.  Code 0x7F / 0xFF is NaN. */
double orc_e4m3_value(uint8_t code) {
    int e = (code >> 3) & 15, m = code & 7;
    double v = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return (code & 0x80) ? -v : v;
}

/* Nearest non-negative finite E4M3 value to v >= 0, ties to the even code
 * (the code's lowest bit is the mantissa's lowest bit); anything above the
 * largest finite value 448 lands on 448 (saturating). */
uint8_t orc_e4m3_encode(float v) {
    double a = (double)v;
    if (a >= 448.0) return 0x7E;  /* at or beyond the largest finite value */
    int best = 0;
    double best_d = fabs(a - orc_e4m3_value(0));
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(a - orc_e4m3_value((uint8_t)c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)best;
}

double orc_e8m0_value(uint8_t code) { return ldexp(1.0, (int)code - 127); }

float orc_bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* BF16 nearest to a finite float, ties to even: the two candidates are the
 * float truncated to 16 bits and the next BF16 away from zero. */
uint16_t orc_bf16_from_f32(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t lo = (uint16_t)(u >> 16);
    if ((u & 0xFFFFu) == 0) return lo;
    uint16_t hi = (uint16_t)(lo + 1);        /* next magnitude up, same sign */
    double dl = fabs((double)f - (double)orc_bf16_value(lo));
    double dh = fabs((double)orc_bf16_value(hi) - (double)f);
    if (isinf(orc_bf16_value(hi))) dh = ldexp(1.0, 127 - 8);  /* half ulp of max */
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1) ? hi : lo;
}

/* MXFP4 block exponent: the smallest integer e in [-127, 127] with
 * 6 * 2^e >= amax (every element then fits the grid without clipping).
 * An all-zero block gets e = -127. */
int orc_mx_exponent(float amax) {
    for (int e = -127; e <= 127; ++e)
        if (6.0 * ldexp(1.0, e) >= (double)amax) return e;
    return 127;
}

/* NVFP4 tensor scale from the tensor (or group) amax: t = A / 2688 with
 * 2688 = 6 * 448, so the largest block maps its amax onto 6 * 448. */
float orc_nv_tensor_scale(float amax) {
    float t = amax / 2688.0f;
    if (amax == 0.0f || t == 0.0f) t = 1.0f;
    return t;
}

/* ------------------------------------------------------------------------ */
/* Quantizer                                                                 */
/* ------------------------------------------------------------------------ */

static float absf_bf16(uint16_t h) { return fabsf(orc_bf16_value(h)); }


/*
 * Quantize X (bf16 [rows, cols], row stride ldx) in row groups
 * [off[g], off[g+1]) (off == NULL: a single group of all rows).
 * Outputs: q [rows, cols/2], scales [rows, cols/blk],
 * tensor_scale [num_groups] (NVFP4 only), resid bf16 [rows, n_chan] for the
 * channels chan_idx[g*n_chan .. +n_chan) of each row's group.
 * Returns 0, or -1 for a shape the formats do not allow.
 */
int orc_quantize(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                 const int32_t* off, int32_t num_groups, const int32_t* chan_idx,
                 int32_t n_chan, uint8_t* q, uint8_t* scales, float* tensor_scale,
                 uint16_t* resid) {
    const int blk = (fmt == ORC_NVFP4) ? 16 : 32;
    if (fmt != ORC_NVFP4 && fmt != ORC_MXFP4) return -1;
    if (cols % blk != 0 || num_groups < 1) return -1;
    const int64_t nb = cols / blk;

    for (int32_t g = 0; g < num_groups; ++g) {
        int64_t r0 = off ? off[g] : 0, r1 = off ? off[g + 1] : rows;
        const int32_t* S = chan_idx ? chan_idx + (int64_t)g * n_chan : NULL;
        /* jmap[c] = position of channel c in the group's channel list, or -1 */
        int32_t* jmap = (int32_t*)malloc(sizeof(int32_t) * (size_t)cols);
        if (!jmap) return -1;
        for (int64_t c = 0; c < cols; ++c) jmap[c] = -1;
        for (int32_t j = 0; S && j < n_chan; ++j) jmap[S[j]] = j;

        /* Tensor scale (NVFP4): amax over the group's rows. */
        float t = 1.0f;
        if (fmt == ORC_NVFP4) {
            float A = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = 0; c < cols; ++c) {
                    float a = absf_bf16(x[r * ldx + c]);
                    if (a > A) A = a;
                }
            t = orc_nv_tensor_scale(A);
            tensor_scale[g] = t;
        }

#pragma omp parallel for schedule(static)
        for (int64_t r = r0; r < r1; ++r) {
            for (int64_t b = 0; b < nb; ++b) {
                const uint16_t* xb = x + r * ldx + b * blk;
                float amax = 0.0f;
                for (int k = 0; k < blk; ++k) {
                    float a = absf_bf16(xb[k]);
                    if (a > amax) amax = a;
                }
                /* Block scale. */
                uint8_t sc;
                float d;            /* the divisor that maps x onto the grid */
                float sb = 0.0f;    /* NVFP4 decoded block scale */
                int e = 0;          /* MXFP4 exponent */
                if (fmt == ORC_NVFP4) {
                    float v = (amax / 6.0f) / t;
                    sc = orc_e4m3_encode(v);
                    sb = (float)orc_e4m3_value(sc);
                    d = sb * t;
                } else {
                    e = orc_mx_exponent(amax);
                    sc = (uint8_t)(e + 127);
                    d = (float)ldexp(1.0, e);
                }
                scales[r * nb + b] = sc;

                for (int k = 0; k < blk; ++k) {
                    uint16_t h = xb[k];
                    float xv = orc_bf16_value(h);
                    uint8_t mag;
                    if (fmt == ORC_NVFP4)
                        mag = (d == 0.0f) ? 0 : orc_e2m1_encode_mag(fabsf(xv) / d);
                    else
                        mag = orc_e2m1_encode_mag(fabsf(xv) * (float)ldexp(1.0, -e));
                    uint8_t code = (uint8_t)(((h >> 15) << 3) | mag);
                    int64_t kk = b * blk + k;
                    uint8_t* byte = q + r * (cols / 2) + kk / 2;
                    if ((kk & 1) == 0)
                        *byte = (uint8_t)((*byte & 0xF0) | code);
                    else
                        *byte = (uint8_t)((*byte & 0x0F) | (code << 4));

                    if (S && resid) {
                        int32_t j = jmap[kk];
                        if (j >= 0) {
                            /* Dequantized value, one FP32 rounding per step. */
                            float p;
                            if (fmt == ORC_NVFP4)
                                p = ((float)E2M1_GRID[mag] * sb) * t;
                            else
                                p = (float)E2M1_GRID[mag] * d;
                            if (code & 8) p = -p;
                            float rr = xv - p;
                            resid[r * n_chan + j] = orc_bf16_from_f32(rr);
                        }
                    }
                }
            }
        }
        free(jmap);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Online channel selection                                                  */
/* ------------------------------------------------------------------------ */

/* The BF16 residual of element (r, c) from X and its quantized form, with
 * the same FP32 steps as the quantizer's residual output. */
static uint16_t residual_at(int fmt, const uint16_t* x, int64_t ldx, const uint8_t* q,
                            const uint8_t* scales, float t, int64_t cols, int64_t r, int64_t c) {
    const int blk = (fmt == ORC_NVFP4) ? 16 : 32;
    const uint8_t byte = q[r * (cols / 2) + c / 2];
    const uint8_t code = (c & 1) ? (byte >> 4) : (byte & 15);
    const uint8_t sc = scales[r * (cols / blk) + c / blk];
    float p;
    if (fmt == ORC_NVFP4)
        p = ((float)E2M1_GRID[code & 7] * (float)orc_e4m3_value(sc)) * t;
    else
        p = (float)E2M1_GRID[code & 7] * (float)orc_e8m0_value(sc);
    if (code & 8) p = -p;
    return orc_bf16_from_f32(orc_bf16_value(x[r * ldx + c]) - p);
}

typedef struct {
    float score;
    int64_t c;
} ChanScore;

/* larger score first, then the lower channel index */
static int by_score(const void* a, const void* b) {
    const ChanScore* u = (const ChanScore*)a;
    const ChanScore* v = (const ChanScore*)b;
    if (u->score != v->score) return u->score > v->score ? -1 : 1;
    return u->c < v->c ? -1 : (u->c > v->c ? 1 : 0);
}

static int by_index(const void* a, const void* b) {
    const int32_t u = *(const int32_t*)a, v = *(const int32_t*)b;
    return u < v ? -1 : (u > v ? 1 : 0);
}

/* Select the k channels of largest residual magnitude from X [rows, cols]
 * and its quantized form (q, scales, tensor scale t; row-major).  Writes
 * chan_out [k] ascending and resid_out [rows, k] (BF16 residual on them).
 * Returns 0, or -1 for k outside [0, cols]. */
int orc_select_channels(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                        const uint8_t* q, const uint8_t* scales, float t, int32_t k,
                        int32_t* chan_out, uint16_t* resid_out) {
    if (k < 0 || k > cols) return -1;
    ChanScore* sc = (ChanScore*)malloc(sizeof(ChanScore) * (size_t)(cols > 0 ? cols : 1));
    if (!sc) return -1;
    const float tt = (fmt == ORC_NVFP4) ? t : 1.0f;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        float m = 0.0f;
        for (int64_t r = 0; r < rows; ++r) {
            const float a = fabsf(orc_bf16_value(residual_at(fmt, x, ldx, q, scales, tt, cols, r, c)));
            if (a > m) m = a;
        }
        sc[c].score = m;
        sc[c].c = c;
    }
    qsort(sc, (size_t)cols, sizeof(ChanScore), by_score);
    for (int32_t j = 0; j < k; ++j) chan_out[j] = (int32_t)sc[j].c;
    free(sc);
    qsort(chan_out, (size_t)k, sizeof(int32_t), by_index);
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t j = 0; j < k; ++j)
            resid_out[r * k + j] = residual_at(fmt, x, ldx, q, scales, tt, cols, r, chan_out[j]);
    return 0;
}

/* Quantize-before-permute: q, scales (row-major, one group, tensor scale t)
 * are the quantization of the token matrix x [tokens, cols].  Row m of the
 * expert-ordered output is token row_src[m]: its codes and block scales are
 * copied, and for the group g holding m (offsets[g] <= m < offsets[g+1]) the
 * residual on chan[g][j] is the quantizer's residual at that token.  Returns
 * -1 for a token index or offsets out of range. */
int orc_permute_quantized(int fmt, const uint16_t* x, int64_t tokens, int64_t cols, int64_t ldx,
                          const uint8_t* q, const uint8_t* scales, float t,
                          const int32_t* row_src, int64_t rows, const int32_t* offsets,
                          int32_t G, const int32_t* chan, int32_t nS, uint8_t* q_out,
                          uint8_t* s_out, uint16_t* r_out) {
    const int blk = (fmt == ORC_NVFP4) ? 16 : 32;
    const float tt = (fmt == ORC_NVFP4) ? t : 1.0f;
    if (G < 1 || offsets[0] != 0 || offsets[G] != rows) return -1;
    for (int32_t g = 0; g < G; ++g)
        if (offsets[g + 1] < offsets[g]) return -1;
    for (int64_t m = 0; m < rows; ++m)
        if (row_src[m] < 0 || row_src[m] >= tokens) return -1;
    for (int64_t m = 0; m < rows; ++m) {
        const int64_t tok = row_src[m];
        memcpy(q_out + m * (cols / 2), q + tok * (cols / 2), (size_t)(cols / 2));
        memcpy(s_out + m * (cols / blk), scales + tok * (cols / blk), (size_t)(cols / blk));
    }
    for (int32_t g = 0; g < G; ++g)
        for (int64_t m = offsets[g]; m < offsets[g + 1]; ++m)
            for (int32_t j = 0; j < nS; ++j)
                r_out[m * nS + j] = residual_at(fmt, x, ldx, q, scales, tt, cols, row_src[m],
                                                chan[(int64_t)g * nS + j]);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantization and the compensated W4A4 GEMM (FP64 definition)            */
/* ------------------------------------------------------------------------ */

/* Value of element k of row r of a packed FP4 matrix with its block scale
 * and tensor scale: e2m1 * block scale * tensor scale. */
static double deq(int fmt, const uint8_t* qm, const uint8_t* sm, double ts, int64_t K,
                  int64_t r, int64_t k) {
    const int blk = (fmt == ORC_NVFP4) ? 16 : 32;
    uint8_t byte = qm[r * (K / 2) + k / 2];
    uint8_t code = (k & 1) ? (byte >> 4) : (byte & 15);
    uint8_t sc = sm[r * (K / blk) + k / blk];
    double s = (fmt == ORC_NVFP4) ? orc_e4m3_value(sc) * ts : orc_e8m0_value(sc);
    return orc_e2m1_value(code) * s;
}

/* The residual operand of the compensation term: BF16 values R[m][j], or
 * (second pass) the FP4 codes rq / block scales rs / tensor scale rts of
 * R quantized as an M x nS tensor. */
typedef struct {
    const uint16_t* R;
    const uint8_t* rq;
    const uint8_t* rs;
    double rts;
} ResidOperand;

static double resid_value(int fmt, const ResidOperand* ro, int32_t nS, int64_t m, int32_t j) {
    if (ro->rq) return deq(fmt, ro->rq, ro->rs, ro->rts, nS, m, j);
    return (double)orc_bf16_value(ro->R[m * nS + j]);
}

/* One output element: y = sum_k A[m,k] B[n,k] + sum_j R[m,j] B[n,S_j], with
 * yabs the same sum over absolute values of every term. */
static void gemm_point_r(int fmt, int64_t K, const uint8_t* aq, const uint8_t* as, double ats,
                         const uint8_t* bq, const uint8_t* bs, double bts, const int32_t* S,
                         int32_t nS, const ResidOperand* ro, int64_t m, int64_t n, double* y,
                         double* yabs) {
    double acc = 0.0, aabs = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = deq(fmt, aq, as, ats, K, m, k) * deq(fmt, bq, bs, bts, K, n, k);
        acc += p;
        aabs += fabs(p);
    }
    for (int32_t j = 0; j < nS; ++j) {
        double p = resid_value(fmt, ro, nS, m, j) * deq(fmt, bq, bs, bts, K, n, S[j]);
        acc += p;
        aabs += fabs(p);
    }
    *y = acc;
    *yabs = aabs;
}

static void gemm_point(int fmt, int64_t K, const uint8_t* aq, const uint8_t* as, double ats,
                       const uint8_t* bq, const uint8_t* bs, double bts, const int32_t* S,
                       int32_t nS, const uint16_t* R, int64_t m, int64_t n, double* y,
                       double* yabs) {
    const ResidOperand ro = {R, NULL, NULL, 0.0};
    gemm_point_r(fmt, K, aq, as, ats, bq, bs, bts, S, nS, &ro, m, n, y, yabs);
}

/* Dense GEMM at chosen points (pm[i], pn[i]).  A = activations [M, K]
 * quantized, B = weights stored as W^T [N, K] quantized; tensor scales are
 * host values (1 for MXFP4). */
int orc_gemm_points(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* aq,
                    const uint8_t* as, float ats, const uint8_t* bq, const uint8_t* bs,
                    float bts, const int32_t* S, int32_t nS, const uint16_t* R,
                    const int64_t* pm, const int64_t* pn, int64_t npts, double* y,
                    double* yabs) {
    (void)M;
    (void)N;
    double ta = (fmt == ORC_NVFP4) ? ats : 1.0, tb = (fmt == ORC_NVFP4) ? bts : 1.0;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < npts; ++i)
        gemm_point(fmt, K, aq, as, ta, bq, bs, tb, S, nS, R, pm[i], pn[i], &y[i], &yabs[i]);
    return 0;
}

/* Dense GEMM, every output: y, yabs [M, N] row-major. */
int orc_gemm_full(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* aq,
                  const uint8_t* as, float ats, const uint8_t* bq, const uint8_t* bs,
                  float bts, const int32_t* S, int32_t nS, const uint16_t* R, double* y,
                  double* yabs) {
    double ta = (fmt == ORC_NVFP4) ? ats : 1.0, tb = (fmt == ORC_NVFP4) ? bts : 1.0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            gemm_point(fmt, K, aq, as, ta, bq, bs, tb, S, nS, R, m, n, &y[m * N + n],
                       &yabs[m * N + n]);
    return 0;
}

/* Dense GEMM at points with the second-pass (FP4) residual: rq [M, nS/2]
 * codes, rs [M, nS/blk] block scales, rts its tensor scale (NVFP4; ignored
 * for MXFP4). */
int orc_gemm_points_r4(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* aq,
                       const uint8_t* as, float ats, const uint8_t* bq, const uint8_t* bs,
                       float bts, const int32_t* S, int32_t nS, const uint8_t* rq,
                       const uint8_t* rs, float rts, const int64_t* pm, const int64_t* pn,
                       int64_t npts, double* y, double* yabs) {
    (void)M;
    (void)N;
    const int blk = (fmt == ORC_NVFP4) ? 16 : 32;
    if (nS > 0 && (nS % blk != 0 || !rq || !rs)) return -1;
    double ta = (fmt == ORC_NVFP4) ? ats : 1.0, tb = (fmt == ORC_NVFP4) ? bts : 1.0;
    const ResidOperand ro = {NULL, rq, rs, (fmt == ORC_NVFP4) ? (double)rts : 1.0};
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < npts; ++i)
        gemm_point_r(fmt, K, aq, as, ta, bq, bs, tb, S, nS, &ro, pm[i], pn[i], &y[i], &yabs[i]);
    return 0;
}

/* The same, every output: y, yabs [M, N] row-major. */
int orc_gemm_full_r4(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* aq,
                     const uint8_t* as, float ats, const uint8_t* bq, const uint8_t* bs, float bts,
                     const int32_t* S, int32_t nS, const uint8_t* rq, const uint8_t* rs,
                     float rts, double* y, double* yabs) {
    const int blk = (fmt == ORC_NVFP4) ? 16 : 32;
    if (nS > 0 && (nS % blk != 0 || !rq || !rs)) return -1;
    double ta = (fmt == ORC_NVFP4) ? ats : 1.0, tb = (fmt == ORC_NVFP4) ? bts : 1.0;
    const ResidOperand ro = {NULL, rq, rs, (fmt == ORC_NVFP4) ? (double)rts : 1.0};
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            gemm_point_r(fmt, K, aq, as, ta, bq, bs, tb, S, nS, &ro, m, n, &y[m * N + n],
                         &yabs[m * N + n]);
    return 0;
}

/* Expert-grouped GEMM at chosen points.  Row m belongs to the group g with
 * off[g] <= m < off[g+1]; group g uses weight slice g (bq + g*N*K/2, ...),
 * its own tensor scales ats[g], bts[g] and channel list S + g*nS.  The
 * residual rows are indexed by the global row m. */
int orc_grouped_gemm_points(int fmt, int64_t total_rows, int64_t N, int64_t K,
                            const int32_t* off, int32_t G, const uint8_t* aq,
                            const uint8_t* as, const float* ats, const uint8_t* bq,
                            const uint8_t* bs, const float* bts, const int32_t* S, int32_t nS,
                            const uint16_t* R, const int64_t* pm, const int64_t* pn,
                            int64_t npts, double* y, double* yabs) {
    const int blk = (fmt == ORC_NVFP4) ? 16 : 32;
    (void)total_rows;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < npts; ++i) {
        int64_t m = pm[i];
        int32_t g = 0;
        while (g < G && !(off[g] <= m && m < off[g + 1])) ++g;
        if (g == G) {
            y[i] = NAN;
            yabs[i] = NAN;
            continue;
        }
        double ta = (fmt == ORC_NVFP4) ? ats[g] : 1.0, tb = (fmt == ORC_NVFP4) ? bts[g] : 1.0;
        gemm_point(fmt, K, aq, as, ta, bq + (int64_t)g * N * (K / 2),
                   bs + (int64_t)g * N * (K / blk), tb, S ? S + (int64_t)g * nS : NULL, nS, R, m,
                   pn[i], &y[i], &yabs[i]);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Exact three-way MXFP4 error decomposition                                 */
/* ------------------------------------------------------------------------ */

/*
 * Per 32-block: s = 2^e is the scale the quantizer uses, s* = amax/6 the
 * ideal (unrounded) scale.  Q_s is the MXFP4 quantizer; Q* rounds x/s* to the
 * E2M1 grid with the same tie rule.  Per element:
 *   total      = x - Q_s(x)
 *   deadzone   = x              if Q_s(x) == 0, else 0
 *   grid_noise = x - Q*(x)      if Q_s(x) != 0, else 0
 *   scale_bias = Q*(x) - Q_s(x) if Q_s(x) != 0, else 0
 * so total = scale_bias + deadzone + grid_noise for every element.  Values are
 * produced multiplied by 6 (6x, g*amax, 6*g*2^e are all short dyadic numbers,
 * so each difference is exact in FP64).
 * Component order: 0 total, 1 scale_bias, 2 deadzone, 3 grid_noise.
 */
static void decompose_elem(float xv, float amax, int e, double c6[4], int* in_dz) {
    double x6 = 6.0 * (double)xv;
    double ax = fabs((double)xv);
    double sgn = signbit(xv) ? -1.0 : 1.0;
    /* Q_s: the quantizer's own E2M1 code (same rule as orc_quantize). */
    uint8_t mag = orc_e2m1_encode_mag(fabsf(xv) * (float)ldexp(1.0, -e));
    double qs6 = sgn * 6.0 * E2M1_GRID[mag] * ldexp(1.0, e);
    /* Q*: nearest grid point to |x| / (amax/6) = 6|x|/amax, decided exactly by
     * comparing distances scaled by amax: | 6|x| - g*amax |. */
    int best = 0;
    if (amax > 0.0f) {
        double A = (double)amax;
        double best_d = fabs(6.0 * ax - E2M1_GRID[0] * A);
        for (int c = 1; c < 8; ++c) {
            double d = fabs(6.0 * ax - E2M1_GRID[c] * A);
            if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
                best = c;
                best_d = d;
            }
        }
    }
    double qstar6 = sgn * E2M1_GRID[best] * (double)amax;
    c6[0] = x6 - qs6;
    if (mag == 0) {
        c6[1] = 0.0;
        c6[2] = x6;
        c6[3] = 0.0;
        *in_dz = (xv != 0.0f);
    } else {
        c6[1] = qstar6 - qs6;
        c6[2] = 0.0;
        c6[3] = x6 - qstar6;
        *in_dz = 0;
    }
}

/* Per-element components (times 6), for small tensors: out[4][rows*cols]. */
int orc_error_components(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                         double* out) {
    if (cols % 32 != 0) return -1;
    int64_t n = rows * cols;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < cols / 32; ++b) {
            const uint16_t* xb = x + r * ldx + b * 32;
            float amax = 0.0f;
            for (int k = 0; k < 32; ++k)
                if (absf_bf16(xb[k]) > amax) amax = absf_bf16(xb[k]);
            int e = orc_mx_exponent(amax);
            for (int k = 0; k < 32; ++k) {
                double c6[4];
                int dz;
                decompose_elem(orc_bf16_value(xb[k]), amax, e, c6, &dz);
                for (int c = 0; c < 4; ++c) out[c * n + r * cols + b * 32 + k] = c6[c];
            }
        }
    return 0;
}

/* 320-bit two's complement fixed point, 5 little-endian 64-bit limbs,
 * least significant bit worth 2^-136. */
#define FIX_LIMBS 5
#define FIX_LSB_EXP (-136)

/* acc += v (v an FP64 multiple of 2^-136 whose magnitude is below 2^183). */
static void fix_add(uint64_t acc[FIX_LIMBS], double v) {
    if (v == 0.0) return;
    int ex;
    double fr = frexp(fabs(v), &ex);                 /* |v| = fr * 2^ex */
    uint64_t mant = (uint64_t)ldexp(fr, 53);         /* 53-bit integer */
    int shift = ex - 53 - FIX_LSB_EXP;               /* |v| = mant * 2^(shift-136) */
    while (shift < 0) {                              /* drop trailing zero bits */
        if (mant & 1) abort();                       /* not a multiple of 2^-136 */
        mant >>= 1;
        ++shift;
    }
    uint64_t mag[FIX_LIMBS] = {0};
    int li = shift / 64, bo = shift % 64;
    if (li >= FIX_LIMBS) abort();
    mag[li] = mant << bo;
    if (bo && li + 1 < FIX_LIMBS) mag[li + 1] = mant >> (64 - bo);
    if (v < 0) {  /* negate: invert and add one */
        unsigned __int128 c = 1;
        for (int i = 0; i < FIX_LIMBS; ++i) {
            c += (unsigned __int128)(~mag[i]);
            mag[i] = (uint64_t)c;
            c >>= 64;
        }
    }
    unsigned __int128 c = 0;
    for (int i = 0; i < FIX_LIMBS; ++i) {
        c += (unsigned __int128)acc[i] + mag[i];
        acc[i] = (uint64_t)c;
        c >>= 64;
    }
}

static void fix_add_fix(uint64_t acc[FIX_LIMBS], const uint64_t b[FIX_LIMBS]) {
    unsigned __int128 c = 0;
    for (int i = 0; i < FIX_LIMBS; ++i) {
        c += (unsigned __int128)acc[i] + b[i];
        acc[i] = (uint64_t)c;
        c >>= 64;
    }
}

/* Approximate value of the fixed-point number (for reporting). */
static double fix_to_double(const uint64_t a[FIX_LIMBS]) {
    uint64_t t[FIX_LIMBS];
    memcpy(t, a, sizeof t);
    int neg = (t[FIX_LIMBS - 1] >> 63) & 1;
    if (neg) {
        unsigned __int128 c = 1;
        for (int i = 0; i < FIX_LIMBS; ++i) {
            c += (unsigned __int128)(~t[i]);
            t[i] = (uint64_t)c;
            c >>= 64;
        }
    }
    long double v = 0.0L;
    for (int i = FIX_LIMBS - 1; i >= 0; --i) v = v * 18446744073709551616.0L + (long double)t[i];
    v = ldexpl(v, FIX_LSB_EXP);
    return (double)(neg ? -v : v);
}

typedef struct {
    int64_t exact[4][5];  /* 6 * (sum of component), fixed point as above */
    double sum[4];        /* sum of component (approximate) */
    double sumsq[4];      /* sum of squared component (FP64) */
    double cross_sb_gn;   /* sum of scale_bias * grid_noise (FP64) */
    int64_t n_elems, n_deadzone, n_clipped;
} orc_err_stats;

int orc_error_decompose(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                        orc_err_stats* out) {
    if (cols % 32 != 0) return -1;
    memset(out, 0, sizeof *out);
    /* Per-row partial results, combined afterwards in row order so that the
     * FP64 sums do not depend on the number of threads. */
    typedef struct {
        uint64_t fix[4][FIX_LIMBS];
        double sq[4], cross;
        int64_t ndz, nclip;
    } row_part;
    row_part* parts = (row_part*)calloc((size_t)(rows > 0 ? rows : 1), sizeof(row_part));
    if (!parts) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        row_part* p = &parts[r];
        for (int64_t b = 0; b < cols / 32; ++b) {
            const uint16_t* xb = x + r * ldx + b * 32;
            float amax = 0.0f;
            for (int k = 0; k < 32; ++k)
                if (absf_bf16(xb[k]) > amax) amax = absf_bf16(xb[k]);
            int e = orc_mx_exponent(amax);
            for (int k = 0; k < 32; ++k) {
                double c6[4];
                int dz;
                float xv = orc_bf16_value(xb[k]);
                decompose_elem(xv, amax, e, c6, &dz);
                p->ndz += dz;
                if (fabs((double)xv) > 6.0 * ldexp(1.0, e)) ++p->nclip;
                for (int c = 0; c < 4; ++c) {
                    fix_add(p->fix[c], c6[c]);
                    double cv = c6[c] / 6.0;
                    p->sq[c] += cv * cv;
                }
                p->cross += (c6[1] / 6.0) * (c6[3] / 6.0);
            }
        }
    }
    uint64_t tot[4][FIX_LIMBS];
    memset(tot, 0, sizeof tot);
    for (int64_t r = 0; r < rows; ++r) {
        for (int c = 0; c < 4; ++c) {
            fix_add_fix(tot[c], parts[r].fix[c]);
            out->sumsq[c] += parts[r].sq[c];
        }
        out->cross_sb_gn += parts[r].cross;
        out->n_deadzone += parts[r].ndz;
        out->n_clipped += parts[r].nclip;
    }
    free(parts);
    for (int c = 0; c < 4; ++c) {
        for (int i = 0; i < FIX_LIMBS; ++i) out->exact[c][i] = (int64_t)tot[c][i];
        out->sum[c] = fix_to_double(tot[c]) / 6.0;
    }
    out->n_elems = rows * cols;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* The three-way decomposition with the NVFP4 quantizer                      */
/* ------------------------------------------------------------------------ */

/*
 * The split above, applied to NVFP4 (16-element blocks, E4M3 block scale,
 * FP32 tensor scale): per block with amax A, the quantizer's own code g of
 * each element (orc_quantize, one group), its block scale value sb and the
 * tensor scale t give Q_s(x) = g sb t, the dequantized value (exact real
 * product); the ideal scale is again s* = A/6, so Q*(x) is the E2M1 point
 * nearest to 6|x|/A times A/6.  Components as for MXFP4; an element is
 * clipped when |x| > 6 sb t.  Times 6, the terms 6x, 6 g sb t and g* A are
 * exact in FP64.  The sums add each term to the fixed point on its own, so
 * they are exact whenever every term is a multiple of 2^-136, which holds
 * for a tensor amax of at least 2^-89 (then t >= 2^-101); a smaller tensor
 * returns -2.
 */
static double nv_qstar6(double ax, double A, double sgn) {
    int best = 0;
    if (A > 0.0) {
        double best_d = fabs(6.0 * ax - E2M1_GRID[0] * A);
        for (int c = 1; c < 8; ++c) {
            double d = fabs(6.0 * ax - E2M1_GRID[c] * A);
            if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
                best = c;
                best_d = d;
            }
        }
    }
    return sgn * E2M1_GRID[best] * A;
}

/* The terms of element (r, c): x6 = 6x, qs6 = 6 Q_s(x), qst6 = 6 Q*(x),
 * and s6 = 6 sb t, the largest value the block can represent; returns the
 * code magnitude g (0..7). */
static int nv_terms(const uint16_t* x, int64_t ldx, const uint8_t* q, const uint8_t* sc, float t,
                    int64_t cols, int64_t r, int64_t c, double* x6, double* qs6, double* qst6,
                    double* s6) {
    const uint16_t* xb = x + r * ldx + (c / 16) * 16;
    float A = 0.0f;
    for (int k = 0; k < 16; ++k)
        if (absf_bf16(xb[k]) > A) A = absf_bf16(xb[k]);
    const uint16_t h = x[r * ldx + c];
    const float xv = orc_bf16_value(h);
    const double sgn = (h & 0x8000u) ? -1.0 : 1.0;
    const uint8_t byte = q[r * (cols / 2) + c / 2];
    const int g = ((c & 1) ? (byte >> 4) : (byte & 15)) & 7;
    const double sb = orc_e4m3_value(sc[r * (cols / 16) + c / 16]);
    *x6 = 6.0 * (double)xv;
    *qs6 = sgn * 6.0 * E2M1_GRID[g] * sb * (double)t;
    *qst6 = nv_qstar6(fabs((double)xv), (double)A, sgn);
    *s6 = 6.0 * sb * (double)t;
    return g;
}

static int nv_quantize_all(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t** q, uint8_t** sc, float* t) {
    *q = (uint8_t*)malloc((size_t)(rows * cols / 2 + 1));
    *sc = (uint8_t*)malloc((size_t)(rows * cols / 16 + 1));
    if (!*q || !*sc) return -1;
    return orc_quantize(ORC_NVFP4, x, rows, cols, ldx, NULL, 1, NULL, 0, *q, *sc, t, NULL);
}

/* Per-element components times 6, NVFP4: out[4][rows*cols] (FP64
 * differences of the exact terms). */
int orc_error_components_nv(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                            double* out) {
    if (cols % 16 != 0) return -1;
    uint8_t *q = NULL, *sc = NULL;
    float t = 1.0f;
    int rc = nv_quantize_all(x, rows, cols, ldx, &q, &sc, &t);
    const int64_t n = rows * cols;
    for (int64_t r = 0; rc == 0 && r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double x6, qs6, qst6, s6;
            const int g = nv_terms(x, ldx, q, sc, t, cols, r, c, &x6, &qs6, &qst6, &s6);
            const int64_t i = r * cols + c;
            out[0 * n + i] = x6 - qs6;
            out[1 * n + i] = g ? qst6 - qs6 : 0.0;
            out[2 * n + i] = g ? 0.0 : x6;
            out[3 * n + i] = g ? x6 - qst6 : 0.0;
        }
    free(q);
    free(sc);
    return rc;
}

/* 1 if v is a multiple of 2^-136 (or zero), so the fixed point holds it. */
static int fix_exact(double v) {
    if (v == 0.0) return 1;
    return ldexp(v, -FIX_LSB_EXP) == floor(ldexp(v, -FIX_LSB_EXP));
}

static void fix_neg(uint64_t a[FIX_LIMBS]) {
    unsigned __int128 c = 1;
    for (int i = 0; i < FIX_LIMBS; ++i) {
        c += (unsigned __int128)(~a[i]);
        a[i] = (uint64_t)c;
        c >>= 64;
    }
}

int orc_error_decompose_nv(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                           orc_err_stats* out) {
    if (cols % 16 != 0) return -1;
    memset(out, 0, sizeof *out);
    uint8_t *q = NULL, *sc = NULL;
    float t = 1.0f;
    if (nv_quantize_all(x, rows, cols, ldx, &q, &sc, &t) != 0) {
        free(q);
        free(sc);
        return -1;
    }
    /* term sums: S[0] = sum of 6x where g == 0, S[1] = sum of 6x where g != 0,
     * S[2] = sum of 6 Q*(x) where g != 0, S[3] = sum of 6 Q_s(x); per row,
     * then combined in row order (the fixed-point sums are exact in any
     * order; the FP64 statistics then do not depend on the thread count) */
    typedef struct {
        uint64_t S[4][FIX_LIMBS];
        double sq[4], cross;
        int64_t ndz, nclip;
        int bad;
    } nv_row;
    nv_row* parts = (nv_row*)calloc((size_t)(rows > 0 ? rows : 1), sizeof(nv_row));
    if (!parts) {
        free(q);
        free(sc);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        nv_row* p = &parts[r];
        for (int64_t c = 0; c < cols; ++c) {
            double x6, qs6, qst6, s6;
            const int g = nv_terms(x, ldx, q, sc, t, cols, r, c, &x6, &qs6, &qst6, &s6);
            if (!fix_exact(x6) || !fix_exact(qs6) || !fix_exact(qst6)) {
                p->bad = 1;
                break;
            }
            fix_add(p->S[g ? 1 : 0], x6);
            if (g) fix_add(p->S[2], qst6);
            fix_add(p->S[3], qs6);
            const double xv = x6 / 6.0;
            if (g == 0 && xv != 0.0) ++p->ndz;
            if (fabs(xv) > s6) ++p->nclip;   /* |x| above 6 sb t */
            const double ct = (x6 - qs6) / 6.0;
            const double csb = g ? (qst6 - qs6) / 6.0 : 0.0;
            const double cdz = g ? 0.0 : xv;
            const double cgn = g ? (x6 - qst6) / 6.0 : 0.0;
            p->sq[0] += ct * ct;
            p->sq[1] += csb * csb;
            p->sq[2] += cdz * cdz;
            p->sq[3] += cgn * cgn;
            p->cross += csb * cgn;
        }
    }
    uint64_t S[4][FIX_LIMBS];
    memset(S, 0, sizeof S);
    double sq[4] = {0, 0, 0, 0}, cross = 0.0;
    int64_t ndz = 0, nclip = 0;
    int ok = 1;
    for (int64_t r = 0; r < rows; ++r) {
        if (parts[r].bad) ok = 0;
        for (int k = 0; k < 4; ++k) {
            fix_add_fix(S[k], parts[r].S[k]);
            sq[k] += parts[r].sq[k];
        }
        cross += parts[r].cross;
        ndz += parts[r].ndz;
        nclip += parts[r].nclip;
    }
    free(parts);
    free(q);
    free(sc);
    if (!ok) return -2;
    /* total = S0 + S1 - S3, scale_bias = S2 - S3, deadzone = S0, grid_noise = S1 - S2 */
    uint64_t tot[4][FIX_LIMBS], neg3[FIX_LIMBS], neg2[FIX_LIMBS];
    memcpy(neg3, S[3], sizeof neg3);
    fix_neg(neg3);
    memcpy(neg2, S[2], sizeof neg2);
    fix_neg(neg2);
    memcpy(tot[0], S[0], sizeof tot[0]);
    fix_add_fix(tot[0], S[1]);
    fix_add_fix(tot[0], neg3);
    memcpy(tot[1], S[2], sizeof tot[1]);
    fix_add_fix(tot[1], neg3);
    memcpy(tot[2], S[0], sizeof tot[2]);
    memcpy(tot[3], S[1], sizeof tot[3]);
    fix_add_fix(tot[3], neg2);
    for (int c = 0; c < 4; ++c) {
        for (int i = 0; i < FIX_LIMBS; ++i) out->exact[c][i] = (int64_t)tot[c][i];
        out->sum[c] = fix_to_double(tot[c]) / 6.0;
        out->sumsq[c] = sq[c];
    }
    out->cross_sb_gn = cross;
    out->n_elems = rows * cols;
    out->n_deadzone = ndz;
    out->n_clipped = nclip;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Outlier Fallback ("Decomposing MXFP4 quantization error ...", abstract:   */
/* the fallback recovers the deadzone entries)                               */
/* ------------------------------------------------------------------------ */

/* The page names the correction and what it recovers, not its mechanics.
 * Reading: the entries the quantizer sends to zero -- code magnitude 0, the
 * deadzone set D of the three-way split -- fall back to their own BF16
 * value; every other entry is dequantized from its code and block scale
 * (one quantization group, orc_quantize's codes):
 *   out = x                  where the code magnitude is 0
 *   out = e2m1(code) * 2^e   (MXFP4)
 *   out = (e2m1(code) * sb) * t   (NVFP4: FP32, first product exact; the
 *                                  same value the quantizer's residual
 *                                  subtracts)
 * out is FP32 [rows, cols] (row stride cols); *n_fallback receives the
 * number of entries with x != 0 that fell back (the deadzone count).
 * Returns 0, or -1 for a shape the formats do not allow. */
int orc_qdq_fallback(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                     float* out, int64_t* n_fallback) {
    const int blk = (fmt == ORC_NVFP4) ? 16 : 32;
    if ((fmt != ORC_NVFP4 && fmt != ORC_MXFP4) || cols % blk != 0 || rows < 0) return -1;
    uint8_t* q = (uint8_t*)malloc((size_t)(rows > 0 ? rows : 1) * (size_t)(cols / 2));
    uint8_t* sc = (uint8_t*)malloc((size_t)(rows > 0 ? rows : 1) * (size_t)(cols / blk));
    if (!q || !sc) {
        free(q);
        free(sc);
        return -1;
    }
    float t = 1.0f;
    if (orc_quantize(fmt, x, rows, cols, ldx, NULL, 1, NULL, 0, q, sc,
                     fmt == ORC_NVFP4 ? &t : NULL, NULL) != 0) {
        free(q);
        free(sc);
        return -1;
    }
    int64_t nfb = 0;
#pragma omp parallel for schedule(static) reduction(+ : nfb)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            const uint8_t byte = q[r * (cols / 2) + c / 2];
            const uint8_t code = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
            const uint16_t h = x[r * ldx + c];
            const float xv = orc_bf16_value(h);
            float v;
            if ((code & 7) == 0) {
                v = xv;                        /* fallback: the entry itself */
                if (xv != 0.0f) ++nfb;
            } else {
                const uint8_t s = sc[r * (cols / blk) + c / blk];
                const float g = (float)orc_e2m1_value(code);
                if (fmt == ORC_NVFP4)
                    v = (g * (float)orc_e4m3_value(s)) * t;
                else
                    v = (float)((double)g * orc_e8m0_value(s));
            }
            out[r * cols + c] = v;
        }
    }
    free(q);
    free(sc);
    if (n_fallback) *n_fallback = nfb;
    return 0;
}
