/*
 * rdg_oracle.c -- the CPU oracle for one GPU's share of a DeepSeek-V3-style
 * MoE layer (route -> EPLB remap -> dispatch layout -> expert FFN -> combine).
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load this library.  It
 * shares no code, header, table or constant generator with the HIP path.
 *
 * Style: plain loops, fp64 wherever the pages fix no precision, one function
 * per step of the method, each citing the passage it follows.  Page names:
 *   [LEP]  "Large-scale EP: DeepEP, EPLB and two-batch overlap" (SGLang
 *          handbook chapter), self-test answers and the EPLB paragraph.
 *   [SBO]  "Single Batch Overlap (SBO): Overlaping of Down GEMM with Combine
 *          Send" (DeepGEMM pull request), sections 2 and 3.
 *   [H100] "SGLang open-sources the first DeepSeek-V3/R1 H100 deployment"
 *          (Chinese article), sections "DeepEP-based EP", "DeepGEMM
 *          integration", "EPLB".
 *   [DEEP] "DeepEP, fully taken apart" (Chinese deep-dive), sections "EP:
 *          spreading experts over GPUs", "How large is the traffic",
 *          "group-limited gating", "why is combine slower than dispatch",
 *          "limitations".
 * Where the pages leave a constant open (scoring function, group score,
 * renormalisation, fp8 scale rule) the oracle follows the definitions
 * of the synthetic workloads and states the reading inline.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math),
 * so that every float operation below is one IEEE-754 operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ECAPACITY (-2)

/* ORC_FP8_UE8M0: e4m3 codes whose block scales are powers of two (an 8-bit
 * exponent-only scale; the variant of the block-scaled fp8 GEMM that scaled
 * matrix instructions consume directly) */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2, ORC_FP8_UE8M0 = 3 };

static int is_fp8(int dt) { return dt == ORC_FP8 || dt == ORC_FP8_UE8M0; }
enum { ORC_CONTIGUOUS = 0, ORC_MASKED = 1 };

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel loops that follow (n >= 1); for timing the
 * oracle single-threaded.  Returns the previous count. */
int orc_set_num_threads(int n) {
    int old = orc_num_threads();
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return old;
}

/* ------------------------------------------------------------------------
 * Number formats.
 * ------------------------------------------------------------------------ */

/* bf16 -> value: bf16 is the upper half of an IEEE binary32. */
double orc_bf16_decode(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* value -> bf16, round to nearest, ties to even, done from the definition:
 * bf16 keeps 8 significant bits; its quantum for |v| in [2^e, 2^(e+1)) is
 * 2^(e-7), and below 2^-126 the quantum is fixed at 2^-133.  nearbyint()
 * under the default rounding mode rounds half to even.  Finite inputs only. */
uint16_t orc_bf16_encode(double v) {
    double a = fabs(v), q, r;
    int e;
    if (v != v) return 0x7FC0;
    if (a < ldexp(1.0, -126)) {
        q = ldexp(1.0, -133);
    } else {
        frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1) */
        q = ldexp(1.0, e - 8); /* 8 significant bits */
    }
    r = nearbyint(a / q) * q;  /* a/q is exact: q is a power of two */
    {
        float f = (float)r;    /* r has <= 8 significant bits: exact in fp32 */
        uint32_t u;
        if (v < 0 || (v == 0 && signbit(v))) f = -f;
        memcpy(&u, &f, 4);
        return (uint16_t)(u >> 16);
    }
}

/* OCP fp8 e4m3fn, from the format definition: sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6);
 * S.1111.111 is NaN; there is no infinity; the largest finite value is
 * 1.75 * 2^8 = 448. */
double orc_fp8_decode(uint8_t c) {
    int s = c >> 7, ex = (c >> 3) & 15, m = c & 7;
    double v;
    if (ex == 15 && m == 7) return NAN;
    if (ex == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, ex - 7);
    return s ? -v : v;
}

/* value -> e4m3fn, round to nearest, ties to even, from the definition:
 * the format keeps 4 significant bits; for |v| in [2^e, 2^(e+1)), e >= -6,
 * the quantum is 2^(e-3), and below 2^-6 it is fixed at 2^-9 (subnormals).
 * The rounded magnitude is then written as sign, biased exponent, mantissa.
 * The caller clamps to [-448, 448] first (the scale rule guarantees it). */
uint8_t orc_fp8_encode(double v) {
    double a = fabs(v), q, r;
    int e, code;
    if (a < ldexp(1.0, -6)) {
        q = ldexp(1.0, -9);
    } else {
        frexp(a, &e);           /* a = m * 2^e, m in [0.5, 1): |v| in [2^(e-1), 2^e) */
        q = ldexp(1.0, e - 4);  /* 4 significant bits */
    }
    r = nearbyint(a / q) * q;   /* exact scaling by a power of two; half to even */
    if (r < ldexp(1.0, -6)) {
        code = (int)(r / ldexp(1.0, -9));          /* subnormal: m * 2^-9, m = 0..7 */
    } else {
        frexp(r, &e);                              /* r in [2^(e-1), 2^e) */
        code = ((e - 1 + 7) << 3) | (int)(ldexp(r, -(e - 1)) * 8.0 - 8.0);
    }
    if (v < 0 || (v == 0 && signbit(v))) code |= 0x80;
    return (uint8_t)code;
}

/* Scale of an fp8 block whose largest magnitude is amax (1 for an all-zero
 * block).  fp32 form: amax / 448, an fp32 division.  Power-of-two form: the
 * smallest 2^k with amax / 2^k <= 448, found by exact comparisons of amax
 * with 448 * 2^k, with k kept in [-126, 127] (a normal fp32, and within the
 * 8-bit exponent-only scale's range). */
static float fp8_block_scale(float amax, int pow2) {
    int k;
    if (!(amax > 0.0f)) return 1.0f;
    if (!pow2) return amax / 448.0f;
    frexp((double)amax / 448.0, &k);          /* a first guess */
    while (k > -126 && ldexp(448.0, k - 1) >= (double)amax) --k;
    while (ldexp(448.0, k) < (double)amax) ++k;
    if (k < -126) k = -126;
    return (float)ldexp(1.0, k);
}

/* Block quantiser (the "1d2d" format of the masked fp8 grouped GEMM,
 * [SBO] section 3: 1-D activation scales, 2-D weight scales).  Reading of
 * the open constants: fp32 scale s = amax / 448 over the block (s = 1 when
 * the block is all zero), or with pow2 the power-of-two scale above;
 * code = RNE(clamp(v / s, -448, 448)), the division done in fp32.  Blocks
 * are block_rows x 128 (1 x 128 for activations, 128 x 128 for weights).
 * src_dt: ORC_F32 or ORC_BF16; rows, cols row-major.  Scales are
 * [ceil(rows/block_rows), cols/128] row-major. */
static int quantize_fp8(const void* src, int src_dt, int rows, int cols, int block_rows, int pow2,
                        uint8_t* q, float* scales) {
    int nbr, nbc;
    if (cols % 128 != 0 || rows <= 0 || block_rows <= 0) return ORC_EINVAL;
    nbr = (rows + block_rows - 1) / block_rows;
    nbc = cols / 128;
#pragma omp parallel for schedule(static)
    for (int br = 0; br < nbr; ++br) {
        for (int bc = 0; bc < nbc; ++bc) {
            int r0 = br * block_rows, r1 = r0 + block_rows, r, c;
            float amax = 0.0f, s;
            if (r1 > rows) r1 = rows;
            for (r = r0; r < r1; ++r)
                for (c = bc * 128; c < bc * 128 + 128; ++c) {
                    float v = src_dt == ORC_F32 ? ((const float*)src)[(size_t)r * cols + c]
                                                : (float)orc_bf16_decode(((const uint16_t*)src)[(size_t)r * cols + c]);
                    if (fabsf(v) > amax) amax = fabsf(v);
                }
            s = fp8_block_scale(amax, pow2);
            scales[(size_t)br * nbc + bc] = s;
            for (r = r0; r < r1; ++r)
                for (c = bc * 128; c < bc * 128 + 128; ++c) {
                    float v = src_dt == ORC_F32 ? ((const float*)src)[(size_t)r * cols + c]
                                                : (float)orc_bf16_decode(((const uint16_t*)src)[(size_t)r * cols + c]);
                    float t = v / s;
                    if (t > 448.0f) t = 448.0f;
                    if (t < -448.0f) t = -448.0f;
                    q[(size_t)r * cols + c] = orc_fp8_encode((double)t);
                }
        }
    }
    return ORC_OK;
}

int orc_quantize_fp8(const void* src, int src_dt, int rows, int cols, int block_rows, uint8_t* q,
                     float* scales) {
    return quantize_fp8(src, src_dt, rows, cols, block_rows, 0, q, scales);
}

int orc_quantize_fp8_ue8m0(const void* src, int src_dt, int rows, int cols, int block_rows, uint8_t* q,
                           float* scales) {
    return quantize_fp8(src, src_dt, rows, cols, block_rows, 1, q, scales);
}

/* ------------------------------------------------------------------------
 * Router score.  The pages say only that the router scores every expert
 * ([DEEP] "EP: spreading experts over GPUs"); the workload definition fixes
 * sigmoid scores.  Selection is an integer decided by floating point, so
 * both sides evaluate one fully specified sigmoid, in fp64 and rounded once
 * to fp32 (every step is a single IEEE-754 double operation):
 *   x (fp32) clamped to [-87, 87], widened to double; z = -x;
 *   n = rint(z * log2e)                    log2e = the double nearest 1/ln 2
 *   r = fma(-n, ln2_hi, z); r = fma(-n, ln2_lo, r)
 *         ln2_hi = the double ln 2 cut to 42 significant bits (n*ln2_hi is
 *         exact), ln2_lo = (double ln 2) - ln2_hi (exact)
 *   p = sum_{k=0..13} r^k / k!  by Horner with fma, 1/k! rounded to double
 *   e = p * 2^n (exact);  sigma = (float)(1 / (1 + e))
 * The truncation error of the degree-13 series on |r| <= ln2/2 is below
 * 2^-55 relative, so sigma is the correctly rounded fp32 value except where
 * the double lies within a few double ulps of an fp32 rounding boundary.
 * ------------------------------------------------------------------------ */
static double g_log2e, g_ln2_hi, g_ln2_lo, g_coef[14];
static int g_sig_init = 0;

static void orc_sigmoid_init(void) {
    double f = 1.0, ln2 = log(2.0);
    int k, ex;
    if (g_sig_init) return;
    g_log2e = 1.0 / ln2;
    frexp(ln2, &ex); /* ln2 = m * 2^ex, m in [0.5, 1) */
    g_ln2_hi = ldexp(floor(ldexp(ln2, 42 - ex)), ex - 42);
    g_ln2_lo = ln2 - g_ln2_hi;
    for (k = 0; k < 14; ++k) {
        if (k > 0) f *= (double)k;
        g_coef[k] = 1.0 / f;
    }
    g_sig_init = 1;
}

float orc_sigmoid(float xf) {
    double x, z, n, r, p, e;
    int k;
    orc_sigmoid_init();
    if (xf < -87.0f) xf = -87.0f;
    if (xf > 87.0f) xf = 87.0f;
    x = (double)xf;
    z = -x;
    n = rint(z * g_log2e);
    r = fma(-n, g_ln2_hi, z);
    r = fma(-n, g_ln2_lo, r);
    p = g_coef[13];
    for (k = 12; k >= 0; --k) p = fma(p, r, g_coef[k]);
    e = ldexp(p, (int)n);
    return (float)(1.0 / (1.0 + e));
}

/* The constants as bit patterns, so that a test can print and check them. */
void orc_sigmoid_constants(double* out) {
    int k;
    orc_sigmoid_init();
    out[0] = g_log2e;
    out[1] = g_ln2_hi;
    out[2] = g_ln2_lo;
    for (k = 0; k < 14; ++k) out[3 + k] = g_coef[k];
}

/* Apply the sigmoid to n values (used by the exhaustive accuracy sweep). */
void orc_sigmoid_many(const float* x, float* y, int64_t n) {
    orc_sigmoid_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = orc_sigmoid(x[i]);
}

/* Sweep every fp32 bit pattern in [lo_bits, hi_bits] (positive patterns)
 * and its negation with the given stride; return the worst error of the
 * sigmoid against 1/(1+exp(-x)) in fp64, in units of the fp32 ulp of the
 * reference, plus the count of monotonicity violations along the sweep. */
double orc_sigmoid_sweep(uint32_t lo_bits, uint32_t hi_bits, uint32_t stride, int64_t* n_checked,
                         int64_t* n_nonmono) {
    double worst = 0.0;
    int64_t cnt = 0, nonmono = 0;
    orc_sigmoid_init();
#pragma omp parallel for schedule(dynamic, 4096) reduction(max : worst) reduction(+ : cnt, nonmono)
    for (int64_t b = lo_bits; b <= (int64_t)hi_bits; b += stride) {
        int sgn;
        for (sgn = 0; sgn < 2; ++sgn) {
            uint32_t u = (uint32_t)b | (sgn ? 0x80000000u : 0u), u2;
            float x, x2, y, y2;
            double ref, ulp, err;
            int ex;
            memcpy(&x, &u, 4);
            y = orc_sigmoid(x);
            ref = 1.0 / (1.0 + exp(-(double)x));
            frexp(ref, &ex);
            ulp = ldexp(1.0, ex - 24);
            if (ref < ldexp(1.0, -126)) ulp = ldexp(1.0, -149);
            err = fabs((double)y - ref) / ulp;
            if (err > worst) worst = err;
            ++cnt;
            /* monotone non-decreasing: compare with the next larger float */
            x2 = nextafterf(x, INFINITY);
            memcpy(&u2, &x2, 4);
            (void)u2;
            y2 = orc_sigmoid(x2);
            if (y2 < y) ++nonmono;
        }
    }
    *n_checked = cnt;
    *n_nonmono = nonmono;
    return worst;
}

/* ------------------------------------------------------------------------
 * Group-limited top-k gating ([DEEP] "group-limited gating": experts are
 * split into groups, the router first keeps the best groups and then picks
 * the top-K experts inside them; [DEEP] "EP": each token picks K experts and
 * its output is the routing-weighted sum of their FFN outputs).
 * Readings: groups are n_group runs of N/n_group consecutive expert ids;
 * a group's score is the fp32 sum of its two largest sigmoid scores (the
 * single score when a group has one expert); ties go to the lower index
 * everywhere; slot k holds the k-th expert in (score desc, id asc) order;
 * the weights are the selected scores renormalised to sum to `scale`.
 * With a selection bias (a variant not on the pages: a per-expert correction
 * added for the choice only), the group scores and the top-K use the fp32
 * sums score + bias, and the weights still renormalise the plain scores.
 * ------------------------------------------------------------------------ */
static int route_impl(const float* logits, const float* bias, int B, int N, int n_group, int topk_group, int K,
                      float scale, int32_t* ids, float* w) {
    if (B < 0 || N <= 0 || n_group <= 0 || N % n_group != 0 || topk_group <= 0 || topk_group > n_group ||
        K <= 0 || K > topk_group * (N / n_group))
        return ORC_EINVAL;
#pragma omp parallel
    {
        float* s = (float*)malloc(sizeof(float) * N);
        float* sel = (float*)malloc(sizeof(float) * N);  /* the choosing score */
        float* gsc = (float*)malloc(sizeof(float) * n_group);
        char* gsel = (char*)malloc(n_group);
        char* esel = (char*)malloc(N);
        int gs = N / n_group;
#pragma omp for schedule(static)
        for (int t = 0; t < B; ++t) {
            int e, j, r, k;
            double sum = 0.0;
            for (e = 0; e < N; ++e) {
                s[e] = orc_sigmoid(logits[(size_t)t * N + e]);
                sel[e] = bias ? s[e] + bias[e] : s[e];
            }
            /* group score: top-1 + top-2 (with multiplicity) */
            for (j = 0; j < n_group; ++j) {
                int i1 = -1, i2 = -1;
                for (e = j * gs; e < (j + 1) * gs; ++e)
                    if (i1 < 0 || sel[e] > sel[i1]) i1 = e;
                for (e = j * gs; e < (j + 1) * gs; ++e)
                    if (e != i1 && (i2 < 0 || sel[e] > sel[i2])) i2 = e;
                gsc[j] = i2 >= 0 ? sel[i1] + sel[i2] : sel[i1];
                gsel[j] = 0;
            }
            /* keep topk_group groups: largest score, lowest index on ties */
            for (r = 0; r < topk_group; ++r) {
                int best = -1;
                for (j = 0; j < n_group; ++j)
                    if (!gsel[j] && (best < 0 || gsc[j] > gsc[best])) best = j;
                gsel[best] = 1;
            }
            /* top-K experts inside the kept groups */
            for (e = 0; e < N; ++e) esel[e] = 0;
            for (k = 0; k < K; ++k) {
                int best = -1;
                for (e = 0; e < N; ++e)
                    if (gsel[e / gs] && !esel[e] && (best < 0 || sel[e] > sel[best])) best = e;
                esel[best] = 1;
                ids[(size_t)t * K + k] = best;
            }
            for (k = 0; k < K; ++k) sum += (double)s[ids[(size_t)t * K + k]];
            for (k = 0; k < K; ++k)
                w[(size_t)t * K + k] = (float)((double)s[ids[(size_t)t * K + k]] / sum * (double)scale);
        }
        free(s);
        free(sel);
        free(gsc);
        free(gsel);
        free(esel);
    }
    return ORC_OK;
}

int orc_route(const float* logits, int B, int N, int n_group, int topk_group, int K, float scale,
              int32_t* ids, float* w) {
    return route_impl(logits, NULL, B, N, n_group, topk_group, K, scale, ids, w);
}

int orc_route_biased(const float* logits, const float* bias, int B, int N, int n_group, int topk_group, int K,
                     float scale, int32_t* ids, float* w) {
    return route_impl(logits, bias, B, N, n_group, topk_group, K, scale, ids, w);
}

/* ------------------------------------------------------------------------
 * EPLB logical -> physical remap ([LEP] EPLB paragraph and self-test answer
 * 3: 256 logical experts in 288 physical slots, popular experts replicated
 * and each copy taking a share of the traffic; [H100] "EPLB").
 * Reading: the replica for token g of logical expert e is
 * log2phy[e][g mod n_replica[e]]; the rank keeps the rows whose physical id
 * lies in [phys_begin, phys_begin + n_local) and renumbers them from 0.
 * Input id -1 (row not sent here) stays -1.
 * ------------------------------------------------------------------------ */
int orc_eplb_remap(const int32_t* ids, const int64_t* gidx, int T, int K, const int32_t* log2phy,
                   const int32_t* n_replica, int r_max, int n_logical, int phys_begin, int n_local,
                   int32_t* local_ids) {
    int t, k;
    for (t = 0; t < T; ++t)
        for (k = 0; k < K; ++k) {
            int32_t e = ids[(size_t)t * K + k], out = -1;
            if (e >= 0) {
                int32_t p;
                if (e >= n_logical || n_replica[e] < 1 || n_replica[e] > r_max) return ORC_EINVAL;
                p = log2phy[(size_t)e * r_max + (int)(gidx[t] % n_replica[e])];
                if (p >= phys_begin && p < phys_begin + n_local) out = p - phys_begin;
            }
            local_ids[(size_t)t * K + k] = out;
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Dispatch layout ([LEP] self-test answer 1 and the DeepEP-modes paragraph:
 * the contiguous layout needs a permute that orders tokens by expert, the
 * masked layout keeps fixed shapes and marks the valid rows; [H100]
 * "DeepGEMM integration": contiguous for prefill, masked for decode;
 * [H100] "DeepEP-based EP": exceeding a preallocated fixed buffer is a
 * runtime error).
 * Flat row index i = t*K + k.  Readings: rows of one expert keep flat-index
 * order (a stable counting sort); contiguous segments are padded to block_m;
 * masked rows at rank >= m_max are dropped and flagged ECAPACITY with the
 * largest count as detail; a contiguous layout that exceeds m_cap drops the
 * rows past it and flags ECAPACITY with the needed row count.
 * Outputs: counts[n_local], offsets[n_local+1], masked_m[n_local] (rows kept
 * per expert, for both kinds), pos[T*K] (-1: not local / dropped),
 * row_src[m_cap] (-1: padding).  Returns the status; *detail as above.
 * ------------------------------------------------------------------------ */
int orc_layout(const int32_t* ids, int T, int K, int n_local, int kind, int block_m, int m_max, int m_cap,
               int32_t* counts, int32_t* offsets, int32_t* masked_m, int32_t* pos, int32_t* row_src,
               int32_t* detail) {
    int64_t n = (int64_t)T * K, i;
    int e, status = ORC_OK;
    int32_t worst = 0;
    if (n_local <= 0 || (kind == ORC_CONTIGUOUS && block_m <= 0) || (kind == ORC_MASKED && m_max <= 0))
        return ORC_EINVAL;
    if (kind == ORC_MASKED && (int64_t)n_local * m_max != m_cap) return ORC_EINVAL;
    *detail = 0;
    for (e = 0; e < n_local; ++e) counts[e] = 0;
    for (i = 0; i < n; ++i)
        if (ids[i] >= 0 && ids[i] < n_local) counts[ids[i]]++;
    offsets[0] = 0;
    for (e = 0; e < n_local; ++e) {
        int32_t seg = kind == ORC_MASKED ? m_max : ((counts[e] + block_m - 1) / block_m) * block_m;
        offsets[e + 1] = offsets[e] + seg;
        masked_m[e] = counts[e];
        if (kind == ORC_MASKED && counts[e] > m_max) {
            masked_m[e] = m_max;
            status = ORC_ECAPACITY;
        }
        if (counts[e] > worst) worst = counts[e];
    }
    if (kind == ORC_CONTIGUOUS && offsets[n_local] > m_cap) {
        status = ORC_ECAPACITY;
        *detail = offsets[n_local];
        for (e = 0; e < n_local; ++e) {
            int32_t room = m_cap - offsets[e];
            if (room < 0) room = 0;
            if (masked_m[e] > room) masked_m[e] = room;
        }
    } else if (status == ORC_ECAPACITY) {
        *detail = worst;
    }
    for (i = 0; i < m_cap; ++i) row_src[i] = -1;
    for (e = 0; e < n_local; ++e) {
        int32_t rank = 0;
        for (i = 0; i < n; ++i) {
            if (ids[i] != e) continue;
            if (rank < masked_m[e]) {
                pos[i] = offsets[e] + rank;
                row_src[offsets[e] + rank] = (int32_t)i;
            } else {
                pos[i] = -1;
            }
            ++rank;
        }
    }
    for (i = 0; i < n; ++i)
        if (!(ids[i] >= 0 && ids[i] < n_local)) pos[i] = -1;
    return status;
}

/* ------------------------------------------------------------------------
 * Expert FFN on one input row (gate/up projection, SiLU-gated product, down
 * projection; the pages call it the expert FFN, [DEEP] "EP").  Weights are
 * K-major ("nt"): W1, W3 are [I, H], W2 is [H, I].
 * Dot products accumulate in fp64 over exact images of the stored operands.
 * For fp8, each 128-long block dot is exact in fp64 and is then multiplied
 * by the activation block scale and the 128x128 weight block scale ([SBO]
 * section 3, "1d2d").  The intermediate h and the output y are rounded the
 * way the kernel stores them: h to fp32 / bf16 / (fp8 + 1x128 scales), y to
 * fp32 (fp32 layer) or bf16.  y_out receives the stored (rounded) values.
 * ------------------------------------------------------------------------ */
static double load_elem(int dt, const void* p, size_t idx) {
    if (dt == ORC_F32) return (double)((const float*)p)[idx];
    if (dt == ORC_BF16) return orc_bf16_decode(((const uint16_t*)p)[idx]);
    return orc_fp8_decode(((const uint8_t*)p)[idx]);
}

static double round_store(int dt, double v) {
    if (dt == ORC_F32) return (double)(float)v;
    return orc_bf16_decode(orc_bf16_encode(v));
}

/* y[j] = sum_k W[j][k] * a[k] for a [rows_w, K] weight matrix; fp8 uses the
 * block-scaled form with a_s[K/128] and w_s[rows_w/128][K/128]. */
static void matvec(int dt, int rows_w, int Kd, const void* W, const float* w_s, const double* a,
                   const float* a_s, double* y) {
    int j, k, b;
    for (j = 0; j < rows_w; ++j) {
        double acc = 0.0;
        if (!is_fp8(dt)) {
            for (k = 0; k < Kd; ++k) acc += load_elem(dt, W, (size_t)j * Kd + k) * a[k];
        } else {
            for (b = 0; b < Kd / 128; ++b) {
                double part = 0.0; /* exact: fp8 x fp8 products, 128 terms */
                for (k = b * 128; k < b * 128 + 128; ++k) part += load_elem(dt, W, (size_t)j * Kd + k) * a[k];
                acc += part * (double)a_s[b] * (double)w_s[(size_t)(j / 128) * (Kd / 128) + b];
            }
        }
        y[j] = acc;
    }
}

/* a_row: H elements of the row's input in dtype dt (fp8: codes) with
 * a_scales[H/128] for fp8.  Scratch: 3*I + H doubles. */
static void expert_ffn_row(int dt, int H, int I, const void* a_row, const float* a_scales, const void* W1,
                           const void* W3, const void* W2, const float* s1, const float* s3, const float* s2,
                           double* scratch, double* y_out) {
    double* a = scratch;       /* H */
    double* g = a + H;         /* I */
    double* u = g + I;         /* I */
    double* h = u + I;         /* I */
    float hs[64];              /* I/128 <= 64 block scales of h */
    int k, i, b;
    for (k = 0; k < H; ++k) a[k] = load_elem(dt, a_row, k);
    matvec(dt, I, H, W1, s1, a, a_scales, g);
    matvec(dt, I, H, W3, s3, a, a_scales, u);
    for (i = 0; i < I; ++i) {
        double sg = 1.0 / (1.0 + exp(-g[i]));
        h[i] = g[i] * sg * u[i];
    }
    if (dt == ORC_F32) {
        for (i = 0; i < I; ++i) h[i] = (double)(float)h[i];
    } else if (dt == ORC_BF16) {
        for (i = 0; i < I; ++i) h[i] = orc_bf16_decode(orc_bf16_encode(h[i]));
    } else {
        /* re-quantise h with 1x128 blocks from its fp32 image (same rule as
         * the block quantiser, in the layer's scale form); the codes are kept
         * as values in h */
        for (b = 0; b < I / 128; ++b) {
            float amax = 0.0f, s;
            for (i = b * 128; i < b * 128 + 128; ++i)
                if (fabsf((float)h[i]) > amax) amax = fabsf((float)h[i]);
            s = fp8_block_scale(amax, dt == ORC_FP8_UE8M0);
            hs[b] = s;
            for (i = b * 128; i < b * 128 + 128; ++i) {
                float t = (float)h[i] / s;
                if (t > 448.0f) t = 448.0f;
                if (t < -448.0f) t = -448.0f;
                h[i] = orc_fp8_decode(orc_fp8_encode((double)t));
            }
        }
    }
    if (is_fp8(dt)) {
        /* y = W2 . h with h as fp8 codes and scales hs */
        int j;
        for (j = 0; j < H; ++j) {
            double acc = 0.0;
            for (b = 0; b < I / 128; ++b) {
                double part = 0.0;
                for (i = b * 128; i < b * 128 + 128; ++i) part += load_elem(dt, W2, (size_t)j * I + i) * h[i];
                acc += part * (double)hs[b] * (double)s2[(size_t)(j / 128) * (I / 128) + b];
            }
            y_out[j] = round_store(ORC_BF16, acc);
        }
    } else {
        matvec(dt, H, I, W2, NULL, h, NULL, y_out);
        for (k = 0; k < H; ++k) y_out[k] = round_store(dt, y_out[k]);
    }
}

/* ------------------------------------------------------------------------
 * The MoE layer by definition ([DEEP] "EP": out = weighted sum over the
 * token's K experts of their FFN outputs; [DEEP] "why is combine slower":
 * combine multiplies by the top-k weights and accumulates; [DEEP]
 * "limitations": bf16 pre-reduction loses precision, so the sum here is
 * fp64 in k order and rounded once).
 *   out[t] = shared(x_t) + sum_{k : local_ids[t,k] >= 0} w[t,k] * FFN_e(x_t)
 * Only the tokens listed in sel (n_sel of them) are computed; out is
 * [n_sel, H] in out_dt (fp32 or bf16 bits).  Per local expert e the weight
 * pointers W1[e], W3[e], W2[e] (and fp8 scales) may be NULL when no selected
 * token uses e.  sh_* describe the shared expert (NULL: none) with its own
 * intermediate size sh_I; it runs on every selected token and is added
 * unweighted.  y_rows (optional, [n_sel, K, H] doubles) receives the stored
 * expert outputs, 0 for rows that are not local.
 * ------------------------------------------------------------------------ */
int orc_moe_layer(int dt, int H, int I, int K, const void* x, const float* x_scales, const int32_t* local_ids,
                  const float* topk_w, const void* const* W1, const void* const* W3, const void* const* W2,
                  const float* const* s1, const float* const* s3, const float* const* s2, const void* shW1,
                  const void* shW3, const void* shW2, const float* shs1, const float* shs3, const float* shs2,
                  int sh_I, const int32_t* sel, int n_sel, int out_dt, void* out, double* y_rows) {
    size_t esz = dt == ORC_F32 ? 4 : (dt == ORC_BF16 ? 2 : 1);
    int maxI = I > sh_I ? I : sh_I;
    if (H <= 0 || I <= 0 || K <= 0 || dt < ORC_F32 || dt > ORC_FP8_UE8M0 ||
        (is_fp8(dt) && (H % 128 || I % 128 || maxI > 64 * 128)))
        return ORC_EINVAL;
#pragma omp parallel
    {
        double* scratch = (double*)malloc(sizeof(double) * (3 * (size_t)maxI + H));
        double* y = (double*)malloc(sizeof(double) * H);
        double* acc = (double*)malloc(sizeof(double) * H);
#pragma omp for schedule(dynamic, 1)
        for (int si = 0; si < n_sel; ++si) {
            int t = sel[si], k, j;
            const void* a_row = (const char*)x + (size_t)t * H * esz;
            const float* a_s = is_fp8(dt) ? x_scales + (size_t)t * (H / 128) : NULL;
            for (j = 0; j < H; ++j) acc[j] = 0.0;
            if (shW1) {
                expert_ffn_row(dt, H, sh_I, a_row, a_s, shW1, shW3, shW2, shs1, shs3, shs2, scratch, y);
                for (j = 0; j < H; ++j) acc[j] += y[j];
            }
            for (k = 0; k < K; ++k) {
                int32_t e = local_ids[(size_t)t * K + k];
                if (e < 0) {
                    if (y_rows)
                        for (j = 0; j < H; ++j) y_rows[((size_t)si * K + k) * H + j] = 0.0;
                    continue;
                }
                expert_ffn_row(dt, H, I, a_row, a_s, W1[e], W3[e], W2[e], is_fp8(dt) ? s1[e] : NULL,
                               is_fp8(dt) ? s3[e] : NULL, is_fp8(dt) ? s2[e] : NULL, scratch, y);
                if (y_rows)
                    for (j = 0; j < H; ++j) y_rows[((size_t)si * K + k) * H + j] = y[j];
                for (j = 0; j < H; ++j) acc[j] += (double)topk_w[(size_t)t * K + k] * y[j];
            }
            for (j = 0; j < H; ++j) {
                if (out_dt == ORC_F32) ((float*)out)[(size_t)si * H + j] = (float)acc[j];
                else ((uint16_t*)out)[(size_t)si * H + j] = orc_bf16_encode(acc[j]);
            }
        }
        free(scratch);
        free(y);
        free(acc);
    }
    return ORC_OK;
}

/* Combine over a layout ([DEEP] "EP" and "why is combine slower"): the
 * same weighted sum, but reading expert outputs from their layout rows,
 * y_perm[pos[t,k]] (bf16 or fp32 per y_dt), and optionally adding a shared
 * output row.  Used to pin the layout path against the definition path. */
int orc_combine(int y_dt, const void* y_perm, const int32_t* pos, const float* topk_w, int T, int K, int H,
                const void* shared_out, int out_dt, void* out) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        int j, k;
        for (j = 0; j < H; ++j) {
            double acc = 0.0;
            if (shared_out)
                acc += out_dt == ORC_F32 ? (double)((const float*)shared_out)[(size_t)t * H + j]
                                         : orc_bf16_decode(((const uint16_t*)shared_out)[(size_t)t * H + j]);
            for (k = 0; k < K; ++k) {
                int32_t p = pos[(size_t)t * K + k];
                double v;
                if (p < 0) continue;
                v = y_dt == ORC_F32 ? (double)((const float*)y_perm)[(size_t)p * H + j]
                                    : orc_bf16_decode(((const uint16_t*)y_perm)[(size_t)p * H + j]);
                acc += (double)topk_w[(size_t)t * K + k] * v;
            }
            if (out_dt == ORC_F32) ((float*)out)[(size_t)t * H + j] = (float)acc;
            else ((uint16_t*)out)[(size_t)t * H + j] = orc_bf16_encode(acc);
        }
    }
    return ORC_OK;
}
