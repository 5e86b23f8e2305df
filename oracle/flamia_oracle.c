/*
 * flamia_oracle.c -- plain FP64 CPU oracle for causal, packed, variable-length
 * attention over microscaled E4M3 operands (the FLAMIA method).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is used by the test-suite, by the
 * package's smoke check and by the benchmark's CPU-baseline leg.  The HIP
 * library never links, loads or calls it, and it shares no code, header or
 * table with the HIP sources.  Everything here is written from the method's
 * description, slow and direct on purpose, so that it can be read against it.
 *
 * Sources (pages and sections):
 *   [R]  "FLAMIA ... technical review" (zhongzhuzhou.org, 2026-11-08)
 *        S2  "Prerequisites"           attention, backward products, D identity,
 *                                       online softmax recurrence
 *        S3  "Reusable scales"         document-local 32-token blocks, one
 *                                       exponent over the block x full head dim
 *        S4  "A causal mask must include scale selection"
 *                                       conservative (ceil) exponent, 448 bound,
 *                                       floor rule as the leaking alternative,
 *                                       causal dQ accumulator prescale
 *        S5  "Reconstructing the forward in the backward", Algorithm 1,
 *                                       "A range budget for probability
 *                                       quantization" (boost 256)
 *        S6  "Packed documents and GPU scheduling" (+inf LSE sentinel,
 *                                       masked keys outside the document)
 *        S3  "Rotation, range, and the alternative", Algorithm 1 step 02
 *                                       (Hadamard rotation of Q and K per token)
 *   [K]  jaehun.me review of arXiv 2611.03344, S1.2 (S, P, O and the five
 *        backward products), S2 (floor-rule group exponent), S3.1-S3.3
 *        (32x32 dS blocks, per-query-row dS exponent option, D from the
 *        quantized dO), S3.4 (Hadamard rotation: dot products preserved,
 *        no mixing across positions).
 *   [F]  richardcheam.github.io "efficient execution", "Attention without the
 *        score matrix" (blockwise online softmax), "Lower precision" (E4M3
 *        OCP max 448).
 *
 * Readings where the pages are silent or garbled (their formulas were lost in
 * extraction) are listed in the repository's design notes; the ones that
 * change arithmetic are restated next to the code that implements them.
 *
 * Comparisons with an FP32 implementation: a GPU evaluates scores and dP in
 * its own precision, so an element of P^ or dS^ lying that close to an E4M3
 * rounding midpoint may round either way, and both are results of the
 * method.  The last section of this file ("Evaluation-noise bookkeeping")
 * says which elements, and to what, for an evaluation error the caller
 * states; it recomputes what it needs and is kept apart from the arithmetic
 * above it, which never depends on the device.
 *
 * Parity pins: every function here is pinned by tests under tests/ that check
 * it against values the pages print, closed forms, invariants or brute force.
 * The dQ prescale exponent (orc_bwd_prep, kpre) has no printed value on the
 * pages (its formula is lost): it is pinned by its bound on every partial sum
 * and, from both sides, by a worst-case input that reaches the bound.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EBADSEQ (-1)
#define ORC_EBADARG (-2)

/* Threads the oracle's parallel loops use. */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------- */
/* Number formats                                                             */
/* ------------------------------------------------------------------------- */

/* Nearest integer to a non-negative q, ties to the even integer. */
static double rne_nonneg(double q)
{
    double f = floor(q);
    double r = q - f;
    if (r > 0.5) return f + 1.0;
    if (r < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* OCP E4M3FN ([F] "Lower precision": max 448; spacing 0.125 just above 1):
 * bias 7, subnormals m/8 * 2^-6, largest finite 1.75 * 2^8 = 448 (0x7E);
 * 0x7F / 0xFF are NaN and never produced.  Round to nearest, ties to even,
 * saturating to +-448; the sign is kept, so -0 encodes as 0x80. */
uint8_t orc_e4m3_encode(double y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs(y);
    uint8_t mag;
    if (a >= 448.0) {
        mag = 0x7E;
    } else if (a < ldexp(1.0, -6)) {
        /* subnormal lattice: integer multiples of 2^-9; 8 * 2^-9 is the
           smallest normal, whose code is 0x08, so the count is the code */
        mag = (uint8_t)rne_nonneg(ldexp(a, 9));
    } else {
        int E;
        frexp(a, &E);
        E -= 1; /* a in [2^E, 2^(E+1)) */
        double q = rne_nonneg(ldexp(a, 3 - E)); /* in [8, 16] */
        if (q == 16.0) {
            q = 8.0;
            E += 1;
        }
        mag = (uint8_t)(((E + 7) << 3) | ((int)q - 8));
    }
    return (uint8_t)(sign | mag);
}

/* IEEE binary16 rounding of a double (the dQ accumulator's format, [R] S4
 * "Forward locality and backward locality differ": a five-bit exponent):
 * nearest value with ties to the even significand; normals carry 10
 * fraction bits from 2^-14 up, subnormals are multiples of 2^-24, and
 * magnitudes from 65520 (half way between the largest finite value 65504 and
 * the next power of two) on round to infinity.  The sign is kept. */
double orc_f16_round(double x)
{
    double a = fabs(x);
    double r;
    if (isnan(x)) return x;
    if (a >= 65520.0) {
        r = INFINITY;
    } else if (a < ldexp(1.0, -14)) {
        r = ldexp(rne_nonneg(ldexp(a, 24)), -24);
    } else {
        int E;
        frexp(a, &E);
        E -= 1; /* a in [2^E, 2^(E+1)) */
        r = ldexp(rne_nonneg(ldexp(a, 10 - E)), E - 10);
    }
    return signbit(x) ? -r : r;
}

double orc_e4m3_decode(uint8_t c)
{
    int E = (c >> 3) & 15, M = c & 7;
    double v = (E == 0) ? ldexp((double)M, -9) : ldexp((double)(8 + M), E - 10);
    return (c & 0x80) ? -v : v;
}

double orc_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double to bfloat16 (8 significant bits, FP32 exponent range),
 * nearest, ties to even. */
uint16_t orc_f64_to_bf16(double x)
{
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int E;
    frexp(a, &E);
    E -= 1;
    int qexp = (E < -126 ? -126 : E) - 7; /* weight of the last kept bit */
    double v = ldexp(rne_nonneg(ldexp(a, -qexp)), qexp);
    if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float f = (float)v; /* exact: v lies on the bf16 lattice */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

void orc_f64_to_bf16_array(int64_t n, const double* x, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(x[i]);
}

/* Conservative exponent ([R] S4 "Why doubling the scale often preserves E4M3
 * values"; [K] S3.2): the smallest integer e with amax / 2^e <= 448.
 * With amax = m * 2^E, m in [1, 2), and 448 = 1.75 * 2^8 this is
 * E - 8 + [m > 1.75].  A zero block takes e = 0 (a conventional finite scale).
 * The result is clamped to the UE8M0 range [-127, 127]. */
int orc_ceil_exponent(double amax)
{
    if (!(amax > 0.0)) return 0;
    int E;
    double f = frexp(amax, &E); /* amax = f * 2^E, f in [0.5, 1) */
    double m = 2.0 * f;
    E -= 1;
    int e = E - 8 + (m > 1.75 ? 1 : 0);
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* The floor rule of the reference MX conversion ([K] S2): e = floor(log2
 * amax) - 8, where 8 is E4M3's largest exponent.  It can push amax / 2^e past
 * 448, and is kept only as a negative control for the causality tests. */
int orc_floor_exponent(double amax)
{
    if (!(amax > 0.0)) return 0;
    int E;
    frexp(amax, &E);
    E -= 1;
    int e = E - 8;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Smallest E4M3 value >= t for t in (0, 448]; 448 when t > 448. */
static double e4m3_ceil_value(double t)
{
    for (int c = 1; c <= 0x7E; ++c) {
        double v = orc_e4m3_decode((uint8_t)c);
        if (v >= t) return v;
    }
    return 448.0;
}

/* ------------------------------------------------------------------------- */
/* Packed-document helpers                                                    */
/* ------------------------------------------------------------------------- */

/* cu_seqlens must start at 0, never decrease and end at or below T. */
int orc_check_seqlens(int T, int B, const int32_t* cu)
{
    if (B < 1 || T < 0) return ORC_EBADSEQ;
    if (cu[0] != 0) return ORC_EBADSEQ;
    for (int b = 0; b < B; ++b)
        if (cu[b + 1] < cu[b]) return ORC_EBADSEQ;
    if (cu[B] > T) return ORC_EBADSEQ;
    return ORC_OK;
}

/* Document holding token t, or -1 for padding rows (t >= cu[B]). */
static int doc_of(int B, const int32_t* cu, int t)
{
    if (t < 0 || t >= cu[B]) return -1;
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    while (cu[lo + 1] <= t) ++lo; /* skip empty documents */
    return lo;
}

/* ------------------------------------------------------------------------- */
/* Token-block quantizer ([R] S3; [K] S3.1)                                   */
/* ------------------------------------------------------------------------- */

/* x: bf16 [T][H][d].  For every head and every document-local block of at most
 * `block` consecutive tokens (blocks start at each document start; the last
 * one may be partial), one exponent e over the block's tokens x all d
 * features; codes = E4M3(x * 2^-e); exps[h][t] = e + 127 replicated on every
 * token of the block (dense per-token scale table, [R] S6).
 * block = 32 is the default policy, block = 1 the per-token exact option.
 * rule 0: conservative ceil exponent; rule 1: floor exponent (control only).
 * Padding rows: codes 0, exponent byte 127. */
/* The token-block rule over one tensor whose values are either bf16 bits (xb)
 * or FP32 (xf, the rotated score operands). */
static int quantize_impl(int T, int B, const int32_t* cu, int H, int d, const uint16_t* xb,
                         const float* xf, int block, int rule, uint8_t* codes, uint8_t* exps)
{
    if (orc_check_seqlens(T, B, cu) != ORC_OK) return ORC_EBADSEQ;
    if (H < 1 || d < 1 || block < 1) return ORC_EBADARG;
    memset(codes, 0, (size_t)T * H * d);
    memset(exps, 127, (size_t)H * T);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int h = 0; h < H; ++h) {
        for (int b = 0; b < B; ++b) {
            for (int s0 = cu[b]; s0 < cu[b + 1]; s0 += block) {
                int s1 = s0 + block < cu[b + 1] ? s0 + block : cu[b + 1];
                double amax = 0.0;
                for (int t = s0; t < s1; ++t)
                    for (int c = 0; c < d; ++c) {
                        size_t k = ((size_t)t * H + h) * d + c;
                        double v = fabs(xb ? orc_bf16_to_f64(xb[k]) : (double)xf[k]);
                        if (v > amax) amax = v;
                    }
                int e = rule == 0 ? orc_ceil_exponent(amax) : orc_floor_exponent(amax);
                for (int t = s0; t < s1; ++t) {
                    exps[(size_t)h * T + t] = (uint8_t)(e + 127);
                    for (int c = 0; c < d; ++c) {
                        size_t k = ((size_t)t * H + h) * d + c;
                        double v = xb ? orc_bf16_to_f64(xb[k]) : (double)xf[k];
                        codes[k] = orc_e4m3_encode(ldexp(v, -e));
                    }
                }
            }
        }
    }
    return ORC_OK;
}

int orc_quantize(int T, int B, const int32_t* cu, int H, int d, const uint16_t* x, int block,
                 int rule, uint8_t* codes, uint8_t* exps)
{
    return quantize_impl(T, B, cu, H, d, x, NULL, block, rule, codes, exps);
}

/* The same rule over FP32 values (the rotated Q and K of the score path). */
int orc_quantize_f32(int T, int B, const int32_t* cu, int H, int d, const float* x, int block,
                     int rule, uint8_t* codes, uint8_t* exps)
{
    return quantize_impl(T, B, cu, H, d, NULL, x, block, rule, codes, exps);
}

/* ------------------------------------------------------------------------- */
/* Hadamard rotation of the score operands ([R] S3 "Rotation, range, and the  */
/* alternative", Algorithm 1 step 02; [K] S3.4 "Hadamard rotation").          */
/* ------------------------------------------------------------------------- */

/* Every row (token, head) of x, bf16 [T][H][d] with d a power of two, times
 * the Sylvester Hadamard matrix H_d (entries (-1)^popcount(i & j), so that
 * H_d H_d = d I; the 1/sqrt(d) normalisation is left to the softmax scale and
 * the gradient un-rotation, where it is a power of two: q_r . k_r = d q . k).
 * Computed as the fast Walsh-Hadamard transform in FP32: stages h = 1, 2, 4,
 * ..., d/2 in that order, each replacing the pair (a, b) = (x[i], x[i + h]),
 * i & h == 0, by (a + b, a - b).  FP32 because the rotated values decide the
 * E4M3 codes, and the kernel forms them in FP32 in the same order. */
int orc_hadamard_rotate(int T, int H, int d, const uint16_t* x, float* out)
{
    if (T < 0 || H < 1 || d < 1 || (d & (d - 1)) != 0) return ORC_EBADARG;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < (int64_t)T * H; ++r) {
        float* y = out + (size_t)r * d;
        for (int c = 0; c < d; ++c) y[c] = (float)orc_bf16_to_f64(x[(size_t)r * d + c]);
        for (int hh = 1; hh < d; hh <<= 1)
            for (int i = 0; i < d; ++i)
                if ((i & hh) == 0) {
                    float a = y[i], bb = y[i + hh];
                    y[i] = a + bb;
                    y[i + hh] = a - bb;
                }
    }
    return ORC_OK;
}

/* Dequantized operand values: decode(code) * 2^(byte - 127), [T][H][d]. */
void orc_dequantize(int T, int H, int d, const uint8_t* codes, const uint8_t* exps, double* out)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < d; ++c) {
                size_t k = ((size_t)t * H + h) * d + c;
                out[k] = ldexp(orc_e4m3_decode(codes[k]), (int)exps[(size_t)h * T + t] - 127);
            }
}

/* ------------------------------------------------------------------------- */
/* E2M1 score view with an E4M3 scale per 16 in-token features ([R] S2 "Codes,
 * scales, and hardware layout"; [K] S3.1), without a tensor-level scale.     */
/* ------------------------------------------------------------------------- */

/* E2M1 magnitudes by code 0..7. */
static const double e2m1_val[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* |x| rounded to the E2M1 lattice scaled by s, nearest with ties to the even
 * code, by comparing |x| with the midpoints times s (exact products). */
static int e2m1_code(double ax, double s)
{
    int best = 7;
    for (int c = 0; c < 7; ++c) {
        double mid = 0.5 * (e2m1_val[c] + e2m1_val[c + 1]) * s;
        if (ax < mid) {
            best = c;
            break;
        }
        if (ax == mid) {
            best = (c % 2 == 0) ? c : c + 1;
            break;
        }
    }
    return best;
}

/* x bf16 [T][H][d] -> codes [T][H][d/2] (element 2k in the low nibble),
 * scales [T][H][d/16] E4M3.  The group scale is the smallest E4M3 value s
 * with amax / s <= 6 (the no-clipping rule applied to E2M1's maximum 6); a
 * zero group takes s = 1.  Padding rows are zero codes with scale 1. */
int orc_quantize_nvfp4(int T, int B, const int32_t* cu, int H, int d, const uint16_t* x,
                       uint8_t* codes, uint8_t* scales)
{
    if (orc_check_seqlens(T, B, cu) != ORC_OK) return ORC_EBADSEQ;
    if (d % 16 != 0) return ORC_EBADARG;
    memset(codes, 0, (size_t)T * H * (d / 2));
    for (size_t i = 0; i < (size_t)T * H * (d / 16); ++i) scales[i] = orc_e4m3_encode(1.0);
#pragma omp parallel for schedule(static)
    for (int t = 0; t < cu[B]; ++t) {
        for (int h = 0; h < H; ++h) {
            for (int g = 0; g < d / 16; ++g) {
                const uint16_t* xs = x + ((size_t)t * H + h) * d + 16 * g;
                double amax = 0.0;
                for (int c = 0; c < 16; ++c) {
                    double v = fabs(orc_bf16_to_f64(xs[c]));
                    if (v > amax) amax = v;
                }
                double s = amax > 0.0 ? e4m3_ceil_value(amax / 6.0) : 1.0;
                scales[((size_t)t * H + h) * (d / 16) + g] = orc_e4m3_encode(s);
                for (int c = 0; c < 16; ++c) {
                    double v = orc_bf16_to_f64(xs[c]);
                    int code = e2m1_code(fabs(v), s) | (signbit(v) ? 8 : 0);
                    size_t k = ((size_t)t * H + h) * (d / 2) + 8 * g + c / 2;
                    codes[k] |= (uint8_t)(c % 2 == 0 ? code : code << 4);
                }
            }
        }
    }
    return ORC_OK;
}

/* Dequantized E2M1 view: code value times its group's E4M3 scale, [T][H][d]. */
void orc_dequantize_nvfp4(int T, int H, int d, const uint8_t* codes, const uint8_t* scales,
                          double* out)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < d; ++c) {
                uint8_t byte = codes[((size_t)t * H + h) * (d / 2) + c / 2];
                int code = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
                double v = e2m1_val[code & 7] *
                           orc_e4m3_decode(scales[((size_t)t * H + h) * (d / 16) + c / 16]);
                out[((size_t)t * H + h) * d + c] = (code & 8) ? -v : v;
            }
}

/* ------------------------------------------------------------------------- */
/* Attention on dequantized operands                                          */
/* ------------------------------------------------------------------------- */

typedef struct {
    int T, B, Hq, Hkv, d, causal;
    const int32_t* cu;
    double scale;             /* softmax scale applied to Q.K */
    const double *Q, *K, *V;  /* dequantized operands, [T][H][d] */
    const double *Qs, *Ks;    /* score view of Q and K (NULL: Q and K) */
} orc_attn;

static inline int kv_head(const orc_attn* a, int h) { return h * a->Hkv / a->Hq; }

static inline const double* row(const double* X, int H, int d, int t, int h)
{
    return X + ((size_t)t * H + h) * d;
}

/* Score s_ij = scale * Q_i . K_j ([R] S2; [K] S1.2).  With a separate score
 * view (the E2M1 route) the score uses it ([R] S2: the mixed route
 * reconstructs scores from the selected Q/K format and re-quantizes Q and K
 * in E4M3 for the gradient products). */
static double score(const orc_attn* a, int h, int i, int j)
{
    const double* q = row(a->Qs ? a->Qs : a->Q, a->Hq, a->d, i, h);
    const double* k = row(a->Ks ? a->Ks : a->K, a->Hkv, a->d, j, kv_head(a, h));
    double acc = 0.0;
    for (int c = 0; c < a->d; ++c) acc += q[c] * k[c];
    return a->scale * acc;
}

/* Visible keys of query i in document b: [s_b, i] when causal, else the whole
 * document ([R] S2: the keys in that document up through i). */
static inline int key_end(const orc_attn* a, int b, int i)
{
    return a->causal ? i + 1 : a->cu[b + 1];
}

/* E4M3 value nearest to y (the rounding of orc_e4m3_encode, decoded). */
static double e4m3_round(double y) { return orc_e4m3_decode(orc_e4m3_encode(y)); }

/* ------------------------------------------------------------------------- */
/* Forward                                                                    */
/* ------------------------------------------------------------------------- */

/* One query row.  mode:
 *   0  microscaled forward, rounded normaliser: base-2 logits s2 = s*log2(e);
 *      integer row reference r = ceil(max s2); unnormalised weights
 *      p = 2^(s2 - r) <= 1; probability operand P^ = E4M3(256 p) / 256 (the
 *      boost 256 of [R] S5 "A range budget"); l = sum P^; O = sum P^ V / l;
 *      LSE = (r + log2 l) ln 2.
 *   1  as 0 with the unrounded normaliser l = sum p.
 *   3  the same microscaled forward following the tile loop of the review's
 *      Algorithm 1 (steps 04-08): over document-local key tiles of `kblock`
 *      keys, the row reference r rises to ceil(max s2) of the keys seen so far;
 *      when it rises, l and the accumulator are multiplied by the exact power
 *      of two 2^(r_old - r_new); each tile's weights are rounded against the
 *      current r, P^ = E4M3(256 * 2^(s2 - r)) / 256, and added to l and to the
 *      accumulator.  Equal to mode 0 except for weights that are E4M3
 *      subnormal (256 p < 2^-6) against one of the references.
 *   2  reference math: blockwise online softmax in FP64 over document-local
 *      key blocks of `kblock` keys ([R] S2 "Why flash tiling recomputes
 *      scores"; [F] "Attention without the score matrix"): running max m,
 *      normaliser l and accumulator, rescaled by exp(m_old - m_new) whenever
 *      the max grows; O = acc / l; LSE = m + ln l.
 * Rows outside every document get O = 0 and LSE = +inf ([R] S6). */
static void fwd_row(const orc_attn* a, int mode, int kblock, int h, int i, double* O, double* LSE,
                    int32_t* n_rescale, double* s_buf)
{
    int d = a->d, g = kv_head(a, h);
    int b = doc_of(a->B, a->cu, i);
    for (int c = 0; c < d; ++c) O[c] = 0.0;
    if (n_rescale) *n_rescale = 0;
    if (b < 0) {
        *LSE = INFINITY;
        return;
    }
    int j0 = a->cu[b], j1 = key_end(a, b, i);
    for (int j = j0; j < j1; ++j) s_buf[j - j0] = score(a, h, i, j);

    if (mode == 0 || mode == 1) {
        double mx = -INFINITY;
        for (int j = j0; j < j1; ++j)
            if (s_buf[j - j0] * M_LOG2E > mx) mx = s_buf[j - j0] * M_LOG2E;
        double r = ceil(mx);
        double l = 0.0;
        for (int j = j0; j < j1; ++j) {
            double p = exp2(s_buf[j - j0] * M_LOG2E - r);
            double ph = e4m3_round(256.0 * p) / 256.0;
            l += (mode == 0) ? ph : p;
            const double* v = row(a->V, a->Hkv, d, j, g);
            for (int c = 0; c < d; ++c) O[c] += ph * v[c];
        }
        for (int c = 0; c < d; ++c) O[c] /= l;
        *LSE = (r + log2(l)) * M_LN2;
        return;
    }

    if (mode == 3) {
        double r = -INFINITY, l = 0.0;
        for (int k0 = j0; k0 < j1; k0 += kblock) {
            int k1 = k0 + kblock < j1 ? k0 + kblock : j1;
            double mb = -INFINITY;
            for (int j = k0; j < k1; ++j)
                if (s_buf[j - j0] * M_LOG2E > mb) mb = s_buf[j - j0] * M_LOG2E;
            double r_new = ceil(mb) > r ? ceil(mb) : r;
            if (r != -INFINITY && r_new > r) {
                double alpha = exp2(r - r_new);
                l *= alpha;
                for (int c = 0; c < d; ++c) O[c] *= alpha;
                if (n_rescale) ++*n_rescale;
            }
            r = r_new;
            for (int j = k0; j < k1; ++j) {
                double ph = e4m3_round(256.0 * exp2(s_buf[j - j0] * M_LOG2E - r)) / 256.0;
                const double* v = row(a->V, a->Hkv, d, j, g);
                l += ph;
                for (int c = 0; c < d; ++c) O[c] += ph * v[c];
            }
        }
        for (int c = 0; c < d; ++c) O[c] /= l;
        *LSE = (r + log2(l)) * M_LN2;
        return;
    }

    /* mode 2: online recurrence over document-local key blocks */
    double m = -INFINITY, l = 0.0;
    int nres = 0;
    for (int k0 = j0; k0 < j1; k0 += kblock) {
        int k1 = k0 + kblock < j1 ? k0 + kblock : j1;
        double mb = -INFINITY;
        for (int j = k0; j < k1; ++j)
            if (s_buf[j - j0] > mb) mb = s_buf[j - j0];
        double m_new = mb > m ? mb : m;
        if (m != -INFINITY && m_new > m) {
            double alpha = exp(m - m_new);
            l *= alpha;
            for (int c = 0; c < d; ++c) O[c] *= alpha;
            ++nres;
        }
        for (int j = k0; j < k1; ++j) {
            double w = exp(s_buf[j - j0] - m_new);
            l += w;
            const double* v = row(a->V, a->Hkv, d, j, g);
            for (int c = 0; c < d; ++c) O[c] += w * v[c];
        }
        m = m_new;
    }
    for (int c = 0; c < d; ++c) O[c] /= l;
    *LSE = m + log(l);
    if (n_rescale) *n_rescale = nres;
}

static int check_attn_args(int T, int B, const int32_t* cu, int Hq, int Hkv, int d)
{
    if (orc_check_seqlens(T, B, cu) != ORC_OK) return ORC_EBADSEQ;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || d < 1) return ORC_EBADARG;
    return ORC_OK;
}

/* Q, K, V: dequantized operands; Qs, Ks: optional score view (else NULL).
 * rows: n_rows pairs (h, t); NULL means every (h, t).  O: [T][Hq][d],
 * LSE: [Hq][T], n_rescale: [Hq][T] or NULL.  Unlisted rows are untouched. */
int orc_attn_fwd(int T, int B, const int32_t* cu, int Hq, int Hkv, int d, double scale,
                 int causal, const double* Q, const double* K, const double* V, const double* Qs,
                 const double* Ks, int mode, int kblock, int64_t n_rows, const int32_t* rows,
                 double* O, double* LSE, int32_t* n_rescale)
{
    if (check_attn_args(T, B, cu, Hq, Hkv, d) != ORC_OK) return ORC_EBADARG;
    if (kblock < 1 || mode < 0 || mode > 3) return ORC_EBADARG;
    orc_attn a = {T, B, Hq, Hkv, d, causal, cu, scale, Q, K, V, Qs, Ks};
    int64_t n = rows ? n_rows : (int64_t)Hq * T;
    int Tn = T > 0 ? T : 1;
#pragma omp parallel
    {
        double* s_buf = (double*)malloc(sizeof(double) * Tn);
#pragma omp for schedule(dynamic, 4)
        for (int64_t k = 0; k < n; ++k) {
            int h = rows ? rows[2 * k] : (int)(k / Tn);
            int t = rows ? rows[2 * k + 1] : (int)(k % Tn);
            fwd_row(&a, mode, kblock, h, t, O + ((size_t)t * Hq + h) * d, LSE + (size_t)h * T + t,
                    n_rescale ? n_rescale + (size_t)h * T + t : NULL, s_buf);
        }
        free(s_buf);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Backward                                                                   */
/* ------------------------------------------------------------------------- */

/* Backward preparation ([R] Algorithm 1 steps "Encode G once; compute D from
 * reconstructed G and saved O" and "Select ... causal row dQ accumulator
 * boosts"; [K] S3.3):
 *   - dO (bf16 [T][Hq][d]) is quantized with the operand rule (block 32 or the
 *     per-token option);
 *   - D_i = dO^_i . O_i with the dequantized dO and the saved bf16 O;
 *   - kpre_i, the power-of-two prescale exponent of row i's FP16 dQ partials,
 *     the stylised boost 2^floor(log2(target / estimate)) of [R] S4 with
 *     target 2^14 and an estimate built only from what row i may see ([R] S4
 *     "Forward locality and backward locality differ": the row's own dO and
 *     running maxima of the visible key and value magnitudes).  Reading: with
 *     e_dO the row's dO exponent and maxV, maxK the largest V and K exponents
 *     over the visible keys, every partial sum of dQ_i is bounded by
 *         2 * scale * d * 448^3 * 2^(e_dO + maxV + maxK),
 *     and the estimate is twice that (a factor 2 of margin), so
 *         kpre_i = 14 - C - (e_dO + maxV + maxK),
 *         C = ceil(log2(4 * scale * d * 448^3)).
 *     Clamped to [-60, 60]; 0 for padding rows and rows whose quantized dO is
 *     all zero.  The pages' own formula is lost; the rule is pinned by its
 *     bound and by a worst-case input that reaches it. */
int orc_bwd_prep(int T, int B, const int32_t* cu, int Hq, int Hkv, int d, double scale,
                 int causal, int block, const uint16_t* dO, const uint16_t* O, const uint8_t* ke,
                 const uint8_t* ve, uint8_t* do_codes, uint8_t* do_exps, double* D, int32_t* kpre)
{
    if (Hkv < 1 || Hq % Hkv != 0) return ORC_EBADARG;
    int rc = orc_quantize(T, B, cu, Hq, d, dO, block, 0, do_codes, do_exps);
    if (rc != ORC_OK) return rc;
    int C = (int)ceil(log2(4.0 * scale * d * 448.0 * 448.0 * 448.0));
    /* largest V and K exponents over the keys each row may see: a running
       maximum along each document (causal), or the document maximum */
    int* vis_v = (int*)malloc(sizeof(int) * ((size_t)Hkv * T + 1));
    int* vis_k = (int*)malloc(sizeof(int) * ((size_t)Hkv * T + 1));
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int g = 0; g < Hkv; ++g) {
        for (int b = 0; b < B; ++b) {
            int mv = -1000, mk = -1000;
            for (int j = cu[b]; j < cu[b + 1]; ++j) {
                int ev = (int)ve[(size_t)g * T + j] - 127, ek = (int)ke[(size_t)g * T + j] - 127;
                if (ev > mv) mv = ev;
                if (ek > mk) mk = ek;
                if (causal) {
                    vis_v[(size_t)g * T + j] = mv;
                    vis_k[(size_t)g * T + j] = mk;
                }
            }
            if (!causal)
                for (int j = cu[b]; j < cu[b + 1]; ++j) {
                    vis_v[(size_t)g * T + j] = mv;
                    vis_k[(size_t)g * T + j] = mk;
                }
        }
    }
#pragma omp parallel for collapse(2) schedule(dynamic, 64)
    for (int h = 0; h < Hq; ++h) {
        for (int t = 0; t < T; ++t) {
            int g = h * Hkv / Hq;
            int b = doc_of(B, cu, t);
            size_t r = (size_t)t * Hq + h;
            if (b < 0) {
                D[(size_t)h * T + t] = 0.0;
                kpre[(size_t)h * T + t] = 0;
                continue;
            }
            double acc = 0.0;
            int nonzero = 0;
            int eg = (int)do_exps[(size_t)h * T + t] - 127;
            for (int c = 0; c < d; ++c) {
                double g_hat = ldexp(orc_e4m3_decode(do_codes[r * d + c]), eg);
                acc += g_hat * orc_bf16_to_f64(O[r * d + c]);
                if (g_hat != 0.0) nonzero = 1;
            }
            D[(size_t)h * T + t] = acc;
            int E = eg + vis_v[(size_t)g * T + t] + vis_k[(size_t)g * T + t];
            int k = 14 - C - E;
            if (k < -60) k = -60;
            if (k > 60) k = 60;
            kpre[(size_t)h * T + t] = nonzero ? k : 0;
        }
    }
    free(vis_v);
    free(vis_k);
    return ORC_OK;
}

/* Sequence-wide dQ prescale (test-only negative control; [R] S4 "Forward
 * locality and backward locality differ" and [K] S3.3: the size estimate
 * taken from sequence-wide maxima of the dO, V and K magnitudes, which lets
 * a later token change the FP16 rounding of every earlier row).  Reading:
 * the same bound as the causal rule with every maximum taken over all tokens
 * of all documents (head h for dO, its kv head for V and K):
 *     kpre = 14 - C - (max e_dO + max e_V + max e_K),
 * clamped to [-60, 60], for every row of every document; 0 for padding rows.
 * do_exps: [Hq][T] (the dO exponents orc_bwd_prep returns). */
int orc_bwd_prescale_seq(int T, int B, const int32_t* cu, int Hq, int Hkv, int d, double scale,
                         const uint8_t* do_exps, const uint8_t* ke, const uint8_t* ve,
                         int32_t* kpre)
{
    if (orc_check_seqlens(T, B, cu) != ORC_OK) return ORC_EBADSEQ;
    if (Hkv < 1 || Hq % Hkv != 0) return ORC_EBADARG;
    int C = (int)ceil(log2(4.0 * scale * d * 448.0 * 448.0 * 448.0));
    int ntok = cu[B];
    for (int h = 0; h < Hq; ++h) {
        int g = h * Hkv / Hq;
        int mg = -1000, mv = -1000, mk = -1000;
        for (int t = 0; t < ntok; ++t) {
            int eg = (int)do_exps[(size_t)h * T + t] - 127;
            int ev = (int)ve[(size_t)g * T + t] - 127, ek = (int)ke[(size_t)g * T + t] - 127;
            mg = eg > mg ? eg : mg;
            mv = ev > mv ? ev : mv;
            mk = ek > mk ? ek : mk;
        }
        int k = 14 - C - (mg + mv + mk);
        if (k < -60) k = -60;
        if (k > 60) k = 60;
        for (int t = 0; t < T; ++t) kpre[(size_t)h * T + t] = t < ntok ? k : 0;
    }
    return ORC_OK;
}

typedef struct {
    const orc_attn* a;
    const double* G;   /* dequantized dO, [T][Hq][d] */
    const double* D;   /* [Hq][T] */
    const double* LSE; /* [Hq][T], natural log, as saved by a forward */
    int mode;          /* 0: E4M3 P^ and dS^; 1: reference math, no rounding */
    int per_row_ds;    /* dS exponent per (query row, key block) for dQ */
} orc_bwd;

/* One document-local 32x32 block (queries [q0,q1) x keys [k0,k1) of one
 * document, head h) of the recomputed backward ([R] Algorithm 1 steps
 * 11-15; [K] S1.2, S3.3), row-major [32][32] outputs:
 *   P   = exp(s_ij - LSE_i)       probabilities rebuilt from the saved LSE
 *   dP  = dO^_i . V^_j
 *   dS  = P (dP - D_i)
 *   Pq  the probability operand of dV: E4M3(256 P) / 256 (mode 0) or P;
 *   dSk dS quantized on the 32x32 block ([K] S3.1: one scale per 32x32 dS
 *       block, from the block's largest |dS| over visible entries, with the
 *       conservative exponent), used for dK, and for dQ unless per_row_ds;
 *   dSq with per_row_ds: dS quantized with one exponent per query row of the
 *       block (the per-query-row option, [R] S4, [K] S3.2), used for dQ.
 * Entries with j > i (causal) and entries outside the block are zero. */
static void bwd_block(const orc_bwd* w, int h, int q0, int q1, int k0, int k1, double* P,
                      double* dP, double* dS, double* Pq, double* dSk, double* dSq)
{
    const orc_attn* a = w->a;
    int T = a->T, d = a->d, g = kv_head(a, h);
    for (int k = 0; k < 1024; ++k) P[k] = dP[k] = dS[k] = Pq[k] = dSk[k] = dSq[k] = 0.0;
    double amax = 0.0;
    for (int i = q0; i < q1; ++i) {
        const double* gi = row(w->G, a->Hq, d, i, h);
        for (int j = k0; j < k1; ++j) {
            if (a->causal && j > i) continue;
            int e = (i - q0) * 32 + (j - k0);
            const double* vj = row(a->V, a->Hkv, d, j, g);
            P[e] = exp(score(a, h, i, j) - w->LSE[(size_t)h * T + i]);
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += gi[c] * vj[c];
            dP[e] = acc;
            dS[e] = P[e] * (dP[e] - w->D[(size_t)h * T + i]);
            if (fabs(dS[e]) > amax) amax = fabs(dS[e]);
            Pq[e] = w->mode == 0 ? e4m3_round(256.0 * P[e]) / 256.0 : P[e];
        }
    }
    int eb = orc_ceil_exponent(amax);
    for (int i = q0; i < q1; ++i) {
        int base = (i - q0) * 32;
        double ramax = 0.0;
        for (int j = k0; j < k1; ++j)
            if (fabs(dS[base + j - k0]) > ramax) ramax = fabs(dS[base + j - k0]);
        int er = orc_ceil_exponent(ramax);
        for (int j = k0; j < k1; ++j) {
            int e = base + (j - k0);
            if (a->causal && j > i) continue;
            if (w->mode == 0) {
                dSk[e] = ldexp(e4m3_round(ldexp(dS[e], -eb)), eb);
                dSq[e] = w->per_row_ds ? ldexp(e4m3_round(ldexp(dS[e], -er)), er) : dSk[e];
            } else {
                dSk[e] = dSq[e] = dS[e];
            }
        }
    }
}

static int check_blocks(int B, const int32_t* cu, int64_t n, const int32_t* blocks, int nheads)
{
    for (int64_t k = 0; k < n; ++k) {
        int b = doc_of(B, cu, blocks[2 * k + 1]);
        if (b < 0 || (blocks[2 * k + 1] - cu[b]) % 32 != 0) return ORC_EBADARG;
        if (blocks[2 * k] < 0 || blocks[2 * k] >= nheads) return ORC_EBADARG;
    }
    return ORC_OK;
}

/* Exposes one block of the recomputed backward (for the invariant checks). */
int orc_bwd_block(int T, int B, const int32_t* cu, int Hq, int Hkv, int d, double scale,
                  int causal, const double* Q, const double* K, const double* V,
                  const double* Qs, const double* Ks, const double* G, const double* D,
                  const double* LSE, int mode, int per_row_ds, int h, int q0, int k0, double* P,
                  double* dP, double* dS, double* Pq, double* dSk, double* dSq)
{
    if (check_attn_args(T, B, cu, Hq, Hkv, d) != ORC_OK) return ORC_EBADARG;
    int b = doc_of(B, cu, q0);
    if (b < 0 || doc_of(B, cu, k0) != b || (q0 - cu[b]) % 32 || (k0 - cu[b]) % 32 || h < 0 ||
        h >= Hq)
        return ORC_EBADARG;
    orc_attn a = {T, B, Hq, Hkv, d, causal, cu, scale, Q, K, V, Qs, Ks};
    orc_bwd w = {&a, G, D, LSE, mode, per_row_ds};
    int q1 = q0 + 32 < cu[b + 1] ? q0 + 32 : cu[b + 1];
    int k1 = k0 + 32 < cu[b + 1] ? k0 + 32 : cu[b + 1];
    bwd_block(&w, h, q0, q1, k0, k1, P, dP, dS, Pq, dSk, dSq);
    return ORC_OK;
}

/* dQ_i = scale * sum_j dS^_ij K^_j for every query of the listed
 * document-local 32-query blocks.  qblocks: n pairs (q head, t0), t0 the
 * first token of a block.  dQ: [T][Hq][d], accumulated into.
 * With kpre (int32 [Hq][T]) and dq16, also the method's FP16 accumulation of
 * dQ ([R] S4 and [K] S3.3: FP16 partials with a power-of-two row prescale):
 * per document-relative tile of `dq_tile` keys (a multiple of 32: the
 * implementation's key tile, as the forward's key step is a parameter) the
 * partial sum_j dS^_ij K^_j times 2^(kpre_i + f), where 2^f <= scale <
 * 2^(f + 1), is rounded to FP16 and added into an FP16 accumulator (rounded
 * again), tiles in key order; dq16 = accumulator * scale / 2^(kpre_i + f). */
int orc_bwd_dq(int T, int B, const int32_t* cu, int Hq, int Hkv, int d, double scale, int causal,
               const double* Q, const double* K, const double* V, const double* Qs,
               const double* Ks, const double* G, const double* D, const double* LSE, int mode,
               int per_row_ds, int64_t n, const int32_t* qblocks, double* dQ,
               const int32_t* kpre, double* dq16, int dq_tile)
{
    if (check_attn_args(T, B, cu, Hq, Hkv, d) != ORC_OK) return ORC_EBADARG;
    if (dq_tile < 32 || dq_tile % 32) return ORC_EBADARG;
    const int tile_blocks = dq_tile / 32;
    if (check_blocks(B, cu, n, qblocks, Hq) != ORC_OK) return ORC_EBADARG;
    orc_attn a = {T, B, Hq, Hkv, d, causal, cu, scale, Q, K, V, Qs, Ks};
    orc_bwd w = {&a, G, D, LSE, mode, per_row_ds};
    int fexp;
    frexp(scale, &fexp);
    fexp -= 1; /* 2^fexp <= scale < 2^(fexp + 1) */
#pragma omp parallel
    {
        double* buf = (double*)malloc(sizeof(double) * 6 * 1024);
        double* part = (double*)malloc(sizeof(double) * 32 * d);
        double* acc16 = (double*)malloc(sizeof(double) * 32 * d);
#pragma omp for schedule(dynamic)
        for (int64_t k = 0; k < n; ++k) {
            int h = qblocks[2 * k], q0 = qblocks[2 * k + 1];
            int b = doc_of(B, cu, q0), g = h * Hkv / Hq;
            int q1 = q0 + 32 < cu[b + 1] ? q0 + 32 : cu[b + 1];
            int kend = causal ? q1 : cu[b + 1];
            double *P = buf, *dP = buf + 1024, *dS = buf + 2048, *Pq = buf + 3072,
                   *dSk = buf + 4096, *dSq = buf + 5120;
            for (int x = 0; x < 32 * d; ++x) part[x] = acc16[x] = 0.0;
            for (int k0 = cu[b]; k0 < kend; k0 += 32) {
                int k1 = k0 + 32 < cu[b + 1] ? k0 + 32 : cu[b + 1];
                bwd_block(&w, h, q0, q1, k0, k1, P, dP, dS, Pq, dSk, dSq);
                for (int i = q0; i < q1; ++i) {
                    double* out = dQ + ((size_t)i * Hq + h) * d;
                    for (int c = 0; c < d; ++c) {
                        double acc = 0.0;
                        for (int j = k0; j < k1; ++j)
                            acc += dSq[(i - q0) * 32 + (j - k0)] * row(K, Hkv, d, j, g)[c];
                        out[c] += scale * acc;
                        part[(i - q0) * d + c] += acc;
                    }
                }
                /* the FP16 model: one partial per key tile */
                if (kpre && dq16 &&
                    (((k0 - cu[b]) / 32) % tile_blocks == tile_blocks - 1 || k0 + 32 >= kend)) {
                    for (int i = q0; i < q1; ++i) {
                        int kp = kpre[(size_t)h * T + i] + fexp;
                        for (int c = 0; c < d; ++c) {
                            double* pc = &part[(i - q0) * d + c];
                            double* ac = &acc16[(i - q0) * d + c];
                            *ac = orc_f16_round(*ac + orc_f16_round(ldexp(*pc, kp)));
                            *pc = 0.0;
                        }
                    }
                }
            }
            if (kpre && dq16)
                for (int i = q0; i < q1; ++i)
                    for (int c = 0; c < d; ++c)
                        dq16[((size_t)i * Hq + h) * d + c] =
                            scale * ldexp(acc16[(i - q0) * d + c], -(kpre[(size_t)h * T + i] + fexp));
        }
        free(buf);
        free(part);
        free(acc16);
    }
    return ORC_OK;
}

/* dV_j = sum over the group's q heads and visible queries of P^_ij dO^_i and
 * dK_j = scale * sum dS^_ij Q^_i, for every key of the listed document-local
 * 32-key blocks.  kblocks: n pairs (kv head, t0).  GQA: q head h reads kv
 * head floor(h * Hkv / Hq) (contiguous groups).  dK, dV: [T][Hkv][d],
 * accumulated into. */
int orc_bwd_dkdv(int T, int B, const int32_t* cu, int Hq, int Hkv, int d, double scale,
                 int causal, const double* Q, const double* K, const double* V, const double* Qs,
                 const double* Ks, const double* G, const double* D, const double* LSE, int mode,
                 int per_row_ds, int64_t n, const int32_t* kblocks, double* dK, double* dV)
{
    if (check_attn_args(T, B, cu, Hq, Hkv, d) != ORC_OK) return ORC_EBADARG;
    if (check_blocks(B, cu, n, kblocks, Hkv) != ORC_OK) return ORC_EBADARG;
    orc_attn a = {T, B, Hq, Hkv, d, causal, cu, scale, Q, K, V, Qs, Ks};
    orc_bwd w = {&a, G, D, LSE, mode, per_row_ds};
    int Gr = Hq / Hkv;
#pragma omp parallel
    {
        double* buf = (double*)malloc(sizeof(double) * 6 * 1024);
#pragma omp for schedule(dynamic)
        for (int64_t k = 0; k < n; ++k) {
            int g = kblocks[2 * k], k0 = kblocks[2 * k + 1];
            int b = doc_of(B, cu, k0);
            int k1 = k0 + 32 < cu[b + 1] ? k0 + 32 : cu[b + 1];
            double *P = buf, *dP = buf + 1024, *dS = buf + 2048, *Pq = buf + 3072,
                   *dSk = buf + 4096, *dSq = buf + 5120;
            for (int h = g * Gr; h < (g + 1) * Gr; ++h) {
                int qstart = causal ? k0 : cu[b];
                for (int q0 = qstart; q0 < cu[b + 1]; q0 += 32) {
                    int q1 = q0 + 32 < cu[b + 1] ? q0 + 32 : cu[b + 1];
                    bwd_block(&w, h, q0, q1, k0, k1, P, dP, dS, Pq, dSk, dSq);
                    for (int j = k0; j < k1; ++j) {
                        double* ov = dV + ((size_t)j * Hkv + g) * d;
                        double* ok = dK + ((size_t)j * Hkv + g) * d;
                        for (int c = 0; c < d; ++c) {
                            double av = 0.0, ak = 0.0;
                            for (int i = q0; i < q1; ++i) {
                                int e = (i - q0) * 32 + (j - k0);
                                av += Pq[e] * row(G, Hq, d, i, h)[c];
                                ak += dSk[e] * row(Q, Hq, d, i, h)[c];
                            }
                            ov[c] += av;
                            ok[c] += scale * ak;
                        }
                    }
                }
            }
        }
        free(buf);
    }
    return ORC_OK;
}

/* ========================================================================= */
/* Evaluation-noise bookkeeping (test support; not part of the method)        */
/* ========================================================================= */
/* A GPU forms each score and each dP as a sum of E4M3 products in its own
 * order and precision, and P, dS in FP32, so a value can land on the other
 * side of an E4M3 rounding midpoint than the FP64 value above; both roundings
 * are results of the method ([R] S8 "What the experiments establish" compares
 * against references within tolerances for this reason).  The routines below
 * take the evaluation error as an argument, `noise`: the largest deviation of
 * a dot product, as a fraction of the sum of the absolute values of its
 * terms (the caller states the figure for its hardware).  For the forward
 * they bound how far such flips can move a row; for the backward they list,
 * per element, the range of E4M3 results that any evaluation within that
 * error could produce.  They recompute what they need from the definitions
 * above and feed nothing back into them. */

/* scale * sum_c |Q_ic K_jc| over the score's terms (its evaluation scale). */
static double score_terms(const orc_attn* a, int h, int i, int j)
{
    const double* q = row(a->Qs ? a->Qs : a->Q, a->Hq, a->d, i, h);
    const double* k = row(a->Ks ? a->Ks : a->K, a->Hkv, a->d, j, kv_head(a, h));
    double ab = 0.0;
    for (int c = 0; c < a->d; ++c) ab += fabs(q[c] * k[c]);
    return a->scale * ab;
}

/* Relative error of a weight or probability whose score may be off by
 * noise * (score terms): exp of that deviation is 1 + (deviation) to first
 * order; 2^-20 more covers the FP32 exponential itself. */
static double weight_rel_tol(double noise, double sterms) { return noise * sterms + ldexp(1.0, -20); }

/* E4M3 results of all values within tol of y: [lo, hi] (rounding is
 * monotone, so the ends suffice). */
static void e4m3_range(double y, double tol, double* lo, double* hi)
{
    *lo = e4m3_round(y - tol);
    *hi = e4m3_round(y + tol);
}

/* Forward: for each listed row (mode 0, 1 or 3 of fwd_row), ties[0] bounds
 * the change of any element of O and ties[1] the relative change of l that
 * different roundings of near-midpoint weights could cause: with step_j the
 * spread of the possible P^_j (in units of the final reference) and l the
 * row's normaliser, a change of P^_j by step_j moves O by step_j (V_j - O) / l
 * and l by step_j, so ties[0] = sum_j step_j (max|V_j| + max|O|) / l and
 * ties[1] = sum_j step_j / l.  Rows outside every document get 0. */
int orc_fwd_ties(int T, int B, const int32_t* cu, int Hq, int Hkv, int d, double scale,
                 int causal, const double* Q, const double* K, const double* V, const double* Qs,
                 const double* Ks, int mode, int kblock, double noise, int64_t n_rows,
                 const int32_t* rows, double* ties)
{
    if (check_attn_args(T, B, cu, Hq, Hkv, d) != ORC_OK) return ORC_EBADARG;
    if (kblock < 1 || !(mode == 0 || mode == 1 || mode == 3)) return ORC_EBADARG;
    orc_attn a = {T, B, Hq, Hkv, d, causal, cu, scale, Q, K, V, Qs, Ks};
    int64_t n = rows ? n_rows : (int64_t)Hq * T;
    int Tn = T > 0 ? T : 1;
#pragma omp parallel
    {
        double* s_buf = (double*)malloc(sizeof(double) * Tn);
        double* r_buf = (double*)malloc(sizeof(double) * Tn);
        double* O = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 4)
        for (int64_t k = 0; k < n; ++k) {
            int h = rows ? rows[2 * k] : (int)(k / Tn);
            int i = rows ? rows[2 * k + 1] : (int)(k % Tn);
            double* out = ties + 2 * ((size_t)h * T + i);
            out[0] = out[1] = 0.0;
            int b = doc_of(B, cu, i);
            if (b < 0) continue;
            double LSE;
            fwd_row(&a, mode, kblock, h, i, O, &LSE, NULL, s_buf);
            int j0 = cu[b], j1 = key_end(&a, b, i), g = kv_head(&a, h);
            /* the reference each weight was rounded against */
            double r = -INFINITY;
            for (int k0 = j0; k0 < j1; k0 += (mode == 3 ? kblock : j1 - j0)) {
                int k1 = (mode == 3 && k0 + kblock < j1) ? k0 + kblock : j1;
                for (int j = k0; j < k1; ++j) {
                    double c = ceil(s_buf[j - j0] * M_LOG2E);
                    r = c > r ? c : r;
                }
                for (int j = k0; j < k1; ++j) r_buf[j - j0] = r;
            }
            double l = exp2(LSE * M_LOG2E - r); /* in units of the final reference */
            double om = 0.0, sw = 0.0, swv = 0.0;
            for (int c = 0; c < d; ++c) om = fabs(O[c]) > om ? fabs(O[c]) : om;
            for (int j = j0; j < j1; ++j) {
                double y = 256.0 * exp2(s_buf[j - j0] * M_LOG2E - r_buf[j - j0]);
                double lo, hi;
                e4m3_range(y, y * weight_rel_tol(noise, score_terms(&a, h, i, j)), &lo, &hi);
                double step = (hi - lo) / 256.0 * exp2(r_buf[j - j0] - r);
                if (step == 0.0) continue;
                const double* vj = row(V, Hkv, d, j, g);
                double vm = 0.0;
                for (int c = 0; c < d; ++c) vm = fabs(vj[c]) > vm ? fabs(vj[c]) : vm;
                sw += step;
                swv += step * vm;
            }
            out[0] = (swv + sw * om) / l;
            out[1] = sw / l;
        }
        free(s_buf);
        free(r_buf);
        free(O);
    }
    return ORC_OK;
}

/* Backward, one 32x32 block computed by bwd_block: for every visible element
 * the most an evaluation within `noise` moves dS (tol_ds: the score's error
 * through P, plus P times the error of dP, a dot product of the same kind;
 * D is a plain FP32 sum whose error is far smaller) and the relative error of
 * P (rel_p). */
static void block_tolerances(const orc_bwd* w, int h, int q0, int q1, int k0, int k1,
                             const double* P, const double* dP, const double* dS, double noise,
                             double* tol_ds, double* rel_p)
{
    const orc_attn* a = w->a;
    int d = a->d, g = kv_head(a, h);
    for (int k = 0; k < 1024; ++k) tol_ds[k] = rel_p[k] = 0.0;
    for (int i = q0; i < q1; ++i) {
        const double* gi = row(w->G, a->Hq, d, i, h);
        for (int j = k0; j < k1; ++j) {
            if (a->causal && j > i) continue;
            int e = (i - q0) * 32 + (j - k0);
            const double* vj = row(a->V, a->Hkv, d, j, g);
            double pterms = 0.0;
            for (int c = 0; c < d; ++c) pterms += fabs(gi[c] * vj[c]);
            rel_p[e] = weight_rel_tol(noise, score_terms(a, h, i, j));
            tol_ds[e] = fabs(dS[e]) * rel_p[e] + P[e] * noise * pterms;
        }
    }
}

/* Exponents a block (or row) maximum amax could take when every entry may be
 * off by up to tmax: [ceil_exp(amax - tmax), ceil_exp(amax + tmax)]. */
static void exponent_range(double amax, double tmax, int* elo, int* ehi)
{
    *elo = orc_ceil_exponent(amax - tmax > 0.0 ? amax - tmax : 0.0);
    *ehi = orc_ceil_exponent(amax + tmax);
    if (amax - tmax <= 0.0) *elo = -127;
}

/* Range of dS^ results for dS within tol when the block exponent may be any
 * of [elo, ehi] (at most a few values): the union of the per-exponent
 * ranges, as an interval. */
static void ds_range(double ds, double tol, int elo, int ehi, double* lo, double* hi)
{
    *lo = INFINITY;
    *hi = -INFINITY;
    if (ehi - elo > 3) elo = ehi - 3; /* below that the entry rounds to 0 or its neighbours */
    for (int e = elo; e <= ehi; ++e) {
        double a, b;
        e4m3_range(ldexp(ds, -e), ldexp(tol, -e), &a, &b);
        a = ldexp(a, e);
        b = ldexp(b, e);
        *lo = a < *lo ? a : *lo;
        *hi = b > *hi ? b : *hi;
    }
}

/* For the 32 query rows of the document-local block starting at q0 (head
 * h): every visible key j whose dS^ of the dQ product could come out
 * differently under an evaluation within `noise`, as (row i, key j, lo, hi),
 * lo and hi the lowest and highest possible dS^ minus the value bwd_block
 * chooses.  Writes at most `cap` entries; returns how many there are (call
 * again with a larger cap if that is more), or a negative error. */
int64_t orc_bwd_dq_ranges(int T, int B, const int32_t* cu, int Hq, int Hkv, int d, double scale,
                          int causal, const double* Q, const double* K, const double* V,
                          const double* Qs, const double* Ks, const double* G, const double* D,
                          const double* LSE, int per_row_ds, double noise, int h, int q0,
                          int64_t cap, int32_t* out_i, int32_t* out_j, double* out_lo,
                          double* out_hi)
{
    if (check_attn_args(T, B, cu, Hq, Hkv, d) != ORC_OK) return ORC_EBADARG;
    int b = doc_of(B, cu, q0);
    if (b < 0 || (q0 - cu[b]) % 32 || h < 0 || h >= Hq) return ORC_EBADARG;
    orc_attn a = {T, B, Hq, Hkv, d, causal, cu, scale, Q, K, V, Qs, Ks};
    orc_bwd w = {&a, G, D, LSE, 0, per_row_ds};
    int q1 = q0 + 32 < cu[b + 1] ? q0 + 32 : cu[b + 1];
    int kend = causal ? q1 : cu[b + 1];
    int nkb = (kend - cu[b] + 31) / 32;
    /* per key block: up to 1024 entries, gathered in key order afterwards */
    int32_t* cnt = (int32_t*)calloc((size_t)nkb + 1, sizeof(int32_t));
    int32_t* ei = (int32_t*)malloc(sizeof(int32_t) * 1024 * (size_t)(nkb + 1));
    int32_t* ej = (int32_t*)malloc(sizeof(int32_t) * 1024 * (size_t)(nkb + 1));
    double* elo = (double*)malloc(sizeof(double) * 1024 * (size_t)(nkb + 1));
    double* ehi = (double*)malloc(sizeof(double) * 1024 * (size_t)(nkb + 1));
#pragma omp parallel
    {
        double* buf = (double*)malloc(sizeof(double) * 8 * 1024);
        double *P = buf, *dP = buf + 1024, *dS = buf + 2048, *Pq = buf + 3072,
               *dSk = buf + 4096, *dSq = buf + 5120, *tol = buf + 6144, *relp = buf + 7168;
#pragma omp for schedule(dynamic)
        for (int kb = 0; kb < nkb; ++kb) {
            int k0 = cu[b] + 32 * kb;
            int k1 = k0 + 32 < cu[b + 1] ? k0 + 32 : cu[b + 1];
            bwd_block(&w, h, q0, q1, k0, k1, P, dP, dS, Pq, dSk, dSq);
            block_tolerances(&w, h, q0, q1, k0, k1, P, dP, dS, noise, tol, relp);
            double amax = 0.0, tmax = 0.0;
            for (int e = 0; e < 1024; ++e) {
                amax = fabs(dS[e]) > amax ? fabs(dS[e]) : amax;
                tmax = tol[e] > tmax ? tol[e] : tmax;
            }
            int xlo, xhi;
            exponent_range(amax, tmax, &xlo, &xhi);
            size_t o = (size_t)kb * 1024;
            for (int i = q0; i < q1; ++i) {
                int base = (i - q0) * 32;
                int rlo = xlo, rhi = xhi;
                if (per_row_ds) {
                    double ra = 0.0, rt = 0.0;
                    for (int j = k0; j < k1; ++j) {
                        ra = fabs(dS[base + j - k0]) > ra ? fabs(dS[base + j - k0]) : ra;
                        rt = tol[base + j - k0] > rt ? tol[base + j - k0] : rt;
                    }
                    exponent_range(ra, rt, &rlo, &rhi);
                }
                for (int j = k0; j < k1; ++j) {
                    if (causal && j > i) continue;
                    int e = base + (j - k0);
                    double lo, hi;
                    ds_range(dS[e], tol[e], rlo, rhi, &lo, &hi);
                    /* the oracle's own choice is always one of the results */
                    lo = lo < dSq[e] ? lo : dSq[e];
                    hi = hi > dSq[e] ? hi : dSq[e];
                    if (lo == dSq[e] && hi == dSq[e]) continue;
                    ei[o + cnt[kb]] = i;
                    ej[o + cnt[kb]] = j;
                    elo[o + cnt[kb]] = lo - dSq[e];
                    ehi[o + cnt[kb]] = hi - dSq[e];
                    ++cnt[kb];
                }
            }
        }
        free(buf);
    }
    int64_t n = 0;
    for (int kb = 0; kb < nkb; ++kb)
        for (int k = 0; k < cnt[kb]; ++k, ++n)
            if (n < cap) {
                size_t o = (size_t)kb * 1024 + k;
                out_i[n] = ei[o];
                out_j[n] = ej[o];
                out_lo[n] = elo[o];
                out_hi[n] = ehi[o];
            }
    free(cnt);
    free(ei);
    free(ej);
    free(elo);
    free(ehi);
    return n;
}

/* The same for the dK and dV products of the 32 keys of the document-local
 * block starting at k0 (kv head g): `which` 0 lists the probability operand
 * P^ of dV, 1 the dS^ of dK (32x32 block exponents), over the group's q heads
 * and the visible queries, as (head, query i, key j, lo, hi). */
int64_t orc_bwd_dkdv_ranges(int T, int B, const int32_t* cu, int Hq, int Hkv, int d, double scale,
                            int causal, const double* Q, const double* K, const double* V,
                            const double* Qs, const double* Ks, const double* G, const double* D,
                            const double* LSE, int per_row_ds, double noise, int g, int k0,
                            int which, int64_t cap, int32_t* out_h, int32_t* out_i,
                            int32_t* out_j, double* out_lo, double* out_hi)
{
    if (check_attn_args(T, B, cu, Hq, Hkv, d) != ORC_OK) return ORC_EBADARG;
    int b = doc_of(B, cu, k0);
    if (b < 0 || (k0 - cu[b]) % 32 || g < 0 || g >= Hkv || which < 0 || which > 1)
        return ORC_EBADARG;
    orc_attn a = {T, B, Hq, Hkv, d, causal, cu, scale, Q, K, V, Qs, Ks};
    orc_bwd w = {&a, G, D, LSE, 0, per_row_ds};
    int k1 = k0 + 32 < cu[b + 1] ? k0 + 32 : cu[b + 1];
    int Gr = Hq / Hkv;
    int qs = causal ? k0 : cu[b];
    int nqb = (cu[b + 1] - qs + 31) / 32;
    int nblk = Gr * nqb;
    int32_t* cnt = (int32_t*)calloc((size_t)nblk + 1, sizeof(int32_t));
    int32_t* eh = (int32_t*)malloc(sizeof(int32_t) * 1024 * (size_t)(nblk + 1));
    int32_t* ei = (int32_t*)malloc(sizeof(int32_t) * 1024 * (size_t)(nblk + 1));
    int32_t* ej = (int32_t*)malloc(sizeof(int32_t) * 1024 * (size_t)(nblk + 1));
    double* elo = (double*)malloc(sizeof(double) * 1024 * (size_t)(nblk + 1));
    double* ehi = (double*)malloc(sizeof(double) * 1024 * (size_t)(nblk + 1));
#pragma omp parallel
    {
        double* buf = (double*)malloc(sizeof(double) * 8 * 1024);
        double *P = buf, *dP = buf + 1024, *dS = buf + 2048, *Pq = buf + 3072,
               *dSk = buf + 4096, *dSq = buf + 5120, *tol = buf + 6144, *relp = buf + 7168;
#pragma omp for schedule(dynamic)
        for (int x = 0; x < nblk; ++x) {
            int h = g * Gr + x / nqb, q0 = qs + 32 * (x % nqb);
            int q1 = q0 + 32 < cu[b + 1] ? q0 + 32 : cu[b + 1];
            bwd_block(&w, h, q0, q1, k0, k1, P, dP, dS, Pq, dSk, dSq);
            block_tolerances(&w, h, q0, q1, k0, k1, P, dP, dS, noise, tol, relp);
            int xlo = 0, xhi = 0;
            if (which == 1) {
                double amax = 0.0, tmax = 0.0;
                for (int e = 0; e < 1024; ++e) {
                    amax = fabs(dS[e]) > amax ? fabs(dS[e]) : amax;
                    tmax = tol[e] > tmax ? tol[e] : tmax;
                }
                exponent_range(amax, tmax, &xlo, &xhi);
            }
            size_t o = (size_t)x * 1024;
            for (int i = q0; i < q1; ++i)
                for (int j = k0; j < k1; ++j) {
                    if (causal && j > i) continue;
                    int e = (i - q0) * 32 + (j - k0);
                    double lo, hi, ch;
                    if (which == 0) {
                        double y = 256.0 * P[e];
                        e4m3_range(y, y * relp[e], &lo, &hi);
                        lo /= 256.0;
                        hi /= 256.0;
                        ch = Pq[e];
                    } else {
                        ds_range(dS[e], tol[e], xlo, xhi, &lo, &hi);
                        ch = dSk[e];
                    }
                    lo = lo < ch ? lo : ch;
                    hi = hi > ch ? hi : ch;
                    if (lo == ch && hi == ch) continue;
                    eh[o + cnt[x]] = h;
                    ei[o + cnt[x]] = i;
                    ej[o + cnt[x]] = j;
                    elo[o + cnt[x]] = lo - ch;
                    ehi[o + cnt[x]] = hi - ch;
                    ++cnt[x];
                }
        }
        free(buf);
    }
    int64_t n = 0;
    for (int x = 0; x < nblk; ++x)
        for (int k = 0; k < cnt[x]; ++k, ++n)
            if (n < cap) {
                size_t o = (size_t)x * 1024 + k;
                out_h[n] = eh[o];
                out_i[n] = ei[o];
                out_j[n] = ej[o];
                out_lo[n] = elo[o];
                out_hi[n] = ehi[o];
            }
    free(cnt);
    free(eh);
    free(ei);
    free(ej);
    free(elo);
    free(ehi);
    return n;
}
