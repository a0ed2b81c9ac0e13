/*
 * kvcache.c -- plain CPU reference of 4-bit KV-cache decode attention.
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c (it is linked into the same
 * liboracle.so): only the test suite, the smoke check and the benchmark's
 * cpu_baseline leg load it.  The HIP library never calls it and shares no
 * code, header or table with it.
 *
 * Source: [UQ] "FP4 训练 vs FP4 推理：LLM 量化路线正在分叉" (reports.10n1j.top),
 * section on UltraQuant: decode attention with an FP8 query against an FP4 KV
 * cache, UE8M0 group scales, on CDNA4's native scaled-MFMA path; K and V
 * treated asymmetrically; a Walsh-Hadamard rotation.  The page gives no
 * formulas.  The readings taken here (each stated at its function):
 *   - group = 32 elements with one UE8M0 (power-of-two) scale, the OCP MX
 *     rule E = floor(log2 amax) - emax (emax 2 for E2M1, 8 for E4M3), clamped
 *     to [-127, 127], the element rounded to nearest-even and saturated;
 *   - K: one group per 32 head-dim channels of a token (the contraction axis
 *     of Q K^T), after a Walsh-Hadamard transform over the head dim; V: one
 *     group per channel over 32 consecutive tokens (the contraction axis of
 *     P V), no rotation -- the asymmetric treatment;
 *   - Q: E4M3 groups of 32 channels after the same transform scaled by 1/D,
 *     so that the rotation cancels in Q K^T;
 *   - the FP8 KV baseline the page measures against is read as the same cache
 *     in MXFP8 (E4M3 codes, the same groups and rotation);
 *   - the softmax probabilities P are the second FP8 operand: quantized to
 *     E4M3 per 32 consecutive tokens with the exponent floor(log2 amax) - 7,
 *     one above the MX rule, so the group maximum is never clamped; the
 *     normaliser is the sum of the unquantized probabilities.
 * The arithmetic that decides codes from bf16 inputs (transform, scaling,
 * rounding of Q, K, V) is binary32 like the rest of the oracle; scores,
 * probabilities and the output are binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* From oracle.c (same library). */
float orc_bf16_to_f32(uint16_t b);
int orc_round_rtne(float z, int fmt);
float orc_e4m3_decode(uint8_t b);

#define ORC_E2M1_FMT 0

/* E2M1 magnitudes by code. */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Walsh-Hadamard transform of length n (a power of two) in binary32, natural
 * (Sylvester) order, butterfly spans 1, 2, 4, ..., n/2 in that order, each
 * butterfly (a, b) -> (a + b, a - b), no normalisation: the result is H_n v
 * with H_n[i][j] = (-1)^popcount(i & j).  [UQ] names a Walsh-Hadamard
 * rotation; size, order and scaling are this reading. */
void orc_fwht_f32(float *v, int n)
{
    for (int h = 1; h < n; h <<= 1)
        for (int i = 0; i < n; ++i)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

/* UE8M0 exponent of a group: floor(log2 amax) - emax, clamped to
 * [-127, 127]; an all-zero group gets -127.  floor(log2) from frexp (exact). */
int orc_mx_exponent(double amax, int emax)
{
    if (!(amax > 0.0)) return -127;
    int ex;
    frexp(amax, &ex); /* amax = f 2^ex, f in [0.5, 1) */
    int e = (ex - 1) - emax;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* E4M3FN encode of a non-negative binary64 value: the nearest of the 127
 * finite non-negative codes, ties to the even byte, anything above 448
 * saturating to 448 (0x7E).  A plain nearest-point search. */
uint8_t orc_e4m3_encode_d(double a)
{
    if (!(a <= 448.0)) return 0x7E;
    int best = 0;
    double bestd = fabs(a);
    for (int b = 1; b <= 0x7E; ++b) {
        double d = fabs(a - (double)orc_e4m3_decode((uint8_t)b));
        if (d < bestd || (d == bestd && (b % 2) == 0 && (best % 2) != 0)) {
            best = b;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* Value of an E4M3FN byte (sign in bit 7). */
static double e4m3_value(uint8_t b)
{
    double m = (double)orc_e4m3_decode((uint8_t)(b & 0x7F));
    return (b & 0x80) ? -m : m;
}

static double e2m1_value(uint8_t nib)
{
    double m = kE2M1[nib & 7];
    return (nib & 8) ? -m : m;
}

/* MXFP8 (E4M3, UE8M0 per 32) of one query row of D channels, after the
 * optional rotation q' = (H_D q) / D in binary32 (the 1/D is a power of two,
 * so it is exact).  codes[D] are E4M3FN bytes (sign in bit 7), scales[D/32]
 * biased exponents.  Element: E4M3 nearest-even of |q'| 2^-E (exact
 * scaling), saturating at 448. */
void orc_q_quantize(const uint16_t *q, int D, int rotate, uint8_t *codes, uint8_t *scales)
{
    float y[512];
    for (int d = 0; d < D; ++d) y[d] = orc_bf16_to_f32(q[d]);
    if (rotate) {
        orc_fwht_f32(y, D);
        const float inv = (float)ldexp(1.0, -(int)log2((double)D));
        for (int d = 0; d < D; ++d) y[d] = y[d] * inv;
    }
    for (int g = 0; g < D / 32; ++g) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)y[32 * g + i]));
        int e = orc_mx_exponent(amax, 8);
        scales[g] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; ++i) {
            float z = y[32 * g + i];
            uint8_t mag = orc_e4m3_encode_d(ldexp(fabs((double)z), -e));
            codes[32 * g + i] = (uint8_t)((signbit(z) ? 0x80 : 0) | mag);
        }
    }
}

/* One MX group of 32 values: the exponent E = floor(log2 amax) - emax
 * (emax 2 for E2M1, 8 for E4M3), then each value scaled by 2^-E (exact) and
 * rounded to nearest-even, saturating at the format maximum.  E2M1 codes are
 * packed two per byte (element 2j in the low nibble of byte j), E4M3FN codes
 * one per byte with the sign in bit 7.  Returns the biased exponent. */
static uint8_t mx_group(const float *y, int fp8, uint8_t *codes)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)y[i]));
    const int e = orc_mx_exponent(amax, fp8 ? 8 : 2);
    if (fp8) {
        for (int i = 0; i < 32; ++i)
            codes[i] = (uint8_t)((signbit(y[i]) ? 0x80 : 0) | orc_e4m3_encode_d(ldexp(fabs((double)y[i]), -e)));
    } else {
        for (int i = 0; i < 32; i += 2) {
            int c0 = orc_round_rtne((float)ldexp((double)y[i], -e), ORC_E2M1_FMT);
            int c1 = orc_round_rtne((float)ldexp((double)y[i + 1], -e), ORC_E2M1_FMT);
            codes[i / 2] = (uint8_t)(c0 | (c1 << 4));
        }
    }
    return (uint8_t)(e + 127);
}

/* Value (without the group scale) of element i of a code array. */
static double code_value(const uint8_t *codes, int64_t i, int fp8)
{
    if (fp8) return e4m3_value(codes[i]);
    const uint8_t b = codes[i / 2];
    return e2m1_value((uint8_t)((i & 1) ? b >> 4 : b & 15));
}

/* One key row of D channels after the optional unnormalised transform H_D k
 * in binary32, in MX groups of 32 channels: E2M1 (fp8 = 0, codes[D/2]) or
 * E4M3 (fp8 = 1, codes[D]); scales[D/32] biased exponents. */
void orc_k_quantize_row(const uint16_t *k, int D, int rotate, int fp8, uint8_t *codes, uint8_t *scales)
{
    float y[512];
    for (int d = 0; d < D; ++d) y[d] = orc_bf16_to_f32(k[d]);
    if (rotate) orc_fwht_f32(y, D);
    for (int g = 0; g < D / 32; ++g) scales[g] = mx_group(y + 32 * g, fp8, codes + g * (fp8 ? 32 : 16));
}

/* The KV cache of one sequence (one batch entry, one KV head), natural layout,
 * FP4 (E2M1, fp8 = 0) or the FP8 baseline (E4M3, fp8 = 1); cb = bytes per code
 * (1/2 or 1).
 *   k, v: bf16 [token][tok_stride], channels contiguous; tokens [0, len) hold
 *         data, tokens [len, ntok) count as zeros (ntok a multiple of 32).
 *   kcodes [ntok][D cb], kscales [ntok][D/32]: K along the head dim.
 *   vcodes [D][ntok cb], vscales [D][ntok/32]: V along tokens, one group per
 *         channel and 32 tokens. */
void orc_kv_quantize_seq(const uint16_t *k, const uint16_t *v, int64_t tok_stride, int64_t len, int64_t ntok, int D,
                         int rotate, int fp8, uint8_t *kcodes, uint8_t *kscales, uint8_t *vcodes, uint8_t *vscales)
{
    uint16_t zero[512];
    memset(zero, 0, sizeof(zero));
    const int64_t krow = fp8 ? D : D / 2, vrow = fp8 ? ntok : ntok / 2;
    for (int64_t t = 0; t < ntok; ++t)
        orc_k_quantize_row(t < len ? k + t * tok_stride : zero, D, 0 != rotate, fp8, kcodes + t * krow,
                           kscales + t * (D / 32));
    for (int d = 0; d < D; ++d)
        for (int64_t g = 0; g < ntok / 32; ++g) {
            float y[32];
            for (int i = 0; i < 32; ++i) {
                int64_t t = 32 * g + i;
                y[i] = t < len ? orc_bf16_to_f32(v[t * tok_stride + d]) : 0.0f;
            }
            vscales[(int64_t)d * (ntok / 32) + g] = mx_group(y, fp8, vcodes + (int64_t)d * vrow + g * (fp8 ? 32 : 16));
        }
}

/* Dequantized cache of one sequence: kh [len][D], vh [len][D] (binary64,
 * exact), from the quantization above.  Returns 0, or -2 if out of memory. */
static int dequantized_seq(const uint16_t *k, const uint16_t *v, int64_t tok_stride, int64_t len, int D, int rotate,
                           int fp8, double *kh, double *vh)
{
    const int64_t ntok = (len + 31) / 32 * 32;
    const int64_t krow = fp8 ? D : D / 2, vrow = fp8 ? ntok : ntok / 2;
    uint8_t *kc = malloc((size_t)(ntok * krow)), *ks = malloc((size_t)(ntok * (D / 32)));
    uint8_t *vc = malloc((size_t)(D * vrow)), *vs = malloc((size_t)(D * (ntok / 32)));
    if (!kc || !ks || !vc || !vs) {
        free(kc), free(ks), free(vc), free(vs);
        return -2;
    }
    orc_kv_quantize_seq(k, v, tok_stride, len, ntok, D, rotate, fp8, kc, ks, vc, vs);
    for (int64_t t = 0; t < len; ++t)
        for (int d = 0; d < D; ++d) {
            kh[t * D + d] = ldexp(code_value(kc + t * krow, d, fp8), (int)ks[t * (D / 32) + d / 32] - 127);
            vh[t * D + d] = ldexp(code_value(vc + (int64_t)d * vrow, t, fp8), (int)vs[(int64_t)d * (ntok / 32) + t / 32] - 127);
        }
    free(kc), free(ks), free(vc), free(vs);
    return 0;
}

/* Dequantized MXFP8 query row. */
static void query_row(const uint16_t *q, int D, int rotate, double *qh)
{
    uint8_t qc[512], qs[16];
    orc_q_quantize(q, D, rotate, qc, qs);
    for (int d = 0; d < D; ++d) qh[d] = ldexp(e4m3_value(qc[d]), (int)qs[d / 32] - 127);
}

/* E4M3 value of p in a block with exponent e: E4M3(p 2^-e) 2^e. */
static double deq_p(double p, int e)
{
    return ldexp((double)orc_e4m3_decode(orc_e4m3_encode_d(ldexp(p, -e))), e);
}

/* Decode attention of one sequence: G query rows against its KV cache (FP4,
 * or the FP8 baseline with fp8 = 1).
 *   q [G][D] bf16; k, v as for orc_kv_quantize_seq; out [G][D] binary64.
 *   Q' = MXFP8(q), K', V' the dequantized cache (exact);
 *   s_t = <Q'_r, K'_t>, x_t = s_t sm_scale log2(e) for t < len;
 *   p_t = 2^(x_t - m) with m = ceil(max_t x_t) (any integer m gives the same
 *   output: the group scales below absorb the power of two);
 *   per 32-token group a = max p, E = floor(log2 a) - 7 (>= -127; a = 0 gives
 *   -127), p'_t = E4M3(p_t 2^-E) 2^E;
 *   out_r = sum_t p'_t V'_t / sum_t p_t.   len = 0 gives zeros.
 * Returns 0, -1 for a bad shape, -2 if out of memory. */
int orc_kv_decode_seq(const uint16_t *q, int G, const uint16_t *k, const uint16_t *v, int64_t tok_stride, int64_t len,
                      int D, float sm_scale, int rotate, int fp8, double *out)
{
    if (D % 32 || D > 512 || G < 1) return -1;
    memset(out, 0, sizeof(double) * (size_t)G * (size_t)D);
    if (len <= 0) return 0;
    const int64_t ntok = (len + 31) / 32 * 32;
    double *kh = malloc(sizeof(double) * (size_t)(len * D)), *vh = malloc(sizeof(double) * (size_t)(len * D));
    double *x = malloc(sizeof(double) * (size_t)len);
    if (!kh || !vh || !x || dequantized_seq(k, v, tok_stride, len, D, rotate, fp8, kh, vh)) {
        free(kh), free(vh), free(x);
        return -2;
    }
    const double c = (double)sm_scale / log(2.0);
    for (int r = 0; r < G; ++r) {
        double qh[512];
        query_row(q + (int64_t)r * D, D, rotate, qh);
        double xmax = -INFINITY;
        for (int64_t t = 0; t < len; ++t) {
            double s = 0.0;
            for (int d = 0; d < D; ++d) s += qh[d] * kh[t * D + d];
            x[t] = s * c;
            xmax = fmax(xmax, x[t]);
        }
        const double m = ceil(xmax);
        double l = 0.0;
        double *o = out + (int64_t)r * D;
        for (int64_t g = 0; g < ntok / 32; ++g) {
            double p[32], a = 0.0;
            for (int i = 0; i < 32; ++i) {
                int64_t t = 32 * g + i;
                p[i] = t < len ? exp2(x[t] - m) : 0.0;
                a = fmax(a, p[i]);
                l += p[i];
            }
            const int e = orc_mx_exponent(a, 7);
            for (int i = 0; i < 32; ++i) {
                int64_t t = 32 * g + i;
                if (t >= len) continue;
                const double ph = deq_p(p[i], e);
                if (ph == 0.0) continue;
                for (int d = 0; d < D; ++d) o[d] += ph * vh[t * D + d];
            }
        }
        for (int d = 0; d < D; ++d) o[d] /= l;
    }
    free(kh), free(vh), free(x);
    return 0;
}

/* Comparison bound for a decode computed in binary32 (test infrastructure).
 * An implementation that forms the scores with binary32 accumulation and
 * 2^x with a few-ulp exponential takes the E4M3 decisions of P from values
 * within a small relative distance of these binary64 ones, so a probability
 * (or a block exponent) lying that close to a rounding boundary may go
 * either way; both results are correct.  For each output element this
 * writes
 *   mass[r][d] = sum_t p'_t |V'_t[d]| / sum_t p_t   (the scale of the sum),
 *   amb[r][d]  = sum over such tokens of |largest possible change of p'_t|
 *                |V'_t[d]| / sum_t p_t, plus mass[r][d] times the largest
 *                relative change of the normaliser, sum_t eps_t p_t / sum p,
 * with the relative perturbation of p_t taken as
 *   eps_t = c eps_s sum_d |Q'_d K'_td| + 2^-20 (|x_t| + 1)
 * (eps_s: accumulation error of a score relative to the sum of the
 * magnitudes of its products). */
int orc_kv_decode_bounds(const uint16_t *q, int G, const uint16_t *k, const uint16_t *v, int64_t tok_stride,
                         int64_t len, int D, float sm_scale, int rotate, int fp8, double eps_s, double *mass,
                         double *amb, int64_t *fragile)
{
    if (D % 32 || D > 512 || G < 1) return -1;
    memset(mass, 0, sizeof(double) * (size_t)G * (size_t)D);
    memset(amb, 0, sizeof(double) * (size_t)G * (size_t)D);
    *fragile = 0;
    if (len <= 0) return 0;
    const int64_t ntok = (len + 31) / 32 * 32;
    double *kh = malloc(sizeof(double) * (size_t)(len * D)), *vh = malloc(sizeof(double) * (size_t)(len * D));
    double *x = malloc(sizeof(double) * (size_t)len), *sabs = malloc(sizeof(double) * (size_t)len);
    if (!kh || !vh || !x || !sabs || dequantized_seq(k, v, tok_stride, len, D, rotate, fp8, kh, vh)) {
        free(kh), free(vh), free(x), free(sabs);
        return -2;
    }
    const double c = (double)sm_scale / log(2.0);
    for (int r = 0; r < G; ++r) {
        double qh[512];
        query_row(q + (int64_t)r * D, D, rotate, qh);
        double xmax = -INFINITY;
        for (int64_t t = 0; t < len; ++t) {
            double s = 0.0, sa = 0.0;
            for (int d = 0; d < D; ++d) {
                s += qh[d] * kh[t * D + d];
                sa += fabs(qh[d] * kh[t * D + d]);
            }
            x[t] = s * c;
            sabs[t] = sa;
            xmax = fmax(xmax, x[t]);
        }
        const double m = ceil(xmax);
        double l = 0.0, wsum = 0.0;
        for (int64_t t = 0; t < len; ++t) l += exp2(x[t] - m);
        double *ms = mass + (int64_t)r * D, *am = amb + (int64_t)r * D;
        for (int64_t g = 0; g < ntok / 32; ++g) {
            double p[32], eps[32], a = 0.0, emax = 0.0;
            for (int i = 0; i < 32; ++i) {
                int64_t t = 32 * g + i;
                p[i] = 0.0;
                eps[i] = 0.0;
                if (t >= len) continue;
                p[i] = exp2(x[t] - m);
                eps[i] = c * eps_s * sabs[t] + ldexp(fabs(x[t]) + 1.0, -20);
                a = fmax(a, p[i]);
                emax = fmax(emax, eps[i]);
            }
            const int e = orc_mx_exponent(a, 7);
            const int e_lo = orc_mx_exponent(a * (1.0 - emax), 7), e_hi = orc_mx_exponent(a * (1.0 + emax), 7);
            for (int i = 0; i < 32; ++i) {
                int64_t t = 32 * g + i;
                if (t >= len) continue;
                const double ph = deq_p(p[i], e);
                double worst = 0.0;
                for (int ee = e_lo; ee <= e_hi; ++ee) {
                    worst = fmax(worst, fabs(deq_p(p[i] * (1.0 - eps[i]), ee) - ph));
                    worst = fmax(worst, fabs(deq_p(p[i] * (1.0 + eps[i]), ee) - ph));
                    worst = fmax(worst, fabs(deq_p(p[i], ee) - ph));
                }
                /* a change within the perturbation itself is not a flip */
                if (worst <= 2.0 * eps[i] * p[i]) worst = 0.0;
                if (worst > 0.0) ++*fragile;
                wsum += eps[i] * p[i];
                for (int d = 0; d < D; ++d) {
                    const double va = fabs(vh[t * D + d]);
                    ms[d] += ph * va / l;
                    am[d] += worst * va / l;
                }
            }
        }
        for (int d = 0; d < D; ++d) am[d] += ms[d] * wsum / l;
    }
    free(kh), free(vh), free(x), free(sabs);
    return 0;
}
