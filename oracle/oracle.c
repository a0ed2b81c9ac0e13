/*
 * oracle.c -- plain, slow CPU reference of the 4-bit block quantizer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's cpu_baseline leg load this library.  The product path (the HIP
 * library under block_scaled_bit_ufp4_amd/) never calls it and shares no code,
 * header or table with it.
 *
 * Sources (the pages are web explainers of the methods; cited by page title
 * and section):
 *   [UFP4-ZC]  "当你的 GPU 学不会算账：FP4 训练里那个被忽视了 30 年的几何陷阱"
 *              (zhichai.net) -- sections "E2M1：一块刻度不均的尺子",
 *              "复利效应的反向版本", "UFP4：换一把尺子" (recipe table).
 *   [UFP4-TW]  "蚂蚁集团揭秘：为什么给AI'降精度省电'会悄悄让它越来越笨？"
 *              (techwalker.com) -- sections 二, 四, 五, 六.
 *   [MXFP4]    "AMD全新研究揭示：FP4训练不稳定性源于结构误差而非随机性不足"
 *              (cannews.ca) -- section "MXFP4：一种基于微缩放的低精度数据格式".
 *   [IF4]      "低精度量化技术：IF4自适应数据类型的原理与应用" (bxzpzcl.cn) --
 *              sections 2.1, 2.2 (format table), 3.1.1, 3.2, 6.1.
 *   [PHILOX]   Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
 *              as 1, 2, 3", SC'11 -- the Philox-4x32 round and key schedule.
 *
 * Numeric rules (the pages fix none of them; these are the readings taken):
 *   - the quantizer's arithmetic is IEEE binary32, round-to-nearest-even on
 *     every operation, no contraction (built with -ffp-contract=off), denormals
 *     kept, division correctly rounded; the integer codes are decided in that
 *     precision;
 *   - statistics and GEMM references accumulate in binary64.
 * Each function says which passage it follows.  Functions that are pinned
 * only by invariants say so ("parity unpinned") in their comment.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Configuration: the same field meanings as the library's ufp4_config, but   */
/* an independent declaration (the oracle includes no header of the library). */
/* ------------------------------------------------------------------------ */
enum { ORC_E2M1 = 0, ORC_E1M2 = 1, ORC_INT4 = 2, ORC_IF4 = 3, ORC_E2M1_MAX4 = 4, ORC_E2M1_MAX3 = 5, ORC_E2M1_MAX2 = 6 };
enum { ORC_SCALE_FP32 = 0, ORC_SCALE_E4M3 = 1, ORC_SCALE_E8M0 = 2 };
enum { ORC_RHT_NONE = 0, ORC_RHT_RANDOM = 1, ORC_RHT_DET = 2 };
enum { ORC_RTNE = 0, ORC_SR = 1 };
enum { ORC_ROW = 0, ORC_COL = 1 };
enum { ORC_BF16 = 0, ORC_F32 = 1 };

typedef struct {
    int32_t format;
    int32_t scale;
    int32_t block;
    int32_t rht;
    int32_t rounding;
    int32_t axis;
    uint64_t rht_seed;
    uint64_t sr_seed;
    uint32_t sr_stream;
    uint32_t reserved;
} orc_config;

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* Non-negative grid points, indexed by the 3-bit magnitude code k.
 * E2M1 {0,.5,1,1.5,2,3,4,6}: [UFP4-ZC] "E2M1：一块刻度不均的尺子"; [IF4] 1.
 * E1M2 {0,.5,...,3.5}: [UFP4-ZC] "UFP4：换一把尺子"; [UFP4-TW] 一.
 * INT4 {0..7}: the symmetric integer grid of NVINT4 ([IF4] 2.2 table, max 7). */
static const double GRID[3][8] = {
    {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0},
    {0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 3.0, 3.5},
    {0.0, 1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0},
};

/* Restricted-range E2M1 ([UFP4-ZC] "UFP4：换一把尺子": the attempt to emulate a
 * uniform grid on E2M1 by capping its range): the E2M1 points up to 4, 3 or
 * 2, i.e. magnitude codes k <= 6, 5 or 4; the cap is the format's maximum.
 * IF4's FP4 candidate uses the full E2M1 grid. */
static const double *grid_of(int fmt)
{
    return GRID[(fmt == ORC_IF4 || fmt >= ORC_E2M1_MAX4) ? ORC_E2M1 : fmt];
}
static int kmax_of(int fmt)
{
    return fmt == ORC_E2M1_MAX4 ? 6 : fmt == ORC_E2M1_MAX3 ? 5 : fmt == ORC_E2M1_MAX2 ? 4 : 7;
}

double orc_grid_value(int fmt, int k) { return grid_of(fmt)[k & 7]; }
float orc_gridmax(int fmt) { return (float)grid_of(fmt)[kmax_of(fmt)]; }

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 is the top half of a binary32. */
float orc_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* Nearest bfloat16, ties to the even bit pattern (plain definition: compare
 * the two neighbouring bf16 values).  Used only for the bf16 GEMM operands
 * of the dequantize-to-bf16 path. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u = f2u(f);
    uint16_t lo = (uint16_t)(u >> 16);           /* truncation toward zero    */
    uint16_t hi = (uint16_t)(lo + 1);            /* next magnitude up         */
    double dlo = fabs((double)f - (double)orc_bf16_to_f32(lo));
    double dhi = fabs((double)f - (double)orc_bf16_to_f32(hi));
    if ((u & 0xFFFFu) == 0) return lo;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1) ? hi : lo;
}

/* Round-to-nearest onto the grid, ties to the even code index.
 * [UFP4-TW] 二: nearest-even rounding (RTNE); every value in [1.75, 2.5] goes
 * to 2.  [IF4] 3.1.1 uses Python round(), which is half-to-even.
 * Plain definition: the grid point at the smallest distance; the distances are
 * exact in binary64 near every tie, because a and the grid points are short
 * binary fractions.  Above the grid maximum the nearest point is the maximum
 * (saturation).  The sign bit of z becomes bit 3 of the code. */
int orc_round_rtne(float z, int fmt)
{
    const double *g = grid_of(fmt);
    const int km = kmax_of(fmt);
    double a = fabs((double)z);
    /* at or above the largest point that point is nearest (saturation); the
     * explicit test keeps binary64 distances from losing their order for
     * huge |z| */
    if (a >= g[km]) return (signbit(z) ? 8 : 0) | km;
    int best = 0;
    double bestd = fabs(g[0] - a);
    for (int k = 1; k <= km; ++k) {
        double d = fabs(g[k] - a);
        if (d < bestd || (d == bestd && (k % 2) == 0 && (best % 2) != 0)) {
            best = k;
            bestd = d;
        }
    }
    return (signbit(z) ? 8 : 0) | best;
}

/* Stochastic rounding: [IF4] 6.1 gives floor(x) + (random() < frac); [UFP4-TW]
 * 五 applies it to dY only.  On a non-uniform grid "floor" is the grid point
 * just below |z| and frac the position inside that cell.  The pages fix no
 * resolution; here both sides of the comparison have 16 bits: frac is cut to
 * F = floor(frac 2^16) and random() is U 2^-16 with U = 2^16 - 1 - (w >> 16),
 * the complement of the element's 16 random bits, which orc_sr_word puts in
 * the top half of w (the low half is ignored).  The element rounds up when
 * U < F, i.e. when (w >> 16) + F reaches 2^16; so P(up) = F 2^-16, within
 * 2^-16 below frac, and an |z| less than 2^-16 of a cell above its lower
 * point always rounds down.  |z| at or above the grid maximum gives the
 * maximum.  (F is exact: frac is a short binary fraction, the cell widths
 * being powers of two.) */
int orc_round_sr(float z, int fmt, uint32_t w)
{
    const double *g = grid_of(fmt);
    const int km = kmax_of(fmt);
    double a = fabs((double)z);
    int k;
    if (a >= g[km]) {
        k = km;
    } else {
        int lo = 0;
        for (int j = 1; j <= km; ++j)
            if (g[j] <= a) lo = j;
        double frac = (a - g[lo]) / (g[lo + 1] - g[lo]);
        uint32_t F = (uint32_t)floor(frac * 0x1p16);
        uint32_t U = 0xFFFFu - (w >> 16);
        k = lo + (U < F ? 1 : 0);
    }
    return (signbit(z) ? 8 : 0) | k;
}

/* OCP E4M3FN (bias 7, no infinities, 0x7F is NaN): value of a byte with the
 * sign bit clear.  [IF4] 2.2 table: NVFP4's E4M3 scale spans 448 down to
 * 2^-9. */
float orc_e4m3_decode(uint8_t b)
{
    int e = (b >> 3) & 15, m = b & 7;
    if (e == 0) return (float)ldexp((double)m, -9);
    return (float)ldexp((double)(8 + m), e - 10);
}

/* Encode a non-negative binary32 as E4M3FN: the nearest finite E4M3 value,
 * ties to the even byte (= even mantissa), anything above 448 saturating to
 * 448 (0x7E) -- nearest-point search over the 127 finite non-negative codes.
 * The pages state neither the rounding nor the saturation; this is the
 * conversion NVFP4-style scale encoding uses. */
uint8_t orc_e4m3_encode(float v)
{
    double a = (double)v;
    if (!(a <= 448.0)) return 0x7E; /* above the largest finite value (or inf) */
    int best = 0;
    double bestd = fabs(a - 0.0);
    for (int b = 1; b <= 0x7E; ++b) {
        double d = fabs(a - (double)orc_e4m3_decode((uint8_t)b));
        if (d < bestd || (d == bestd && (b % 2) == 0 && (best % 2) != 0)) {
            best = b;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* MXFP4 shared exponent: [MXFP4] -- one E8M0 exponent per 32 elements (OCP MX).
 * Reading: E = floor(log2(amax)) - 2, 2 being the largest exponent of E2M1,
 * clamped to the E8M0 range [-127, 127]; an all-zero block gets -127.
 * floor(log2) comes from frexp (exact). */
int orc_e8m0_exponent(float amax)
{
    if (amax == 0.0f) return -127;
    int ex;
    frexp((double)amax, &ex); /* amax = f * 2^ex, f in [0.5, 1) */
    int e = (ex - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 [PHILOX]                                                     */
/* ------------------------------------------------------------------------ */
static void mulhilo32(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo)
{
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

/* Ten rounds of the Philox-4x32 S-box/P-box round from the SC'11 paper:
 * two 32x32->64 multiplies by the paper's constants, the high halves XORed
 * with the other two words and the round key; the key advances by the two
 * Weyl constants (golden ratio and sqrt(3)-1) between rounds. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo32(0xD2511F53u, c0, &hi0, &lo0);
        mulhilo32(0xCD9E8D57u, c2, &hi1, &lo1);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The SR random bits of element n of a quantization view, in the top half of
 * the returned word (the low half zero).  The view's elements read Philox's
 * 32-bit output stream 16 bits at a time, low half first: element n takes
 * half n mod 2 of word (n / 2) mod 4 of the block at key = (seed lo, seed hi),
 * counter = (lo32(n/8), hi32(n/8), stream, 0). */
uint32_t orc_sr_word(uint64_t seed, uint32_t stream, uint64_t n)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint64_t q = n >> 3;
    uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), stream, 0u};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    uint32_t word = out[(n >> 1) & 3];
    uint32_t half = (n & 1) ? (word >> 16) : (word & 0xFFFFu);
    return half << 16;
}

/* ------------------------------------------------------------------------ */
/* Hadamard transform                                                        */
/* ------------------------------------------------------------------------ */

/* The 16 signs of the RHT diagonal.  [UFP4-ZC] "治病药反而喂养了病菌": RHT is a
 * random orthogonal rotation before quantization; [UFP4-TW] 六: Hadamard block
 * = quantization block = 16.  Reading: one diagonal d of 16 signs per tensor,
 * d_i = -1 iff bit i of Philox word 0 at key = seed, counter = (0,0,"RHT\0",0).
 * The deterministic H16 of [MXFP4] (its fixed, unrandomised rotation) has d = +1.
 * Returns the 16-bit mask of negative positions. */
uint32_t orc_rht_sign_mask(int rht_kind, uint64_t seed)
{
    if (rht_kind != ORC_RHT_RANDOM) return 0u;
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t ctr[4] = {0u, 0u, 0x52485400u, 0u};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return out[0] & 0xFFFFu;
}

/* 16-point fast Walsh-Hadamard transform in binary32, natural (Sylvester)
 * order, butterfly spans h = 1, 2, 4, 8 in that order, each butterfly
 * (a, b) -> (a + b, a - b), then a multiply by 1/4 so the transform is
 * orthonormal.  The pages give the block size only ([UFP4-TW] 六); the
 * ordering, stage order and normalisation are this reading. */
void orc_fwht16(float v[16])
{
    for (int h = 1; h < 16; h <<= 1)
        for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    for (int i = 0; i < 16; ++i) v[i] = v[i] * 0.25f;
}

/* ------------------------------------------------------------------------ */
/* Tensor views                                                              */
/* ------------------------------------------------------------------------ */
/* A quantization runs along rows (axis ROW) or down columns (axis COL).  The
 * "view" has V rows of L elements, blocks run along the view row:
 *   ROW: V = R, L = C, view(v, l) = x[v][l]
 *   COL: V = C, L = R, view(v, l) = x[l][v]
 * Codes are stored [V][L/2], scales [V][L/B]. */
static float load_src(const void *x, int dtype, int64_t ld, int64_t r, int64_t c)
{
    if (dtype == ORC_BF16) return orc_bf16_to_f32(((const uint16_t *)x)[r * ld + c]);
    return ((const float *)x)[r * ld + c];
}

static float load_view(const void *x, int dtype, int64_t ld, int axis, int64_t v, int64_t l)
{
    return axis == ORC_ROW ? load_src(x, dtype, ld, v, l) : load_src(x, dtype, ld, l, v);
}

/* One view row after the optional RHT: y[0..L). */
static void view_row_transformed(const void *x, int dtype, int64_t ld, int axis, int64_t v, int64_t L,
                                 int rht, uint32_t smask, float *y)
{
    for (int64_t l = 0; l < L; ++l) y[l] = load_view(x, dtype, ld, axis, v, l);
    if (rht == ORC_RHT_NONE) return;
    for (int64_t c0 = 0; c0 < L; c0 += 16) {
        float t[16];
        for (int i = 0; i < 16; ++i) t[i] = ((smask >> i) & 1u) ? -y[c0 + i] : y[c0 + i];
        orc_fwht16(t);
        for (int i = 0; i < 16; ++i) y[c0 + i] = t[i];
    }
}

/* Standalone transform of view rows [v0, v1) into y (row-major view, ld L). */
int orc_rht_view(const void *x, int dtype, int64_t R, int64_t C, int64_t ld, int axis, int rht,
                 uint64_t seed, int64_t v0, int64_t v1, float *y)
{
    int64_t L = axis == ORC_ROW ? C : R;
    if (L % 16) return -1;
    uint32_t smask = orc_rht_sign_mask(rht, seed);
    for (int64_t v = v0; v < v1; ++v) view_row_transformed(x, dtype, ld, axis, v, L, rht, smask, y + (v - v0) * L);
    return 0;
}

/* Tensor amax after the transform, for the two-level scale.
 * [IF4] 3.2: alpha = max|X| / (6 x 448); the tensor that is quantized is the
 * transformed one, so the max is taken after the RHT. */
float orc_amax(const void *x, int dtype, int64_t R, int64_t C, int64_t ld, const orc_config *cfg)
{
    int64_t V = cfg->axis == ORC_ROW ? R : C, L = cfg->axis == ORC_ROW ? C : R;
    uint32_t smask = orc_rht_sign_mask(cfg->rht, cfg->rht_seed);
    float *y = (float *)malloc(sizeof(float) * (size_t)L);
    float m = 0.0f;
    for (int64_t v = 0; v < V; ++v) {
        view_row_transformed(x, dtype, ld, cfg->axis, v, L, cfg->rht, smask, y);
        for (int64_t l = 0; l < L; ++l) {
            float a = fabsf(y[l]);
            if (a > m) m = a;
        }
    }
    free(y);
    return m;
}

/* The constant G in alpha = A_t / G: grid maximum times 448, the largest
 * E4M3 value ([IF4] 2.2: NVFP4 max 6x448, NVINT4 max 7x448; E1M2 3.5x448). */
float orc_two_level_denominator(int fmt) { return orc_gridmax(fmt) * 448.0f; }

/* ------------------------------------------------------------------------ */
/* Block quantization                                                        */
/* ------------------------------------------------------------------------ */

/* Per-block result used by quantize and stats. */
typedef struct {
    float s_eff;      /* effective scale: x_hat = value * s_eff          */
    int int4;         /* IF4 only: 1 if the block chose INT4            */
    uint8_t scale_b;  /* stored byte (E4M3 / E8M0 / IF4)               */
    float scale_f;    /* stored FP32 scale                               */
    int code[32];
    float zabs[32];   /* |scaled value| before rounding (stats)        */
    float xhat[32];   /* dequantized value                               */
} orc_block;

/* Scaled value z = y / s ([IF4] 3.1.1 pseudo-code divides by the scale),
 * correctly rounded binary32 division; a zero scale gives z = +0. */
static float scaled(float y, float s) { return s == 0.0f ? 0.0f : y / s; }

/* Dequantized value of a code on a plain grid: its grid value times the
 * block's effective scale ([IF4] 3.1.1). */
static float deq_plain(int fmt, int code, float s)
{
    float v = (float)orc_grid_value(fmt, code & 7);
    if (code & 8) v = -v;
    return v * s;
}

/* IF4's INT4 candidate ([IF4] 3.1.1, 3.2).  The integer grid reaches 7 while
 * E2M1 reaches 6, so with the shared block scale the integer levels are
 * stretched: a value in units of the scale is enlarged by 7/6 before it is
 * rounded to a level, and a level stands for 6/7 of (level x scale).  Reading
 * in binary32 (each step rounded once): with z = RN(y / s), the quotient the
 * E2M1 candidate rounds, the level is |RN(z * 7/6)| rounded half to even and
 * capped at 7; its value is RN(RN(level * s) * 6/7), where 7/6 and 6/7 are
 * the binary32 constants nearest them. */
static const float IF4_STRETCH = 7.0f / 6.0f;
static const float IF4_SHRINK = 6.0f / 7.0f;

static int if4_int_code(float z)
{
    float t = z * IF4_STRETCH;
    int level = (int)nearbyintf(fabsf(t)); /* default rounding mode: half to even */
    if (level > 7) level = 7;
    return (signbit(t) ? 8 : 0) | level;
}

static float if4_int_value(int code, float s)
{
    float level = (float)(code & 7);
    if (code & 8) level = -level;
    float scaled_level = level * s;
    return scaled_level * IF4_SHRINK;
}

/* Quantize one block of B transformed values y[0..B). */
static void quantize_block(const orc_config *cfg, const float *y, int B, float alpha, uint64_t n0,
                           orc_block *out)
{
    int fmt = cfg->format;
    float gmax = orc_gridmax(fmt);
    float m = 0.0f;                                   /* block amax ([IF4] 3.1.1) */
    for (int i = 0; i < B; ++i) {
        float a = fabsf(y[i]);
        if (a > m) m = a;
    }
    float s;
    out->int4 = 0;
    out->scale_b = 0;
    out->scale_f = 0.0f;
    if (cfg->scale == ORC_SCALE_FP32) {
        /* Single-level FP32 scale ([UFP4-ZC] recipe table; [UFP4-TW] 五):
         * s = amax / gridmax. */
        s = m / gmax;
        out->scale_f = s;
    } else if (cfg->scale == ORC_SCALE_E4M3) {
        /* Two-level scale ([IF4] 3.2): Delta = amax_block / (alpha x 6),
         * stored as E4M3; the effective scale is alpha x Delta_q. */
        float den = alpha * gmax;
        float delta = den == 0.0f ? 0.0f : m / den;
        uint8_t e = orc_e4m3_encode(delta);
        s = alpha * orc_e4m3_decode(e);
        out->scale_b = e;
    } else {
        /* E8M0 power-of-two scale ([MXFP4]). */
        int e = orc_e8m0_exponent(m);
        s = ldexpf(1.0f, e);
        out->scale_b = (uint8_t)(e + 127);
    }
    out->s_eff = s;

    if (fmt != ORC_IF4) {
        for (int i = 0; i < B; ++i) {
            float z = scaled(y[i], s);
            int code;
            if (s == 0.0f) {
                code = 0;
            } else if (cfg->rounding == ORC_SR) {
                code = orc_round_sr(z, fmt, orc_sr_word(cfg->sr_seed, cfg->sr_stream, n0 + (uint64_t)i));
            } else {
                code = orc_round_rtne(z, fmt);
            }
            out->code[i] = code;
            out->zabs[i] = fabsf(z);
            out->xhat[i] = deq_plain(fmt, code, s);
        }
        return;
    }

    /* IF4 ([IF4] 3.1, 3.2): every block gets both an E2M1 and an INT4
     * candidate under the same scale; the one whose reconstruction is closer
     * (smaller sum of squared errors) is kept, and bit 7 of the scale byte
     * records which (1 = INT4).  Readings: the errors are measured in units of
     * the block scale, against z = RN(y / s): g - z for the E2M1 grid value g,
     * and level * 6/7 - z rounded once (a fused multiply-add) for the signed
     * INT4 level (in exact arithmetic both are the reconstruction's error
     * divided by s, so the ranking is the same); each candidate's squares are
     * accumulated in element order, each square fused into the running sum
     * (one rounding per element, as a dot product of the errors with
     * themselves), and an exact tie keeps E2M1. */
    int fp4_code[16], int_code[16];
    float fp4_z[16], int_z[16], fp4_val[16], int_val[16];
    float fp4_sq = 0.0f, int_sq = 0.0f;
    for (int i = 0; i < B; ++i) {
        if (s == 0.0f) {
            fp4_code[i] = int_code[i] = 0;
            fp4_z[i] = int_z[i] = 0.0f;
        } else {
            fp4_z[i] = scaled(y[i], s);
            fp4_code[i] = orc_round_rtne(fp4_z[i], ORC_E2M1);
            int_code[i] = if4_int_code(fp4_z[i]);
            int_z[i] = fp4_z[i] * IF4_STRETCH;
        }
        fp4_val[i] = deq_plain(ORC_E2M1, fp4_code[i], s);
        int_val[i] = if4_int_value(int_code[i], s);
        float g = (float)grid_of(ORC_E2M1)[fp4_code[i] & 7];
        if (fp4_code[i] & 8) g = -g;
        float level = (float)(int_code[i] & 7);
        if (int_code[i] & 8) level = -level;
        float dev_fp4 = g - fp4_z[i];
        float dev_int = fmaf(level, IF4_SHRINK, -fp4_z[i]);
        fp4_sq = fmaf(dev_fp4, dev_fp4, fp4_sq);
        int_sq = fmaf(dev_int, dev_int, int_sq);
    }
    int use_int = (s != 0.0f) && (int_sq < fp4_sq);
    out->int4 = use_int;
    out->scale_b = (uint8_t)(out->scale_b | (use_int ? 0x80 : 0));
    for (int i = 0; i < B; ++i) {
        out->code[i] = use_int ? int_code[i] : fp4_code[i];
        out->zabs[i] = use_int ? fabsf(int_z[i]) : fabsf(fp4_z[i]);
        out->xhat[i] = use_int ? int_val[i] : fp4_val[i];
    }
}

static int config_ok(const orc_config *c)
{
    if (c->block != 16 && c->block != 32) return 0;
    if (c->format < 0 || c->format > 6) return 0;
    if (c->format == ORC_IF4 && (c->scale != ORC_SCALE_E4M3 || c->block != 16 || c->rounding != ORC_RTNE)) return 0;
    if (c->format >= ORC_E2M1_MAX4 && (c->scale == ORC_SCALE_E8M0 || c->rounding != ORC_RTNE)) return 0;
    if (c->scale == ORC_SCALE_E8M0 && (c->format != ORC_E2M1 || c->block != 32)) return 0;
    if (c->scale != ORC_SCALE_E8M0 && c->block != 16) return 0;
    return 1;
}

/* Quantize view rows [v0, v1).  Outputs are written for those rows only, at
 * their positions in the full [V][L/2] / [V][L/B] arrays.  amax is the
 * tensor amax for the two-level scale (ignored otherwise).  Returns alpha for
 * E4M3 scales (0 otherwise), or a negative value on a bad argument. */
float orc_quantize(const void *x, int dtype, int64_t R, int64_t C, int64_t ld, const orc_config *cfg,
                   float amax, int64_t v0, int64_t v1, uint8_t *codes, void *scales)
{
    if (!config_ok(cfg)) return -1.0f;
    int64_t V = cfg->axis == ORC_ROW ? R : C, L = cfg->axis == ORC_ROW ? C : R;
    int B = cfg->block;
    if (L % B) return -2.0f;
    (void)V;
    float alpha = 0.0f;
    if (cfg->scale == ORC_SCALE_E4M3) alpha = amax / orc_two_level_denominator(cfg->format);
    uint32_t smask = orc_rht_sign_mask(cfg->rht, cfg->rht_seed);
    float *y = (float *)malloc(sizeof(float) * (size_t)L);
    orc_block blk;
    for (int64_t v = v0; v < v1; ++v) {
        view_row_transformed(x, dtype, ld, cfg->axis, v, L, cfg->rht, smask, y);
        for (int64_t b = 0; b < L / B; ++b) {
            quantize_block(cfg, y + b * B, B, alpha, (uint64_t)(v * L + b * B), &blk);
            for (int i = 0; i < B; i += 2) {
                codes[(v * L + b * B + i) / 2] = (uint8_t)(blk.code[i] | (blk.code[i + 1] << 4));
            }
            if (cfg->scale == ORC_SCALE_FP32)
                ((float *)scales)[v * (L / B) + b] = blk.scale_f;
            else
                ((uint8_t *)scales)[v * (L / B) + b] = blk.scale_b;
        }
    }
    free(y);
    return alpha;
}

/* Effective scale and type flag of a stored block. */
static float stored_scale(const orc_config *cfg, const void *scales, int64_t idx, float alpha, int *int4)
{
    *int4 = 0;
    if (cfg->scale == ORC_SCALE_FP32) return ((const float *)scales)[idx];
    uint8_t b = ((const uint8_t *)scales)[idx];
    if (cfg->scale == ORC_SCALE_E8M0) return ldexpf(1.0f, (int)b - 127);
    if (cfg->format == ORC_IF4) *int4 = (b >> 7) & 1;
    return alpha * orc_e4m3_decode((uint8_t)(b & 0x7F));
}

/* Dequantize view rows [v0, v1) to binary32 ([IF4] 3.1.1: code x scale, and
 * x 6/7 for IF4's INT4 blocks).  With inverse != 0 the RHT is undone: the
 * transform is its own inverse up to the sign diagonal, so apply the FWHT
 * (x 1/4) and then the signs.  Output is the view, row-major, ld L. */
int orc_dequantize(const orc_config *cfg, int64_t R, int64_t C, const uint8_t *codes, const void *scales,
                   float alpha, int inverse, int64_t v0, int64_t v1, float *out)
{
    if (!config_ok(cfg)) return -1;
    int64_t L = cfg->axis == ORC_ROW ? C : R;
    int B = cfg->block;
    uint32_t smask = orc_rht_sign_mask(cfg->rht, cfg->rht_seed);
    for (int64_t v = v0; v < v1; ++v) {
        float *o = out + (v - v0) * L;
        for (int64_t l = 0; l < L; ++l) {
            int64_t e = v * L + l;
            int code = (codes[e / 2] >> (4 * (e & 1))) & 15;
            int int4;
            float s = stored_scale(cfg, scales, v * (L / B) + l / B, alpha, &int4);
            o[l] = int4 ? if4_int_value(code, s) : deq_plain(cfg->format, code, s);
        }
        if (inverse && cfg->rht != ORC_RHT_NONE) {
            for (int64_t c0 = 0; c0 < L; c0 += 16) {
                orc_fwht16(o + c0);
                for (int i = 0; i < 16; ++i)
                    if ((smask >> i) & 1u) o[c0 + i] = -o[c0 + i];
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Statistics                                                                */
/* ------------------------------------------------------------------------ */
/* The quantities the pages use to describe quantization quality:
 * SQNR ([UFP4-ZC] "治病药反而喂养了病菌": 21.90 vs 19.94 dB; [UFP4-TW] 四),
 * the signal factor alpha of A_hat = alpha A + R ([UFP4-ZC] "复利效应的反向版本"),
 * per-cell rounding bias ([UFP4-ZC] "E2M1：一块刻度不均的尺子"; [UFP4-TW] 二),
 * bucket use ([UFP4-ZC]), and the IF4 type shares ([IF4] 6.2).
 * Layout of the 48 binary64 sums (same meaning as the library's):
 *  0 n          1 sum y^2      2 sum e^2     3 sum e       4 sum sign(y) e
 *  5 sum xhat y 6 sum |e|      7 blocks      8 INT4 blocks
 *  16 + 8t + k  count of magnitude code k in blocks of type t (0 grid/FP4, 1 INT4)
 *  32 + 8t + k  sum of (g_t[k] - |z|) over those elements
 * e = xhat - y, computed in binary64 from the binary32 values. */
#define ORC_NSUMS 48

int orc_stats(const void *x, int dtype, int64_t R, int64_t C, int64_t ld, const orc_config *cfg, float amax,
              int64_t v0, int64_t v1, double *sums)
{
    if (!config_ok(cfg)) return -1;
    int64_t L = cfg->axis == ORC_ROW ? C : R;
    int B = cfg->block;
    float alpha = 0.0f;
    if (cfg->scale == ORC_SCALE_E4M3) alpha = amax / orc_two_level_denominator(cfg->format);
    uint32_t smask = orc_rht_sign_mask(cfg->rht, cfg->rht_seed);
    float *y = (float *)malloc(sizeof(float) * (size_t)L);
    orc_block blk;
    for (int i = 0; i < ORC_NSUMS; ++i) sums[i] = 0.0;
    for (int64_t v = v0; v < v1; ++v) {
        view_row_transformed(x, dtype, ld, cfg->axis, v, L, cfg->rht, smask, y);
        for (int64_t b = 0; b < L / B; ++b) {
            quantize_block(cfg, y + b * B, B, alpha, (uint64_t)(v * L + b * B), &blk);
            int t = blk.int4;
            const double *g = t ? GRID[ORC_INT4] : grid_of(cfg->format);
            sums[7] += 1.0;
            sums[8] += t;
            for (int i = 0; i < B; ++i) {
                double yy = y[b * B + i], xh = blk.xhat[i], e = xh - yy;
                sums[0] += 1.0;
                sums[1] += yy * yy;
                sums[2] += e * e;
                sums[3] += e;
                sums[4] += (yy > 0 ? 1.0 : (yy < 0 ? -1.0 : 0.0)) * e;
                sums[5] += xh * yy;
                sums[6] += fabs(e);
                int k = blk.code[i] & 7;
                sums[16 + 8 * t + k] += 1.0;
                sums[32 + 8 * t + k] += g[k] - (double)blk.zabs[i];
            }
        }
    }
    free(y);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* GEMM references                                                           */
/* ------------------------------------------------------------------------ */
/* Z[m][n] = sum_k A[m][k] B[n][k] in binary64 for rows m in [m0, m1):
 * the plain definition of the product of two K-major operands
 * ([UFP4-ZC] "复利效应的反向版本": Z_q = A_hat B_hat^T). */
void orc_gemm_nt_f32(const float *A, const float *B, int64_t N, int64_t K, int64_t m0, int64_t m1, double *Z)
{
    for (int64_t m = m0; m < m1; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            const float *a = A + (m - m0) * K, *b = B + n * K;
            for (int64_t k = 0; k < K; ++k) acc += (double)a[k] * (double)b[k];
            Z[(m - m0) * N + n] = acc;
        }
}

/* Attenuation of a GEMM output ([UFP4-ZC] "复利效应的反向版本"): a quantized
 * operand behaves like a shrunk copy of the exact one plus noise that is
 * uncorrelated with it, so the quantized product Zq carries a factor eta of
 * the exact product Z = A B^T (both operands' factors multiplied) plus noise.
 * eta is the least-squares factor <Zq, Z> / <Z, Z>; the output SQNR is
 * 10 log10(<Z, Z> / ||Zq - Z||^2).  The three binary64 sums, element by
 * element in index order: out[0] = <Zq, Z>, out[1] = <Z, Z>,
 * out[2] = ||Zq - Z||^2. */
void orc_eta_sums(const double *zq, const double *z, int64_t n, double out[3])
{
    double cross = 0.0, ref = 0.0, err = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double d = zq[i] - z[i];
        cross += zq[i] * z[i];
        ref += z[i] * z[i];
        err += d * d;
    }
    out[0] = cross;
    out[1] = ref;
    out[2] = err;
}

/* Number of sums in a statistics record. */
int orc_nsums(void) { return ORC_NSUMS; }

/* ------------------------------------------------------------------------ */
/* Array forms of the scalar steps (loops over the functions above; used by   */
/* the pin tests to sweep many binary32 values).                             */
/* ------------------------------------------------------------------------ */
void orc_round_rtne_array(const float *z, int64_t n, int fmt, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_round_rtne(z[i], fmt);
}

void orc_round_sr_array(const float *z, const uint32_t *w, int64_t n, int fmt, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_round_sr(z[i], fmt, w[i]);
}

void orc_e4m3_encode_array(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

void orc_f32_to_bf16_array(const float *f, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(f[i]);
}

void orc_sr_word_array(uint64_t seed, uint32_t stream, uint64_t n0, int64_t n, uint32_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_sr_word(seed, stream, n0 + (uint64_t)i);
}
