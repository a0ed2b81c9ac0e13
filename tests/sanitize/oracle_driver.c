/*
 * oracle_driver.c -- exercises every entry point of the CPU oracle
 * (oracle/oracle.c, oracle/kvcache.c) on small, ragged shapes with buffers of
 * exactly the documented sizes, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer reports any out-of-bounds access, use of freed
 * memory, signed overflow or bad shift.  Host code only; the test suite
 * compiles and runs it (tests/test_oracle_sanitize.py).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t format, scale, block, rht, rounding, axis;
    uint64_t rht_seed, sr_seed;
    uint32_t sr_stream, reserved;
} orc_config;

float orc_amax(const void *x, int dtype, int64_t R, int64_t C, int64_t ld, const orc_config *cfg);
float orc_quantize(const void *x, int dtype, int64_t R, int64_t C, int64_t ld, const orc_config *cfg, float amax,
                   int64_t v0, int64_t v1, uint8_t *codes, void *scales);
int orc_dequantize(const orc_config *cfg, int64_t R, int64_t C, const uint8_t *codes, const void *scales, float alpha,
                   int inverse, int64_t v0, int64_t v1, float *out);
int orc_stats(const void *x, int dtype, int64_t R, int64_t C, int64_t ld, const orc_config *cfg, float amax,
              int64_t v0, int64_t v1, double *sums);
int orc_rht_view(const void *x, int dtype, int64_t R, int64_t C, int64_t ld, int axis, int rht, uint64_t seed,
                 int64_t v0, int64_t v1, float *y);
void orc_gemm_nt_f32(const float *A, const float *B, int64_t N, int64_t K, int64_t m0, int64_t m1, double *Z);
void orc_eta_sums(const double *zq, const double *z, int64_t n, double out[3]);
uint16_t orc_f32_to_bf16(float f);
uint8_t orc_e4m3_encode(float v);
int orc_e8m0_exponent(float amax);
uint32_t orc_sr_word(uint64_t seed, uint32_t stream, uint64_t n);
void orc_q_quantize(const uint16_t *q, int D, int rotate, uint8_t *codes, uint8_t *scales);
void orc_kv_quantize_seq(const uint16_t *k, const uint16_t *v, int64_t tok_stride, int64_t len, int64_t ntok, int D,
                         int rotate, int fp8, uint8_t *kcodes, uint8_t *kscales, uint8_t *vcodes, uint8_t *vscales);
int orc_kv_decode_seq(const uint16_t *q, int G, const uint16_t *k, const uint16_t *v, int64_t tok_stride, int64_t len,
                      int D, float sm_scale, int rotate, int fp8, double *out);
int orc_kv_decode_bounds(const uint16_t *q, int G, const uint16_t *k, const uint16_t *v, int64_t tok_stride,
                         int64_t len, int D, float sm_scale, int rotate, int fp8, double eps_s, double *mass,
                         double *amb, int64_t *fragile);

static uint64_t lcg = 12345;
static float urand(void) /* uniform in [-1, 1) */
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((lcg >> 40) * 0x1p-24) * 2.0f - 1.0f;
}

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) exit(3);
    return p;
}

/* bf16 source [R][ld] with a mix of magnitudes, zeros and outliers */
static uint16_t *bf16_source(int64_t R, int64_t C, int64_t ld)
{
    uint16_t *x = xmalloc(sizeof(uint16_t) * (size_t)(R * ld));
    for (int64_t i = 0; i < R * ld; ++i) {
        float v = urand();
        if (i % 97 == 0) v *= 50.0f;
        if (i % 89 == 0) v = 0.0f;
        if (i % 211 == 0) v *= 1e-30f;
        x[i] = orc_f32_to_bf16(v);
    }
    (void)C;
    return x;
}

static int run_config(int64_t R, int64_t C, int64_t ld, orc_config cfg)
{
    const int64_t V = cfg.axis == 0 ? R : C, L = cfg.axis == 0 ? C : R;
    uint16_t *x = bf16_source(R, C, ld);
    float amax = orc_amax(x, 0, R, C, ld, &cfg);
    uint8_t *codes = xmalloc((size_t)(V * L / 2));
    const size_t sbytes = (size_t)(V * (L / cfg.block)) * (cfg.scale == 0 ? 4 : 1);
    void *scales = xmalloc(sbytes);
    float alpha = orc_quantize(x, 0, R, C, ld, &cfg, amax, 0, V, codes, scales);
    if (alpha < 0.0f) return 1;
    float *deq = xmalloc(sizeof(float) * (size_t)(V * L));
    if (orc_dequantize(&cfg, R, C, codes, scales, alpha, 1, 0, V, deq)) return 2;
    double sums[48];
    if (orc_stats(x, 0, R, C, ld, &cfg, amax, 0, V, sums)) return 3;
    float *y = xmalloc(sizeof(float) * (size_t)(V * L));
    if (orc_rht_view(x, 0, R, C, ld, cfg.axis, cfg.rht, cfg.rht_seed, 0, V, y)) return 4;
    free(x), free(codes), free(scales), free(deq), free(y);
    return 0;
}

int main(void)
{
    /* every supported combination of format, scale, rounding, transform and
     * axis on ragged shapes (rows and columns not multiples of 256) */
    struct { int fmt, scale, block, rounding; } combos[] = {
        {0, 0, 16, 0}, {0, 1, 16, 0}, {0, 2, 32, 0}, {0, 0, 16, 1}, {0, 1, 16, 1}, {1, 0, 16, 0},
        {1, 1, 16, 0}, {1, 0, 16, 1}, {1, 1, 16, 1}, {2, 0, 16, 0}, {2, 1, 16, 1}, {3, 1, 16, 0},
        {4, 0, 16, 0}, {5, 1, 16, 0}, {6, 0, 16, 0}};
    const int64_t shapes[][3] = {{32, 48, 48}, {64, 96, 104}, {96, 32, 40}, {32, 32, 32}};
    int n = 0;
    for (size_t c = 0; c < sizeof(combos) / sizeof(combos[0]); ++c)
        for (int axis = 0; axis < 2; ++axis)
            for (int rht = 0; rht < 3; ++rht)
                for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
                    orc_config cfg = {combos[c].fmt, combos[c].scale, combos[c].block, rht, combos[c].rounding,
                                      axis, 77, 5, (uint32_t)axis, 0};
                    const int64_t L = axis == 0 ? shapes[s][1] : shapes[s][0];
                    if (L % cfg.block) continue;
                    int rc = run_config(shapes[s][0], shapes[s][1], shapes[s][2], cfg);
                    if (rc) {
                        fprintf(stderr, "config %zu axis %d rht %d shape %zu failed: %d\n", c, axis, rht, s, rc);
                        return 1;
                    }
                    ++n;
                }
    /* scalar helpers over their whole input ranges */
    for (int i = 0; i < 100000; ++i) {
        float v = urand() * 500.0f;
        (void)orc_e4m3_encode(v < 0 ? -v : v);
        (void)orc_e8m0_exponent(v < 0 ? -v : v);
        (void)orc_sr_word((uint64_t)i * 2654435761u, (uint32_t)i, (uint64_t)i << 20);
    }
    (void)orc_e8m0_exponent(0.0f);
    (void)orc_e8m0_exponent(3.0e38f);
    /* GEMM and attenuation */
    {
        const int64_t M = 5, N = 7, K = 48;
        float *A = xmalloc(sizeof(float) * M * K), *B = xmalloc(sizeof(float) * N * K);
        for (int64_t i = 0; i < M * K; ++i) A[i] = urand();
        for (int64_t i = 0; i < N * K; ++i) B[i] = urand();
        double *Z = xmalloc(sizeof(double) * M * N), *Zq = xmalloc(sizeof(double) * M * N);
        orc_gemm_nt_f32(A, B, N, K, 0, M, Z);
        orc_gemm_nt_f32(A, B, N, K, 1, 3, Zq);
        double e[3];
        orc_eta_sums(Zq, Z, 2 * N, e);
        free(A), free(B), free(Z), free(Zq);
    }
    /* KV cache: ragged lengths, both formats, rotated or not */
    {
        const int D = 128, G = 3;
        const int64_t lens[] = {0, 1, 31, 33, 100};
        for (size_t li = 0; li < sizeof(lens) / sizeof(lens[0]); ++li)
            for (int fp8 = 0; fp8 < 2; ++fp8)
                for (int rot = 0; rot < 2; ++rot) {
                    const int64_t len = lens[li], ntok = (len + 31) / 32 * 32, stride = D + 8;
                    const int64_t T = len > 0 ? len : 1;
                    uint16_t *k = bf16_source(T, D, stride), *v = bf16_source(T, D, stride);
                    uint16_t *q = bf16_source(G, D, D);
                    uint8_t qc[128], qs[4];
                    orc_q_quantize(q, D, rot, qc, qs);
                    const int64_t cb = fp8 ? 1 : 2;
                    uint8_t *kc = xmalloc((size_t)(ntok * D / cb)), *ks = xmalloc((size_t)(ntok * D / 32));
                    uint8_t *vc = xmalloc((size_t)(D * ntok / cb)), *vs = xmalloc((size_t)(D * ntok / 32));
                    orc_kv_quantize_seq(k, v, stride, len, ntok, D, rot, fp8, kc, ks, vc, vs);
                    double *out = xmalloc(sizeof(double) * G * D), *mass = xmalloc(sizeof(double) * G * D);
                    double *amb = xmalloc(sizeof(double) * G * D);
                    int64_t fragile = 0;
                    if (orc_kv_decode_seq(q, G, k, v, stride, len, D, 0.088f, rot, fp8, out)) return 5;
                    if (orc_kv_decode_bounds(q, G, k, v, stride, len, D, 0.088f, rot, fp8, 0x1p-15, mass, amb,
                                             &fragile))
                        return 6;
                    free(k), free(v), free(q), free(kc), free(ks), free(vc), free(vs), free(out), free(mass),
                        free(amb);
                }
    }
    printf("oracle driver: %d quantizer configurations and the GEMM, eta and KV entry points ran clean\n", n);
    return 0;
}
