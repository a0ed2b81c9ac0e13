// api.hip -- the C ABI of libufp4 (declared in include/ufp4.h): argument
// validation on the host, then dispatch to the gfx950 kernels.
//
// The operations and their definitions are documented in ufp4.h, with the
// passages of the pages each follows.  Nothing here allocates device memory;
// every launch goes to the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/ufp4.h"
#include "device.hpp"
#include "kernels.hpp"

using namespace ufp4;

static thread_local int g_last_hip_error = 0;

namespace ufp4 {
LaunchTiming &launch_timing()
{
    static thread_local LaunchTiming t;
    return t;
}

int cu_count()
{
    static std::atomic<int> cus[64];
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        n = cus[dev].load(std::memory_order_relaxed);
        if (n <= 0) {
            if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
                (void)hipGetLastError();
                n = 0;
            } else {
                cus[dev].store(n, std::memory_order_relaxed);
            }
        }
    }
    return n > 0 ? n : 256;
}
}  // namespace ufp4

static int hip_fail(hipError_t e)
{
    if (e == hipSuccess) return UFP4_OK;
    g_last_hip_error = (int)e;
    return UFP4_ERR_HIP;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The GEMM kernels address a 256-row tile of an operand through a buffer
// descriptor with 32-bit offsets: row (< 256) times the row stride plus the
// K offset must stay below 2^32 bytes.
static bool gemm_offsets_fit(int64_t row_stride_bytes, int64_t k_bytes)
{
    return 256 * row_stride_bytes + k_bytes < ((int64_t)1 << 32);
}

// Host-side Philox4x32-10 word 0 for the sign diagonal (SC'11 round function).
static uint32_t host_philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1)
{
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}

static uint32_t sign_mask(int rht, uint64_t seed)
{
    if (rht != UFP4_RHT_RANDOM) return 0u;
    return host_philox_word0(0u, 0u, 0x52485400u, 0u, (uint32_t)seed, (uint32_t)(seed >> 32)) & 0xFFFFu;
}

static int check_config(const ufp4_config *c)
{
    if (!c) return UFP4_ERR_INVALID_ARG;
    if (c->format < UFP4_E2M1 || c->format > UFP4_E2M1_MAX2) return UFP4_ERR_INVALID_ARG;
    if (c->scale < UFP4_SCALE_FP32 || c->scale > UFP4_SCALE_E8M0) return UFP4_ERR_INVALID_ARG;
    if (c->rht < UFP4_RHT_NONE || c->rht > UFP4_RHT_DETERMINISTIC) return UFP4_ERR_INVALID_ARG;
    if (c->rounding != UFP4_RTNE && c->rounding != UFP4_SR) return UFP4_ERR_INVALID_ARG;
    if (c->axis != UFP4_ROW && c->axis != UFP4_COL) return UFP4_ERR_INVALID_ARG;
    if (c->block != 16 && c->block != 32) return UFP4_ERR_INVALID_ARG;
    if (c->reserved != 0) return UFP4_ERR_INVALID_ARG;
    if (c->scale == UFP4_SCALE_E8M0) {
        if (c->format != UFP4_E2M1 || c->block != 32 || c->rounding != UFP4_RTNE) return UFP4_ERR_UNSUPPORTED;
    } else if (c->block != 16) {
        return UFP4_ERR_UNSUPPORTED;
    }
    if (c->format == UFP4_IF4 && (c->scale != UFP4_SCALE_E4M3 || c->rounding != UFP4_RTNE))
        return UFP4_ERR_UNSUPPORTED;
    if (c->format >= UFP4_E2M1_MAX4 && c->rounding != UFP4_RTNE) return UFP4_ERR_UNSUPPORTED;
    return UFP4_OK;
}

// Shape/alignment rules of a source x[rows][ldx] read along `axis`.
static int check_source(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int axis, int block)
{
    if (!x && rows * cols > 0) return UFP4_ERR_INVALID_ARG;
    if (dtype != UFP4_BF16 && dtype != UFP4_F32) return UFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0) return UFP4_ERR_SHAPE;
    if (ldx < cols) return UFP4_ERR_SHAPE;
    const int64_t L = axis == UFP4_ROW ? cols : rows;
    if (L % block) return UFP4_ERR_SHAPE;
    if (axis == UFP4_COL && cols % 8) return UFP4_ERR_SHAPE;
    if (!aligned16(x) || ldx % 8) return UFP4_ERR_ALIGN;
    if (rows * cols >= ((int64_t)1 << 40)) return UFP4_ERR_SHAPE;
    return UFP4_OK;
}

static void fill_args(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int axis, uint32_t smask,
                      RowArgs &ra, ColArgs &ca)
{
    memset(&ra, 0, sizeof(ra));
    memset(&ca, 0, sizeof(ca));
    (void)dtype;
    ra.x = x;
    ra.ldx = ldx;
    ra.L = cols;
    ra.n_ch = axis == UFP4_ROW ? rows * cols / 16 : 0;
    ra.contiguous = ldx == cols;
    ra.smask = smask;
    ca.x = x;
    ca.ldx = ldx;
    ca.R = rows;
    ca.C = cols;
    ca.smask = smask;
}

// Built-in scratch of ufp4_amax_noalloc: room for the partial maxima of the
// amax pass (one per workgroup), 256 KiB on every device the library runs
// on, held until the process ends.  Host code never passes the array's name
// to a kernel (on the host it only stands for the symbol); it looks up the
// array's device address once per device, with that device current, and
// uses that address.
static constexpr int64_t AMAX_SCRATCH_FLOATS = 65536;
static __device__ __align__(256) float amax_scratch[AMAX_SCRATCH_FLOATS];
static constexpr int MAX_DEVICES = 64;
static std::mutex g_scratch_lock;
static float *g_amax_scratch[MAX_DEVICES];  // device address per device, null until looked up

static int amax_scratch_of_current_device(float **out)
{
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= MAX_DEVICES) return UFP4_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> guard(g_scratch_lock);
    if (!g_amax_scratch[dev]) {
        void *p = nullptr;
        const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(amax_scratch));
        if (g != hipSuccess || !p) return hip_fail(g != hipSuccess ? g : hipErrorInvalidSymbol);
        g_amax_scratch[dev] = static_cast<float *>(p);
    }
    *out = g_amax_scratch[dev];
    return UFP4_OK;
}

extern "C" {

int ufp4_version(void) { return (0 << 16) | 1; }

const char *ufp4_strerror(int code)
{
    switch (code) {
    case UFP4_OK: return "ok";
    case UFP4_ERR_INVALID_ARG: return "invalid argument (null pointer, unknown enum value or dtype)";
    case UFP4_ERR_SHAPE: return "shape not supported (block multiple, tile multiple or leading dimension)";
    case UFP4_ERR_ALIGN: return "pointer not 16-byte aligned or leading dimension not a multiple of 8";
    case UFP4_ERR_UNSUPPORTED: return "unsupported combination of format, scale, block and rounding";
    case UFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case UFP4_ERR_HIP: return "HIP launch failed (see ufp4_last_hip_error)";
    }
    return "unknown error code";
}

int ufp4_last_hip_error(void) { return g_last_hip_error; }

int ufp4_time_next_launch(void *start_event, void *stop_event)
{
    if ((start_event == nullptr) != (stop_event == nullptr)) return UFP4_ERR_INVALID_ARG;
    launch_timing() = LaunchTiming{(hipEvent_t)start_event, (hipEvent_t)stop_event};
    return UFP4_OK;
}

size_t ufp4_workspace_size(int op, int64_t rows, int64_t cols, const ufp4_config *cfg)
{
    switch (op) {
    case UFP4_OP_STATS: return (size_t)STATS_WGS * UFP4_NSUMS * sizeof(double);
    case UFP4_OP_ETA: return (size_t)ETA_WGS * 3 * sizeof(double);
    case UFP4_OP_AMAX: {
        const int axis = cfg ? cfg->axis : UFP4_ROW;
        const int64_t t = amax_tiles(axis, rows, cols);
        return (size_t)(t > 0 ? t : 1) * sizeof(float);
    }
    case UFP4_OP_QGEMM:
        // the dequantize-to-bf16 mode holds both operands as bf16 ((M + N) x K),
        // whatever their format; the native MXFP4 mode uses none of it
        return rows > 0 && cols > 0 ? (size_t)(rows * cols * 2) : 0;
    }
    (void)rows;
    (void)cols;
    return 0;
}

int ufp4_rht(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int axis, int rht_kind,
             uint64_t rht_seed, void *y, int y_dtype, int64_t ldy, void *stream)
{
    if (axis != UFP4_ROW && axis != UFP4_COL) return UFP4_ERR_INVALID_ARG;
    if (rht_kind < UFP4_RHT_NONE || rht_kind > UFP4_RHT_DETERMINISTIC) return UFP4_ERR_INVALID_ARG;
    if (y_dtype != UFP4_BF16 && y_dtype != UFP4_F32) return UFP4_ERR_INVALID_ARG;
    int rc = check_source(x, x_dtype, rows, cols, ldx, axis, 16);
    if (rc) return rc;
    const int64_t V = axis == UFP4_ROW ? rows : cols, L = axis == UFP4_ROW ? cols : rows;
    if (!y && V * L > 0) return UFP4_ERR_INVALID_ARG;
    if (ldy < L) return UFP4_ERR_SHAPE;
    if (!aligned16(y) || ldy % 8) return UFP4_ERR_ALIGN;
    RowArgs ra;
    ColArgs ca;
    fill_args(x, x_dtype, rows, cols, ldx, axis, sign_mask(rht_kind, rht_seed), ra, ca);
    ra.y = y;
    ra.ldy = ldy;
    ca.y = y;
    ca.ldy = ldy;
    LaunchSpec sp{0, 0, 0, x_dtype, rht_kind != UFP4_RHT_NONE, axis};
    return hip_fail(launch_rht(sp, y_dtype, ra, ca, (hipStream_t)stream));
}

// The amax pass once its arguments and its partial-maxima buffer (ws, ws
// checked by the caller) are settled.
static int amax_run(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, const ufp4_config *cfg,
                    float *amax, float *ws, void *stream)
{
    RowArgs ra;
    ColArgs ca;
    fill_args(x, x_dtype, rows, cols, ldx, cfg->axis, sign_mask(cfg->rht, cfg->rht_seed), ra, ca);
    ra.partials = ws;
    ca.partials = ws;
    LaunchSpec sp{0, 0, 0, x_dtype, cfg->rht != UFP4_RHT_NONE, cfg->axis};
    return hip_fail(launch_amax(sp, ra, ca, amax, (hipStream_t)stream));
}

static int amax_check(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, const ufp4_config *cfg,
                      const float *amax)
{
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!amax) return UFP4_ERR_INVALID_ARG;
    return check_source(x, x_dtype, rows, cols, ldx, cfg->axis, 16);
}

int ufp4_amax(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, const ufp4_config *cfg,
              float *amax, void *ws, size_t ws_bytes, void *stream)
{
    int rc = amax_check(x, x_dtype, rows, cols, ldx, cfg, amax);
    if (rc) return rc;
    const size_t need = ufp4_workspace_size(UFP4_OP_AMAX, rows, cols, cfg);
    if (!ws || ws_bytes < need) return UFP4_ERR_WORKSPACE;
    if ((uintptr_t)ws & 3u) return UFP4_ERR_ALIGN;
    return amax_run(x, x_dtype, rows, cols, ldx, cfg, amax, static_cast<float *>(ws), stream);
}

int ufp4_amax_noalloc(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, const ufp4_config *cfg,
                      float *amax, void *stream)
{
    int rc = amax_check(x, x_dtype, rows, cols, ldx, cfg, amax);
    if (rc) return rc;
    if (ufp4_workspace_size(UFP4_OP_AMAX, rows, cols, cfg) > sizeof(float) * AMAX_SCRATCH_FLOATS)
        return UFP4_ERR_WORKSPACE;
    float *scratch = nullptr;
    rc = amax_scratch_of_current_device(&scratch);
    if (rc) return rc;
    return amax_run(x, x_dtype, rows, cols, ldx, cfg, amax, scratch, stream);
}

int ufp4_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, const ufp4_config *cfg,
                  const float *amax, ufp4_qtensor *out, void *stream)
{
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!out) return UFP4_ERR_INVALID_ARG;
    rc = check_source(x, x_dtype, rows, cols, ldx, cfg->axis, cfg->block);
    if (rc) return rc;
    if (rows * cols > 0 && (!out->codes || !out->scales)) return UFP4_ERR_INVALID_ARG;
    if (cfg->scale == UFP4_SCALE_E4M3 && (!amax || !out->tensor_scale)) return UFP4_ERR_INVALID_ARG;
    if (((uintptr_t)out->codes & 7u) || ((uintptr_t)out->scales & 3u)) return UFP4_ERR_ALIGN;
    out->rows = rows;
    out->cols = cols;
    out->cfg = *cfg;
    RowArgs ra;
    ColArgs ca;
    fill_args(x, x_dtype, rows, cols, ldx, cfg->axis, sign_mask(cfg->rht, cfg->rht_seed), ra, ca);
    ra.codes = out->codes;
    ra.scales = out->scales;
    ra.amax = amax;
    ra.tensor_scale = out->tensor_scale;
    ra.sr_seed = cfg->sr_seed;
    ra.sr_stream = cfg->sr_stream;
    ca.codes = out->codes;
    ca.scales = out->scales;
    ca.amax = amax;
    ca.tensor_scale = out->tensor_scale;
    ca.sr_seed = cfg->sr_seed;
    ca.sr_stream = cfg->sr_stream;
    LaunchSpec sp{cfg->format, cfg->scale, cfg->rounding == UFP4_SR, x_dtype, cfg->rht != UFP4_RHT_NONE, cfg->axis};
    return hip_fail(launch_quantize(sp, ra, ca, (hipStream_t)stream));
}

static int check_qtensor(const ufp4_qtensor *q)
{
    if (!q) return UFP4_ERR_INVALID_ARG;
    int rc = check_config(&q->cfg);
    if (rc) return rc;
    if (q->rows < 0 || q->cols < 0) return UFP4_ERR_SHAPE;
    const int64_t L = q->cfg.axis == UFP4_ROW ? q->cols : q->rows;
    if (L % q->cfg.block) return UFP4_ERR_SHAPE;
    if (q->rows * q->cols > 0 && (!q->codes || !q->scales)) return UFP4_ERR_INVALID_ARG;
    if (q->cfg.scale == UFP4_SCALE_E4M3 && !q->tensor_scale) return UFP4_ERR_INVALID_ARG;
    if (((uintptr_t)q->codes & 3u) || ((uintptr_t)q->scales & 3u)) return UFP4_ERR_ALIGN;
    return UFP4_OK;
}

int ufp4_dequantize(const ufp4_qtensor *q, int inverse_rht, void *y, int y_dtype, int64_t ldy, void *stream)
{
    int rc = check_qtensor(q);
    if (rc) return rc;
    if (y_dtype != UFP4_BF16 && y_dtype != UFP4_F32) return UFP4_ERR_INVALID_ARG;
    const int64_t V = q->cfg.axis == UFP4_ROW ? q->rows : q->cols, L = q->cfg.axis == UFP4_ROW ? q->cols : q->rows;
    if (!y && V * L > 0) return UFP4_ERR_INVALID_ARG;
    if (ldy < L) return UFP4_ERR_SHAPE;
    if (!aligned16(y) || ldy % 8) return UFP4_ERR_ALIGN;
    DeqArgs a;
    a.codes = q->codes;
    a.scales = q->scales;
    a.tensor_scale = q->tensor_scale;
    a.L = L;
    a.n_oct = V * L / 8;
    a.smask = sign_mask(q->cfg.rht, q->cfg.rht_seed);
    a.y = y;
    a.ldy = ldy;
    const int inv = inverse_rht && q->cfg.rht != UFP4_RHT_NONE;
    return hip_fail(launch_dequant(q->cfg.format, q->cfg.scale, inv, y_dtype, a, (hipStream_t)stream));
}

int ufp4_stats(const void *x, int x_dtype, int64_t ldx, const ufp4_qtensor *q, double *sums, void *ws,
               size_t ws_bytes, void *stream)
{
    int rc = check_qtensor(q);
    if (rc) return rc;
    if (!sums) return UFP4_ERR_INVALID_ARG;
    rc = check_source(x, x_dtype, q->rows, q->cols, ldx, q->cfg.axis, q->cfg.block);
    if (rc) return rc;
    const size_t need = ufp4_workspace_size(UFP4_OP_STATS, q->rows, q->cols, &q->cfg);
    if (!ws || ws_bytes < need) return UFP4_ERR_WORKSPACE;
    if ((uintptr_t)ws & 7u || (uintptr_t)sums & 7u) return UFP4_ERR_ALIGN;
    StatsArgs a = {};
    a.x = x;
    a.ldx = ldx;
    a.V = q->cfg.axis == UFP4_ROW ? q->rows : q->cols;
    a.L = q->cfg.axis == UFP4_ROW ? q->cols : q->rows;
    a.axis = q->cfg.axis;
    a.smask = sign_mask(q->cfg.rht, q->cfg.rht_seed);
    a.codes = q->codes;
    a.scales = q->scales;
    a.tensor_scale = q->tensor_scale;
    a.partials = static_cast<double *>(ws);
    a.sums = sums;
    return hip_fail(launch_stats(q->cfg.format, q->cfg.scale, x_dtype, q->cfg.rht != UFP4_RHT_NONE, a,
                                 (hipStream_t)stream));
}

void ufp4_stats_finalize(const double *s, ufp4_stats_report *r)
{
    memset(r, 0, sizeof(*r));
    const double n = s[0];
    r->n = n;
    r->sqnr_db = s[2] > 0 ? 10.0 * log10(s[1] / s[2]) : INFINITY;
    r->alpha = s[1] > 0 ? s[5] / s[1] : NAN;
    r->mse = n > 0 ? s[2] / n : 0.0;
    r->mean_err = n > 0 ? s[3] / n : 0.0;
    r->mean_shrink = n > 0 ? s[4] / n : 0.0;
    r->int4_share = s[7] > 0 ? s[8] / s[7] : 0.0;
    for (int t = 0; t < 2; ++t)
        for (int k = 0; k < 8; ++k) {
            const double c = s[16 + 8 * t + k];
            r->counts[t][k] = c;
            r->bucket_bias[t][k] = c > 0 ? s[32 + 8 * t + k] / c : NAN;
        }
}

int ufp4_gemm_bf16(const void *a, const void *b, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, float *c,
                   int64_t ldc, void *stream)
{
    if ((!a || !b || !c) && M * N * K > 0) return UFP4_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return UFP4_ERR_SHAPE;
    if (M % 256 || N % 256 || K % 64) return UFP4_ERR_SHAPE;
    if (lda < K || ldb < K || ldc < N) return UFP4_ERR_SHAPE;
    if (!gemm_offsets_fit(2 * lda, 2 * K) || !gemm_offsets_fit(2 * ldb, 2 * K)) return UFP4_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(b) || !aligned16(c) || lda % 8 || ldb % 8 || ldc % 4) return UFP4_ERR_ALIGN;
    if (M == 0 || N == 0) return UFP4_OK;
    return hip_fail(launch_gemm_bf16(static_cast<const uint16_t *>(a), static_cast<const uint16_t *>(b), M, N, K, lda,
                                     ldb, c, ldc, (hipStream_t)stream));
}

int ufp4_qgemm(const ufp4_qtensor *a, const ufp4_qtensor *b, int mode, float *c, int64_t ldc, void *ws,
               size_t ws_bytes, void *stream)
{
    int rc = check_qtensor(a);
    if (rc) return rc;
    rc = check_qtensor(b);
    if (rc) return rc;
    if (!c) return UFP4_ERR_INVALID_ARG;
    // the GEMM runs on the views: a row quantization's view is the matrix, a
    // column quantization's its transpose (both stored K-major)
    const int64_t M = a->cfg.axis == UFP4_ROW ? a->rows : a->cols;
    const int64_t N = b->cfg.axis == UFP4_ROW ? b->rows : b->cols;
    const int64_t K = a->cfg.axis == UFP4_ROW ? a->cols : a->rows;
    if ((b->cfg.axis == UFP4_ROW ? b->cols : b->rows) != K) return UFP4_ERR_SHAPE;
    if (a->cfg.rht != b->cfg.rht || (a->cfg.rht == UFP4_RHT_RANDOM && a->cfg.rht_seed != b->cfg.rht_seed))
        return UFP4_ERR_UNSUPPORTED;
    if (M % 256 || N % 256 || K % 128) return UFP4_ERR_SHAPE;
    if (ldc < N || ldc % 4) return UFP4_ERR_SHAPE;
    // native mode: code rows of K/2 bytes; dequantize mode: bf16 rows of 2K
    if (!gemm_offsets_fit(mode == UFP4_GEMM_NATIVE_MXFP4 ? K / 2 : 2 * K, mode == UFP4_GEMM_NATIVE_MXFP4 ? K / 2 : 2 * K))
        return UFP4_ERR_SHAPE;
    if (!aligned16(c)) return UFP4_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    if (mode == UFP4_GEMM_NATIVE_MXFP4) {
        if (a->cfg.format != UFP4_E2M1 || a->cfg.scale != UFP4_SCALE_E8M0 || b->cfg.format != UFP4_E2M1 ||
            b->cfg.scale != UFP4_SCALE_E8M0)
            return UFP4_ERR_UNSUPPORTED;
        if (!aligned16(a->codes) || !aligned16(b->codes)) return UFP4_ERR_ALIGN;
        if (M == 0 || N == 0) return UFP4_OK;
        return hip_fail(launch_gemm_mxfp4(a->codes, static_cast<const uint8_t *>(a->scales), b->codes,
                                          static_cast<const uint8_t *>(b->scales), M, N, K, c, ldc, st));
    }
    if (mode != UFP4_GEMM_DEQUANT_BF16) return UFP4_ERR_INVALID_ARG;
    const size_t need = (size_t)((M + N) * K * 2);
    if (!ws || ws_bytes < need) return UFP4_ERR_WORKSPACE;
    if (!aligned16(ws)) return UFP4_ERR_ALIGN;
    if (M == 0 || N == 0) return UFP4_OK;
    uint16_t *da = static_cast<uint16_t *>(ws);
    uint16_t *db = da + M * K;
    // x_hat of each operand in bf16 (nearest even), in the rotated domain
    rc = ufp4_dequantize(a, 0, da, UFP4_BF16, K, stream);
    if (rc) return rc;
    rc = ufp4_dequantize(b, 0, db, UFP4_BF16, K, stream);
    if (rc) return rc;
    return hip_fail(launch_gemm_bf16(da, db, M, N, K, K, K, c, ldc, st));
}

int ufp4_eta(const float *zq, const float *z, int64_t M, int64_t N, int64_t ld, double *sums, void *ws, size_t ws_bytes,
             void *stream)
{
    if (!zq || !z || !sums) return UFP4_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || ld < N) return UFP4_ERR_SHAPE;
    if (N % 4 || ld % 4) return UFP4_ERR_SHAPE;
    if (!aligned16(zq) || !aligned16(z) || (uintptr_t)sums & 7u) return UFP4_ERR_ALIGN;
    const size_t need = ufp4_workspace_size(UFP4_OP_ETA, M, N, nullptr);
    if (!ws || ws_bytes < need) return UFP4_ERR_WORKSPACE;
    return hip_fail(launch_eta(zq, z, M, N, ld, static_cast<double *>(ws), sums, (hipStream_t)stream));
}

// ---- FP4 KV cache ------------------------------------------------------

static constexpr int64_t KV_PAGE_TOKENS = 128;
static constexpr int64_t KV_WAVES_PER_WG = 8;  // a decode wave prefetches one page past its last

// Bytes of a 128-token page: FP4 or the FP8 baseline (0 for an unknown format).
static int64_t kv_page_bytes(int kv_format)
{
    return kv_format == UFP4_KV_FP4 ? 17408 : kv_format == UFP4_KV_FP8 ? 33792 : 0;
}

// Pages per split of a decode: requested, or about 256 workgroups in all
// (one 8-wave workgroup per compute unit, all resident at once) with at least
// one page per wave.  With B * Hkv >= 256 every sequence is one split and no
// combine pass runs.
static int64_t kv_pages_per_split(int64_t B, int64_t Hkv, int64_t npages, int64_t req)
{
    if (req > 0) return req < npages ? req : npages;
    const int64_t total = B * Hkv * npages;
    int64_t pps = (total + 255) / 256;
    pps = (pps + 7) / 8 * 8;
    if (pps < 8) pps = 8;
    return pps;
}

static int kv_check_heads(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L_cap)
{
    if (B < 0 || Hkv < 1 || Hq < 1 || L_cap < 1) return UFP4_ERR_SHAPE;
    if (D != 128) return UFP4_ERR_UNSUPPORTED;
    if (Hq % Hkv) return UFP4_ERR_SHAPE;
    if (Hq / Hkv > 16) return UFP4_ERR_UNSUPPORTED;
    if (L_cap % KV_PAGE_TOKENS) return UFP4_ERR_SHAPE;
    // one sequence's pages (of either format) are addressed with 32-bit
    // buffer offsets
    if ((L_cap / KV_PAGE_TOKENS + KV_WAVES_PER_WG) * kv_page_bytes(UFP4_KV_FP8) > INT32_MAX) return UFP4_ERR_SHAPE;
    return UFP4_OK;
}

size_t ufp4_kv_cache_bytes(int64_t B, int64_t Hkv, int64_t L_cap, int64_t D, int kv_format)
{
    if (kv_check_heads(B, Hkv, Hkv, D, L_cap) || !kv_page_bytes(kv_format)) return 0;
    return (size_t)(B * Hkv * (L_cap / KV_PAGE_TOKENS) * kv_page_bytes(kv_format));
}

int ufp4_kv_cache_quantize(const void *k, const void *v, int64_t B, int64_t Hkv, int64_t L_cap, int64_t D,
                           int kv_format, int64_t stride_b, int64_t stride_h, int64_t stride_t, const int32_t *lens,
                           int rotate_k, uint8_t *cache, void *stream)
{
    int rc = kv_check_heads(B, Hkv, Hkv, D, L_cap);
    if (rc) return rc;
    if ((rotate_k != 0 && rotate_k != 1) || !kv_page_bytes(kv_format)) return UFP4_ERR_INVALID_ARG;
    if (B == 0) return UFP4_OK;
    if (!k || !v || !lens || !cache) return UFP4_ERR_INVALID_ARG;
    if (stride_t < D || stride_b < 0 || stride_h < 0 || B > 65535 || Hkv > 65535) return UFP4_ERR_SHAPE;
    if (!aligned16(k) || !aligned16(v) || !aligned16(cache) || stride_b % 8 || stride_h % 8 || stride_t % 8)
        return UFP4_ERR_ALIGN;
    return hip_fail(launch_kv_quantize(static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), B, Hkv, L_cap,
                                       kv_format == UFP4_KV_FP8, stride_b, stride_h, stride_t, lens, rotate_k, cache,
                                       (hipStream_t)stream));
}

int ufp4_kv_q_quantize(const void *q, int64_t rows, int64_t D, int rotate, uint8_t *codes, uint8_t *scales,
                       void *stream)
{
    if (rows < 0) return UFP4_ERR_SHAPE;
    if (D != 128) return UFP4_ERR_UNSUPPORTED;
    if (rotate != 0 && rotate != 1) return UFP4_ERR_INVALID_ARG;
    if (rows == 0) return UFP4_OK;
    if (!q || !codes || !scales) return UFP4_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(codes)) return UFP4_ERR_ALIGN;
    return hip_fail(launch_q_quantize(static_cast<const uint16_t *>(q), rows, rotate, codes, scales,
                                      (hipStream_t)stream));
}

size_t ufp4_kv_decode_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L_cap,
                                     int64_t pages_per_split)
{
    if (kv_check_heads(B, Hq, Hkv, D, L_cap)) return 0;
    const int64_t npages = L_cap / KV_PAGE_TOKENS;
    const int64_t pps = kv_pages_per_split(B, Hkv, npages, pages_per_split);
    const int64_t nsplit = (npages + pps - 1) / pps;
    if (nsplit <= 1) return 0;
    return (size_t)(B * Hq * nsplit * (D + 2) * (int64_t)sizeof(float));
}

int ufp4_kv_decode(const void *q, const uint8_t *cache, const int32_t *lens, int64_t B, int64_t Hq, int64_t Hkv,
                   int64_t D, int kv_format, int64_t L_cap, float sm_scale, int rotate, int64_t pages_per_split,
                   float *out, void *ws, size_t ws_bytes, void *stream)
{
    int rc = kv_check_heads(B, Hq, Hkv, D, L_cap);
    if (rc) return rc;
    if ((rotate != 0 && rotate != 1) || !kv_page_bytes(kv_format)) return UFP4_ERR_INVALID_ARG;
    if (!(fabsf(sm_scale) <= 3.0e38f) || pages_per_split < 0) return UFP4_ERR_INVALID_ARG;
    if (B == 0) return UFP4_OK;
    if (!q || !cache || !lens || !out) return UFP4_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(cache) || !aligned16(out)) return UFP4_ERR_ALIGN;
    const int64_t npages = L_cap / KV_PAGE_TOKENS;
    const int64_t pps = kv_pages_per_split(B, Hkv, npages, pages_per_split);
    const int64_t nsplit = (npages + pps - 1) / pps;
    if (nsplit > 65535 || B > 65535 || Hkv > 65535) return UFP4_ERR_SHAPE;
    float *ws_o = nullptr, *ws_ml = nullptr;
    if (nsplit > 1) {
        const size_t need = ufp4_kv_decode_workspace_size(B, Hq, Hkv, D, L_cap, pages_per_split);
        if (!ws || ws_bytes < need) return UFP4_ERR_WORKSPACE;
        if (!aligned16(ws)) return UFP4_ERR_ALIGN;
        ws_o = static_cast<float *>(ws);
        ws_ml = ws_o + B * Hq * nsplit * D;
    }
    // log2(e) folded into the score scale, rounded once to binary32
    const float c = (float)((double)sm_scale * 1.4426950408889634074);
    return hip_fail(launch_kv_decode(static_cast<const uint16_t *>(q), cache, lens, B, Hkv, (int)(Hq / Hkv),
                                     kv_format == UFP4_KV_FP8, L_cap, c, rotate, (int)pps, (int)nsplit, out, ws_o,
                                     ws_ml, (hipStream_t)stream));
}

}  // extern "C"
