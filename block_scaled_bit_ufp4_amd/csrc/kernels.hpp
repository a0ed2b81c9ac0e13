// kernels.hpp -- argument blocks and launchers shared by the host code and
// the kernel files of libufp4 (internal; the public interface is ufp4.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ufp4 {

// A pending request of ufp4_time_next_launch on this thread (both null when
// none); the next launch_kernel takes and clears it.
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTiming &launch_timing();

// Every library kernel starts here: a plain launch, or one that timestamps
// its own dispatch on the requested events.
template <typename... Params, typename... Args>
inline void launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t st, Args... args)
{
    LaunchTiming &t = launch_timing();
    if (t.start) {
        const LaunchTiming req = t;
        t = LaunchTiming{};
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, req.start, req.stop, 0, static_cast<Params>(args)...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, 0, st, static_cast<Params>(args)...);
    }
}

// Compute units of the current device, read once per device and kept (256,
// the MI355X's count, if the query fails).
int cu_count();

// Row kernel: one lane per 16-element chunk of a view row.
struct RowArgs {
    const void *x;        // source (ROW axis: the view itself)
    int64_t ldx;          // source row stride (elements)
    int64_t L;            // view row length
    int64_t n_ch;         // V * L / 16
    int contiguous;       // ldx == L
    uint32_t smask;       // RHT sign mask (bit i: d_i = -1)
    uint8_t *codes;       // [V][L/2]
    void *scales;         // [V][L/B]
    const float *amax;    // tensor amax (E4M3)
    float *tensor_scale;  // alpha out (E4M3)
    uint64_t sr_seed;
    uint32_t sr_stream;
    void *y;              // RHT output
    int64_t ldy;
    float *partials;      // amax: one partial maximum per workgroup
};

// Column kernel: the view is the transpose of x[R][C].
struct ColArgs {
    const void *x;
    int64_t ldx;
    int64_t R, C;
    uint32_t smask;
    uint8_t *codes;       // [C][R/2]
    void *scales;         // [C][R/B]
    const float *amax;
    float *tensor_scale;
    uint64_t sr_seed;
    uint32_t sr_stream;
    void *y;              // [C][ldy]
    int64_t ldy;
    float *partials;      // amax: one partial maximum per workgroup
};

struct LaunchSpec {
    int format;    // FMT_*
    int scale;     // SC_*
    int sr;        // stochastic rounding
    int in_dtype;  // IN_BF16 / IN_F32
    int rht;       // apply signs + FWHT
    int axis;      // 0 row, 1 column
};

hipError_t launch_quantize(const LaunchSpec &sp, const RowArgs &ra, const ColArgs &ca, hipStream_t st);
hipError_t launch_amax(const LaunchSpec &sp, const RowArgs &ra, const ColArgs &ca, float *amax, hipStream_t st);
int64_t amax_tiles(int axis, int64_t rows, int64_t cols);  // partial maxima the amax pass writes
hipError_t launch_rht(const LaunchSpec &sp, int out_dtype, const RowArgs &ra, const ColArgs &ca, hipStream_t st);

// Dequantization of a view (row-major codes), optional inverse transform.
struct DeqArgs {
    const uint8_t *codes;
    const void *scales;
    const float *tensor_scale;
    int64_t L;
    int64_t n_oct;
    uint32_t smask;
    void *y;
    int64_t ldy;
};
hipError_t launch_dequant(int format, int scale, int inverse_rht, int out_dtype, const DeqArgs &a, hipStream_t st);

// Statistics of a quantized view against its source.
struct StatsArgs {
    const void *x;
    int64_t ldx;
    int64_t V, L;
    int axis;
    uint32_t smask;
    const uint8_t *codes;
    const void *scales;
    const float *tensor_scale;
    double *partials;  // [grid][48]
    double *sums;      // [48]
    int64_t t0, t1;    // blocks [t0, t1) of the view (set per launch)
    int accumulate;    // add to the partial sums instead of storing them
};
constexpr int STATS_WGS = 2048;
hipError_t launch_stats(int format, int scale, int in_dtype, int rht, const StatsArgs &a, hipStream_t st);

constexpr int ETA_WGS = 1024;
hipError_t launch_eta(const float *zq, const float *z, int64_t M, int64_t N, int64_t ld, double *partials,
                      double *sums, hipStream_t st);

// GEMMs: C[M][ldc] = A B^T.
hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *b, int64_t M, int64_t N, int64_t K, int64_t lda,
                            int64_t ldb, float *c, int64_t ldc, hipStream_t st);
// FP4 KV cache (or the FP8 baseline, fp8 = 1) and decode attention (head dim 128).
hipError_t launch_kv_quantize(const uint16_t *k, const uint16_t *v, int64_t B, int64_t Hkv, int64_t L_cap, int fp8,
                              int64_t sb, int64_t sh, int64_t st, const int32_t *lens, int rotate, uint8_t *cache,
                              hipStream_t s);
hipError_t launch_q_quantize(const uint16_t *q, int64_t rows, int rotate, uint8_t *codes, uint8_t *scales,
                             hipStream_t s);
hipError_t launch_kv_decode(const uint16_t *q, const uint8_t *cache, const int32_t *lens, int64_t B, int64_t Hkv, int G,
                            int fp8, int64_t L_cap, float c, int rotate, int pps, int nsplit, float *out, float *ws_o,
                            float *ws_ml, hipStream_t s);

hipError_t launch_gemm_mxfp4(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb, int64_t M,
                             int64_t N, int64_t K, float *c, int64_t ldc, hipStream_t st);

}  // namespace ufp4
