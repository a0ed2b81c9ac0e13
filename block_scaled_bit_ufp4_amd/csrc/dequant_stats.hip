// dequant_stats.hip -- dequantization, quantization statistics and the
// attenuation reductions.
//
// Dequantization is code x scale, with IF4's INT4 blocks scaled by 6/7 (IF4
// page, 3.1.1).  The statistics are those the pages use to compare formats:
// SQNR and the signal factor alpha of A_hat = alpha A + R ("当你的 GPU 学不会
// 算账" sections "治病药反而喂养了病菌" and "复利效应的反向版本"), per-cell
// rounding bias (section "E2M1：一块刻度不均的尺子"; "蚂蚁集团揭秘" 二) and IF4's
// type shares (IF4 page 6.2).  The attenuation eta = <Zq,Z>/<Z,Z> is the
// identity of section "复利效应的反向版本".
#include "device.hpp"
#include "kernels.hpp"

namespace ufp4 {

constexpr int DT = 256;
constexpr int DU = 4;

// ---------------------------------------------------------------------------
// Dequantization: one lane per 8 consecutive view elements, like the row
// quantizer; the inverse transform's span-8 butterfly crosses lanes by DPP.
// ---------------------------------------------------------------------------
template <int F, int S, bool INV, int OUT>
__global__ __launch_bounds__(DT) void dequant_kernel(const DeqArgs a)
{
    const int tid = threadIdx.x;
    const uint32_t half = tid & 1;
    const uint32_t neg_own = half << 31;
    uint32_t sgn[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sgn[i] = ((a.smask >> (8 * half + i)) & 1u) << 31;
    float alpha = 0.0f;
    if constexpr (S == SC_E4M3) alpha = *a.tensor_scale;
    const int64_t base = (int64_t)blockIdx.x * (DT * DU) + tid;
#pragma unroll
    for (int u = 0; u < DU; ++u) {
        const int64_t o = base + u * DT;
        if (o >= a.n_oct) break;
        const uint32_t packed = reinterpret_cast<const uint32_t *>(a.codes)[o];
        float s;
        bool int4 = false;
        if constexpr (S == SC_FP32) {
            s = static_cast<const float *>(a.scales)[o >> 1];
        } else if constexpr (S == SC_E8M0) {
            s = __builtin_amdgcn_ldexpf(1.0f, (int)static_cast<const uint8_t *>(a.scales)[o >> 2] - 127);
        } else {
            const uint32_t b = static_cast<const uint8_t *>(a.scales)[o >> 1];
            s = alpha * e4m3_decode(b & 0x7Fu);
            int4 = (F == FMT_IF4) && (b & 0x80u);
        }
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t c = (packed >> (4 * i)) & 15u;
            const uint32_t k = c & 7u;
            float x;
            if (F == FMT_IF4 && int4) {
                x = ((float)k * s) * (6.0f / 7.0f);
            } else {
                x = grid_value<F == FMT_IF4 ? FMT_E2M1 : F>(k) * s;
            }
            v[i] = (c & 8u) ? -x : x;
        }
        if constexpr (INV) {
            fwht8(v);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p = xor1(v[i]);
                v[i] = u2f(f2u(v[i]) ^ neg_own) + p;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = u2f(f2u(v[i] * 0.25f) ^ sgn[i]);
        }
        int64_t off;
        if (a.ldy == a.L) {
            off = o * 8;
        } else {
            const int64_t L8 = a.L >> 3, vr = o / L8;
            off = vr * a.ldy + (o - vr * L8) * 8;
        }
        if constexpr (OUT == IN_F32) {
            // A whole wave of consecutive octets in a contiguous output goes
            // through LDS, so each of its two stores writes 1 KiB contiguously
            // (per lane they would be 16-byte pieces 32 bytes apart).  The
            // wave's LDS write and read execute in order: no barrier.
            __shared__ float4 stage[DT / 64][128];
            const int w = tid >> 6, l = tid & 63;
            const int64_t o0 = o - l;  // the octet of lane 0
            if (a.ldy == a.L && o0 + 63 < a.n_oct) {
                stage[w][2 * l] = make_float4(v[0], v[1], v[2], v[3]);
                stage[w][2 * l + 1] = make_float4(v[4], v[5], v[6], v[7]);
                const float4 q0 = stage[w][l], q1 = stage[w][64 + l];
                typedef float f32x4 __attribute__((ext_vector_type(4)));
                f32x4 *p = reinterpret_cast<f32x4 *>(static_cast<float *>(a.y) + o0 * 8);
                const f32x4 r0 = {q0.x, q0.y, q0.z, q0.w}, r1 = {q1.x, q1.y, q1.z, q1.w};
                __builtin_nontemporal_store(r0, p + l);
                __builtin_nontemporal_store(r1, p + 64 + l);
            } else {
                float4 *p = reinterpret_cast<float4 *>(static_cast<float *>(a.y) + off);
                p[0] = make_float4(v[0], v[1], v[2], v[3]);
                p[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        } else {
            uint4 w;
            w.x = to_bf16(v[0]) | (to_bf16(v[1]) << 16);
            w.y = to_bf16(v[2]) | (to_bf16(v[3]) << 16);
            w.z = to_bf16(v[4]) | (to_bf16(v[5]) << 16);
            w.w = to_bf16(v[6]) | (to_bf16(v[7]) << 16);
            *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.y) + off) = w;
        }
    }
}

template <int F, int S>
static hipError_t deq_pick(int inverse_rht, int out_dtype, const DeqArgs &a, hipStream_t st)
{
    if (a.n_oct == 0) return hipSuccess;
    const dim3 grid((unsigned)((a.n_oct + DT * DU - 1) / (DT * DU)));
    if (inverse_rht) {
        if (out_dtype == IN_F32)
            launch_kernel((dequant_kernel<F, S, true, IN_F32>), grid, dim3(DT), st, a);
        else
            launch_kernel((dequant_kernel<F, S, true, IN_BF16>), grid, dim3(DT), st, a);
    } else {
        if (out_dtype == IN_F32)
            launch_kernel((dequant_kernel<F, S, false, IN_F32>), grid, dim3(DT), st, a);
        else
            launch_kernel((dequant_kernel<F, S, false, IN_BF16>), grid, dim3(DT), st, a);
    }
    return hipGetLastError();
}

hipError_t launch_dequant(int format, int scale, int inverse_rht, int out_dtype, const DeqArgs &a, hipStream_t st)
{
    if (format == FMT_IF4) return deq_pick<FMT_IF4, SC_E4M3>(inverse_rht, out_dtype, a, st);
    if (scale == SC_E8M0) return deq_pick<FMT_E2M1, SC_E8M0>(inverse_rht, out_dtype, a, st);
#define UFP4_DQ(FF)                                                                                      \
    if (format == FF)                                                                                    \
        return scale == SC_FP32 ? deq_pick<FF, SC_FP32>(inverse_rht, out_dtype, a, st)                   \
                                : deq_pick<FF, SC_E4M3>(inverse_rht, out_dtype, a, st);
    UFP4_DQ(FMT_E2M1)
    UFP4_DQ(FMT_E1M2)
    UFP4_DQ(FMT_INT4)
    UFP4_DQ(FMT_E2M1_M4)
    UFP4_DQ(FMT_E2M1_M3)
    UFP4_DQ(FMT_E2M1_M2)
#undef UFP4_DQ
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Reductions of binary64 partial sums
// ---------------------------------------------------------------------------
template <int NV>
__device__ __forceinline__ void block_reduce_store(double (&acc)[NV], double *out)
{
    __shared__ double red[4][NV];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        double v = acc[k];
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) red[wave][k] = v;
    }
    __syncthreads();
    if (threadIdx.x < NV) {
        const int k = threadIdx.x;
        out[k] = ((red[0][k] + red[1][k]) + red[2][k]) + red[3][k];
    }
}

// One workgroup adds nwg rows of NV partial sums in a fixed order: wave w
// takes sums w, w + 4, ...; for each, lane l adds rows l, l + 64, ... and the
// wave adds its lanes by shuffles.  No barriers.
template <int NV>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const double *partials, int nwg, double *sums)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int k = wave; k < NV; k += 4) {
        double v = 0.0;
        for (int i = lane; i < nwg; i += 64) v += partials[(int64_t)i * NV + k];
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) sums[k] = v;
    }
}

// ---------------------------------------------------------------------------
// Statistics: one thread per block of the view.  Row axis: consecutive lanes
// take consecutive blocks of a view row, and a block's elements are one
// vector load; column axis: consecutive lanes take consecutive view rows (=
// source columns), so the loads x[l][v] coalesce.  The per-code counts and
// rounding-bias sums (32 of the 48) live in LDS bins private to each thread:
// an element adds to its own code's bin with one LDS atomic, in element order,
// so every bin is the same binary64 sum as a register accumulator would hold.
// ---------------------------------------------------------------------------
constexpr int NS = 48;
constexpr int STATS_T = 256;

template <int F, int S, int IN, bool RHT>
__global__ __launch_bounds__(STATS_T) void stats_kernel(const StatsArgs a)
{
    constexpr int B = block_of(S);
    constexpr int FG = F == FMT_IF4 ? FMT_E2M1 : F;
    __shared__ double bias_bin[16][STATS_T];   // code k (FP4) or 8 + k (INT4 blocks of IF4)
    __shared__ uint32_t count_bin[16][STATS_T];
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        bias_bin[q][tid] = 0.0;
        count_bin[q][tid] = 0u;
    }
    double acc[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) acc[k] = 0.0;
    float alpha = 0.0f;
    if constexpr (S == SC_E4M3) alpha = *a.tensor_scale;
    const int64_t nb_row = a.L / B;
    const int64_t nblocks = a.V * nb_row;
    for (int64_t t = (int64_t)blockIdx.x * STATS_T + tid; t < nblocks; t += (int64_t)gridDim.x * STATS_T) {
        int64_t v, j;
        if (a.axis == 0) {
            v = t / nb_row;
            j = t - v * nb_row;
        } else {
            j = t / a.V;
            v = t - j * a.V;
        }
        float y[B];
        if (a.axis == 0) {
            // the block is contiguous and 16-byte aligned (x aligned, ldx a multiple of 8)
            const int64_t idx = v * a.ldx + j * B;
            if constexpr (IN == IN_BF16) {
                const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + idx);
#pragma unroll
                for (int c = 0; c < B / 8; ++c) {
                    const uint4 w = p[c];
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        y[8 * c + 2 * h] = u2f(ws[h] << 16);
                        y[8 * c + 2 * h + 1] = u2f(ws[h] & 0xFFFF0000u);
                    }
                }
            } else {
                const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + idx);
#pragma unroll
                for (int c = 0; c < B / 4; ++c) {
                    const float4 w = p[c];
                    y[4 * c] = w.x;
                    y[4 * c + 1] = w.y;
                    y[4 * c + 2] = w.z;
                    y[4 * c + 3] = w.w;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const int64_t idx = (j * B + i) * a.ldx + v;
                if constexpr (IN == IN_BF16)
                    y[i] = u2f((uint32_t)static_cast<const uint16_t *>(a.x)[idx] << 16);
                else
                    y[i] = static_cast<const float *>(a.x)[idx];
            }
        }
        if constexpr (RHT) {
#pragma unroll
            for (int c = 0; c < B; c += 16) {
#pragma unroll
                for (int i = 0; i < 16; ++i) y[c + i] = u2f(f2u(y[c + i]) ^ (((a.smask >> i) & 1u) << 31));
                fwht16_local(y + c);
            }
        }
        // stored scale
        const int64_t sidx = v * nb_row + j;
        float s;
        bool int4 = false;
        if constexpr (S == SC_FP32) {
            s = static_cast<const float *>(a.scales)[sidx];
        } else if constexpr (S == SC_E8M0) {
            s = __builtin_amdgcn_ldexpf(1.0f, (int)static_cast<const uint8_t *>(a.scales)[sidx] - 127);
        } else {
            const uint32_t b = static_cast<const uint8_t *>(a.scales)[sidx];
            s = alpha * e4m3_decode(b & 0x7Fu);
            int4 = (F == FMT_IF4) && (b & 0x80u);
        }
        const float inv = s == 0.0f ? 0.0f : 1.0f / s;
        const bool fast = fast_div_ok(s);
        // the block's B / 2 code bytes as 32-bit words (codes are 4-byte aligned)
        uint32_t cw[B / 8];
        const uint32_t *cp = reinterpret_cast<const uint32_t *>(a.codes + (v * a.L + j * B) / 2);
#pragma unroll
        for (int i = 0; i < B / 8; ++i) cw[i] = cp[i];
        acc[7] += 1.0;
        acc[8] += int4 ? 1.0 : 0.0;
        const int bin0 = int4 ? 8 : 0;
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const uint32_t c = (cw[i >> 3] >> (4 * (i & 7))) & 15u;
            const uint32_t k = c & 7u;
            float xm, g, ta;
            if (int4) {
                xm = ((float)k * s) * (6.0f / 7.0f);
                g = (float)k;
                ta = fabsf(y[i]) * (7.0f / 6.0f);
            } else {
                xm = grid_value<FG>(k) * s;
                g = grid_value<FG>(k);
                ta = fabsf(y[i]);
            }
            float z;
            if (s == 0.0f)
                z = 0.0f;
            else if (S == SC_E8M0)
                z = ta * inv;
            else
                z = fast ? div_fast(ta, s, inv) : ta / s;
            if (s != 0.0f && z == 0.0f && ta > 0.0f) z = ta / s;
            const double xh = (c & 8u) ? -(double)xm : (double)xm;
            const double yy = (double)y[i];
            const double e = xh - yy;
            acc[0] += 1.0;
            acc[1] += yy * yy;
            acc[2] += e * e;
            acc[3] += e;
            acc[4] += (yy > 0.0 ? e : (yy < 0.0 ? -e : 0.0));
            acc[5] += xh * yy;
            acc[6] += fabs(e);
            atomicAdd(&bias_bin[bin0 + k][tid], (double)g - (double)z);
            atomicAdd(&count_bin[bin0 + k][tid], 1u);
        }
    }
    double out[NS];
#pragma unroll
    for (int k = 0; k < 9; ++k) out[k] = acc[k];
#pragma unroll
    for (int k = 9; k < 16; ++k) out[k] = 0.0;
    // each thread reads back only its own bins (its own LDS atomics are done
    // in order before these reads)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        out[16 + q] = (double)count_bin[q][tid];
        out[24 + q] = (double)count_bin[8 + q][tid];
        out[32 + q] = bias_bin[q][tid];
        out[40 + q] = bias_bin[8 + q][tid];
    }
    block_reduce_store<NS>(out, a.partials + (int64_t)blockIdx.x * NS);
}

template <int F, int S>
static hipError_t stats_pick(int in_dtype, int rht, const StatsArgs &a, hipStream_t st)
{
    const int64_t nblocks = a.V * (a.L / block_of(S));
    int64_t g = (nblocks + STATS_T - 1) / STATS_T;
    // the 48 KiB of LDS bins fit three workgroups on a CU: one full wave of
    // them over the 256 CUs, no tail (the workspace holds STATS_WGS rows)
    constexpr int64_t kResident = 3 * 256;
    static_assert(kResident <= STATS_WGS, "stats grid");
    if (g > kResident) g = kResident;
    if (g < 1) g = 1;
    const dim3 grid((unsigned)g);
    if (in_dtype == IN_BF16) {
        if (rht)
            launch_kernel((stats_kernel<F, S, IN_BF16, true>), grid, dim3(STATS_T), st, a);
        else
            launch_kernel((stats_kernel<F, S, IN_BF16, false>), grid, dim3(STATS_T), st, a);
    } else {
        if (rht)
            launch_kernel((stats_kernel<F, S, IN_F32, true>), grid, dim3(STATS_T), st, a);
        else
            launch_kernel((stats_kernel<F, S, IN_F32, false>), grid, dim3(STATS_T), st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_kernel(reduce_partials_kernel<NS>, dim3(1), dim3(256), st, a.partials, (int)g, a.sums);
    return hipGetLastError();
}

hipError_t launch_stats(int format, int scale, int in_dtype, int rht, const StatsArgs &a, hipStream_t st)
{
    if (format == FMT_IF4) return stats_pick<FMT_IF4, SC_E4M3>(in_dtype, rht, a, st);
    if (scale == SC_E8M0) return stats_pick<FMT_E2M1, SC_E8M0>(in_dtype, rht, a, st);
#define UFP4_ST(FF)                                                                                       \
    if (format == FF)                                                                                     \
        return scale == SC_FP32 ? stats_pick<FF, SC_FP32>(in_dtype, rht, a, st)                           \
                                : stats_pick<FF, SC_E4M3>(in_dtype, rht, a, st);
    UFP4_ST(FMT_E2M1)
    UFP4_ST(FMT_E1M2)
    UFP4_ST(FMT_INT4)
    UFP4_ST(FMT_E2M1_M4)
    UFP4_ST(FMT_E2M1_M3)
    UFP4_ST(FMT_E2M1_M2)
#undef UFP4_ST
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Attenuation sums <Zq,Z>, <Z,Z>, ||Zq - Z||^2 in binary64.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void eta_kernel(const float *zq, const float *z, int64_t M, int64_t N, int64_t ld,
                                                  double *partials)
{
    double acc[3] = {0.0, 0.0, 0.0};
    const int64_t n4 = N / 4;
    const int64_t total = M * n4;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        const int64_t r = t / n4, c = (t - r * n4) * 4;
        const float4 a = *reinterpret_cast<const float4 *>(zq + r * ld + c);
        const float4 b = *reinterpret_cast<const float4 *>(z + r * ld + c);
        const double qa[4] = {a.x, a.y, a.z, a.w}, zb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[0] += qa[i] * zb[i];
            acc[1] += zb[i] * zb[i];
            const double d = qa[i] - zb[i];
            acc[2] += d * d;
        }
    }
    block_reduce_store<3>(acc, partials + (int64_t)blockIdx.x * 3);
}

hipError_t launch_eta(const float *zq, const float *z, int64_t M, int64_t N, int64_t ld, double *partials,
                      double *sums, hipStream_t st)
{
    launch_kernel(eta_kernel, dim3(ETA_WGS), dim3(256), st, zq, z, M, N, ld, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_kernel(reduce_partials_kernel<3>, dim3(1), dim3(256), st, partials, ETA_WGS, sums);
    return hipGetLastError();
}

}  // namespace ufp4
