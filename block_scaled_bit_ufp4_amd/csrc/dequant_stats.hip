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
#include <type_traits>

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
template <int NV, typename Slot>
__device__ __forceinline__ void block_reduce_store(double (&acc)[NV], double *out, Slot slot, bool add = false)
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
        const double v = ((red[0][k] + red[1][k]) + red[2][k]) + red[3][k];
        out[slot(k)] = add ? out[slot(k)] + v : v;
    }
}

// One workgroup per sum k (grid NV) adds column k of nwg rows of NV partial
// sums: thread t loads rows t, t + RED_T, ... (all its loads issued at once,
// nwg <= RED_T RED_ROWS), adds them in row order, and the workgroup adds its
// threads in a fixed tree (lane butterfly, then the waves in order).  The
// order is fixed, so the result is the same on every run; with one round of
// loads per thread the reduction is one memory latency long.
constexpr int RED_T = 256;
constexpr int RED_ROWS = 8;
static_assert(STATS_WGS <= RED_T * RED_ROWS && ETA_WGS <= RED_T * RED_ROWS, "one round of loads");
template <int NV>
__global__ __launch_bounds__(RED_T) void reduce_partials_kernel(const double *partials, int nwg, double *sums)
{
    const int k = blockIdx.x, t = threadIdx.x;
    double v[RED_ROWS];
#pragma unroll
    for (int u = 0; u < RED_ROWS; ++u) {
        const int row = t + u * RED_T;
        v[u] = row < nwg ? partials[(int64_t)row * NV + k] : 0.0;
    }
    double acc = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    __shared__ double red[RED_T / 64];
    if ((t & 63) == 0) red[t >> 6] = acc;
    __syncthreads();
    if (t == 0) sums[k] = ((red[0] + red[1]) + red[2]) + red[3];
}

// ---------------------------------------------------------------------------
// Statistics: one thread per block of the view.  Row axis: consecutive lanes
// take consecutive blocks of a view row, and a block's elements are one
// vector load; column axis: consecutive lanes take consecutive view rows (=
// source columns), so the loads x[l][v] coalesce.  Loads run up to three
// blocks ahead of the block being processed.
//
// Sums 1..6 are binary64 registers.  Each block's terms are first summed in
// binary32 (the element's products and the error e = x_hat - y are binary32
// operations), then scaled and added in binary64.  A wave whose blocks all
// have scales in [2^-30, 2^30] sums the values as they are; otherwise every
// block is first scaled by a power of two P near 1 / s (exact), so that
// squares of values up to the binary32 maximum neither overflow nor lose
// precision, and the sums are scaled back exactly.
//
// Per-code counts and rounding-bias sums: one 64-bit LDS word per thread and
// code (no two lanes share a word, so the LDS adds never conflict), which
// adds 2^48 + floor(z 2^26) per element, z = |y| / s in grid units.  A launch
// adds at most STATS_CHUNK elements per thread, so the count (bits 48..63)
// and the fixed-point sum of z (below 2^47 while z < 64; the quantizer's z
// stay below 1.5 x the grid maximum) never meet, and the bias sum of code k
// is count x g[k] - sum z.  Truncation moves a bias sum by less than 2^-26
// per element.  Each thread reads back only its own words.
//
// Every sum is added in a fixed order, so the results are the same on every
// run; they differ from the oracle's element-order binary64 sums only by
// rounding: about 1e-7 relative for the whole-tensor sums, and for a bucket's
// bias sum about one unit in the last place of z per element (z = |y| / s
// with the refined reciprocal), far below 1e-6 of its count.
// ---------------------------------------------------------------------------
constexpr int NS = 48;
constexpr int STATS_T = 256;
constexpr int64_t STATS_CHUNK = 1 << 15;  // elements per thread and launch
// Blocks whose loads are in flight per thread: three for 16-element blocks
// (two for IF4, whose 16 bins and two candidates take more registers), one
// for 32-element blocks (a second set would cost a resident wave).
constexpr int STATS_DEPTH(int B, bool IF4) { return B == 16 ? (IF4 ? 2 : 3) : 1; }

template <int B, int IN>
struct StatsRaw;
template <int B>
struct StatsRaw<B, IN_BF16> {
    uint4 w[B / 8];
};
template <int B>
struct StatsRaw<B, IN_F32> {
    float4 w[B / 4];
};

// Signed values of the 8 codes of w on a uniform grid (sign << 3 | k per
// nibble): each nibble becomes the FP8 E4M3 byte sign << 7 | k, the subnormal
// k 2^-9, which the FP8 decode scaled by 2^9 x step turns into k x step
// (exact).
template <int F>
__device__ __forceinline__ void decode8_uniform(uint32_t w, float *g)
{
    constexpr float SC = F == FMT_E1M2 ? 256.0f : 512.0f;
    const uint32_t even = (w & 0x07070707u) | ((w << 4) & 0x80808080u);  // nibbles 0, 2, 4, 6
    const uint32_t odd = ((w >> 4) & 0x07070707u) | (w & 0x80808080u);   // nibbles 1, 3, 5, 7
    const v2f e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(even, SC, false);
    const v2f e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(even, SC, true);
    const v2f o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(odd, SC, false);
    const v2f o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(odd, SC, true);
    g[0] = e0.x;
    g[2] = e0.y;
    g[4] = e1.x;
    g[6] = e1.y;
    g[1] = o0.x;
    g[3] = o0.y;
    g[5] = o1.x;
    g[7] = o1.y;
}

// Grid value g[q] of bin q (IF4: bins 8..15 are the INT4 blocks' codes).
template <int F>
__device__ __forceinline__ double bin_grid(int q)
{
    if constexpr (F == FMT_IF4) return q < 8 ? (double)grid_value<FMT_E2M1>(q) : (double)(q - 8);
    return (double)grid_value<F>(q);
}

template <int F, int S, int IN, bool RHT>
__global__ __launch_bounds__(STATS_T) __attribute__((amdgpu_waves_per_eu(block_of(S) == 16 ? 3 : 2))) void stats_kernel(const StatsArgs a)
{
    constexpr int B = block_of(S);
    constexpr bool IF4 = F == FMT_IF4;
    constexpr int FG = IF4 ? FMT_E2M1 : F;
    constexpr int NBIN = IF4 ? 16 : 8;  // code k, or 8 + k in IF4's INT4 blocks
    constexpr bool FOLD = RHT && IN == IN_BF16;
    __shared__ uint64_t bins[NBIN][STATS_T];
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < NBIN; ++q) bins[q][tid] = 0u;
    double acc[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) acc[k] = 0.0;
    uint32_t nblk = 0, nint4 = 0;
    float alpha = 0.0f;
    if constexpr (S == SC_E4M3) alpha = *a.tensor_scale;
    uint32_t sgn[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sgn[i] = RHT ? ((a.smask >> i) & 1u) << 31 : 0u;
    const int64_t nb_row = a.L / B;
    const int64_t step = (int64_t)gridDim.x * STATS_T;

    // One block: its values (the source's, signs applied), code words and
    // stored scale.
    auto block = [&](float (&y)[B], const uint32_t (&c_cur)[B / 8], uint32_t s_cur) {
        // the transform; for bf16 sources its final x 1/4 is folded into the
        // scale (y = v / 4 exactly, every partial sum being a multiple of
        // 2^-133), so the sums below are of 4 y, 4 x_hat and 4 e
        if constexpr (RHT) {
#pragma unroll
            for (int c = 0; c < B; c += 16) {
                fwht8(y + c);
                fwht8(y + c + 8);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p = y[c + i], q = y[c + i + 8];
                    y[c + i] = p + q;
                    y[c + i + 8] = p - q;
                }
                if constexpr (!FOLD) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) y[c + i] = y[c + i] * 0.25f;
                }
            }
        }
        // the stored scale
        float s;
        bool int4 = false;
        if constexpr (S == SC_FP32) {
            s = u2f(s_cur);
        } else if constexpr (S == SC_E8M0) {
            s = __builtin_amdgcn_ldexpf(1.0f, (int)s_cur - 127);
        } else {
            s = alpha * e4m3_decode_hw(s_cur & 0x7Fu);
            int4 = IF4 && (s_cur & 0x80u);
        }
        const float sk = FOLD ? s * 4.0f : s;  // exact
        // signed grid values of the codes
        float gv[B];
        if constexpr (e2m1_codes(FG)) {
#pragma unroll
            for (int i = 0; i < B; i += 2) {
                const v2f d = decode2_e2m1(c_cur[i >> 3], (i & 7) >> 1);
                gv[i] = d.x;
                gv[i + 1] = d.y;
            }
            if constexpr (IF4) {
                float gi[B];
#pragma unroll
                for (int w = 0; w < B / 8; ++w) decode8_uniform<FMT_INT4>(c_cur[w], gi + 8 * w);
#pragma unroll
                for (int i = 0; i < B; ++i) gv[i] = int4 ? gi[i] : gv[i];
            }
        } else {
#pragma unroll
            for (int w = 0; w < B / 8; ++w) decode8_uniform<FG>(c_cur[w], gv + 8 * w);
        }
        // x_hat = g s (IF4's INT4 blocks: (g s) 6/7); z = |y| / s (INT4
        // blocks: |y| 7/6 / s) in units of 2^-26, as one product with the
        // refined reciprocal
        const float post = int4 ? 6.0f / 7.0f : 1.0f;
        const float pre = int4 ? 7.0f / 6.0f * 0x1p26f : 0x1p26f;
        const int bin0 = int4 ? 8 : 0;
        // With s = 0 (an all-zero block, or an E4M3 block scale that rounded
        // to zero) the block's scale of reference is the tensor scale alpha,
        // above every such block's values; an FP32 scale is 0 only for a
        // block below 2^-147, whose values the largest scaling (2^126) keeps
        // exact and normal.
        const float pref = s != 0.0f ? s : (S == SC_E4M3 ? alpha : 0x1p-149f);
        const bool far = !(pref >= 0x1p-30f && pref <= 0x1p30f);
        auto terms = [&](auto scaled) {
            constexpr bool SCALED = decltype(scaled)::value;
            int pe = 0;
            float P = 1.0f;
            if constexpr (SCALED) {
                pe = pref != 0.0f ? __builtin_amdgcn_frexp_expf(pref) : 0;
                pe = pe > 126 ? 126 : (pe < -126 ? -126 : pe);
                P = __builtin_amdgcn_ldexpf(1.0f, -pe);
            }
            const float skp = SCALED ? sk * P : sk;  // exact
            const float zinv = s == 0.0f ? 0.0f : pre * rcp_rn(skp);
            float p1 = 0.f, p2 = 0.f, p3 = 0.f, p4 = 0.f, p5 = 0.f, p6 = 0.f;
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const float v = SCALED ? y[i] * P : y[i];
                // P x_hat (x 4 when folded).  Scaled blocks take x_hat as the
                // dequantizer rounds it, g s (then x 6/7 in IF4's INT4 blocks),
                // before the exact scalings by P and by 4 (one at a time: P
                // reaches 2^126): for blocks whose x_hat is subnormal that
                // rounding is coarser than a product taken after scaling.
                const float xk = SCALED ? ((IF4 ? (gv[i] * s) * post : gv[i] * s) * P) * (FOLD ? 4.0f : 1.0f)
                                        : (IF4 ? (gv[i] * skp) * post : gv[i] * skp);
                const float ek = xk - v;
                p1 = __builtin_fmaf(v, v, p1);
                p2 = __builtin_fmaf(ek, ek, p2);
                p3 += ek;
                p4 += u2f(f2u(ek) ^ (f2u(v) & 0x80000000u));  // sign(y) e (y = +-0 gives e = +-0)
                p5 = __builtin_fmaf(xk, v, p5);
                p6 += fabsf(ek);
                const uint32_t k = (c_cur[i >> 3] >> (4 * (i & 7))) & 7u;
                const uint32_t zf = (uint32_t)(fabsf(v) * zinv);
                atomicAdd(&bins[bin0 + (int)k][tid], (1ull << 48) | zf);
            }
            constexpr double F2 = FOLD ? 1.0 / 16.0 : 1.0, F1 = FOLD ? 0.25 : 1.0;  // exact
            double G2 = F2, G1 = F1;
            if constexpr (SCALED) {
                G2 = __builtin_amdgcn_ldexp(F2, 2 * pe);
                G1 = __builtin_amdgcn_ldexp(F1, pe);
            }
            acc[0] = __builtin_fma((double)p1, G2, acc[0]);
            acc[1] = __builtin_fma((double)p2, G2, acc[1]);
            acc[2] = __builtin_fma((double)p3, G1, acc[2]);
            acc[3] = __builtin_fma((double)p4, G1, acc[3]);
            acc[4] = __builtin_fma((double)p5, G2, acc[4]);
            acc[5] = __builtin_fma((double)p6, G1, acc[5]);
        };
        if (__builtin_amdgcn_ballot_w64(far) == 0)
            terms(std::false_type{});
        else
            terms(std::true_type{});
        ++nblk;
        if constexpr (IF4) nint4 += int4 ? 1u : 0u;
    };

    // Block t is block j of view row v: t = v nb_row + j (row axis) or
    // t = j V + v (column axis).  Loads run STATS_DEPTH blocks ahead of the
    // block being processed, in register sets used in turn; their position
    // advances by a fixed step, so it is kept as a (major, minor) pair and
    // stepped without divisions.
    const int64_t minor_n = a.axis == 0 ? nb_row : a.V;
    const int64_t d_major = step / minor_n, d_minor = step - d_major * minor_n;
    const int64_t first = a.t0 + (int64_t)blockIdx.x * STATS_T + tid;
    int64_t lt = first, major = first / minor_n, minor = first - major * minor_n;
    auto advance = [&] {
        lt += step;
        minor += d_minor;
        major += d_major;
        if (minor >= minor_n) {
            minor -= minor_n;
            ++major;
        }
    };
    // the block's B / 2 code bytes and its scale
    auto load_codes = [&](int64_t coff, int64_t sidx, uint32_t (&cw)[B / 8], uint32_t &sraw) {
        if constexpr (B == 16) {
            const uint2 c2 = *reinterpret_cast<const uint2 *>(a.codes + coff);
            cw[0] = c2.x;
            cw[1] = c2.y;
        } else {
            const uint4 c4 = *reinterpret_cast<const uint4 *>(a.codes + coff);
            cw[0] = c4.x;
            cw[1] = c4.y;
            cw[2] = c4.z;
            cw[3] = c4.w;
        }
        if constexpr (S == SC_FP32)
            sraw = __float_as_uint(static_cast<const float *>(a.scales)[sidx]);
        else
            sraw = static_cast<const uint8_t *>(a.scales)[sidx];
    };
    // Every load is issued unconditionally: the position stops at the
    // thread's last block, which the loads past the range read again (from
    // the cache, just after its first read), so no branch surrounds a load
    // and the waits stay as deep as the prefetch.
    auto run = [&](auto (&sets)[STATS_DEPTH(B, IF4)], auto load, auto unpack) {
        auto issue = [&](auto &d) {
            load(d);
            if (lt + step < a.t1) advance();
        };
#pragma unroll
        for (int k = 0; k < STATS_DEPTH(B, IF4); ++k) issue(sets[k]);
        for (int64_t t = first; t < a.t1;) {
#pragma unroll
            for (int k = 0; k < STATS_DEPTH(B, IF4); ++k) {
                float y[B];
                unpack(sets[k], y);
                // The set's registers are consumed before its next load is
                // issued: the unpacked values are pinned in registers (so no
                // use of them sinks into the branch below) and the code words
                // and scale copied to fresh ones.  The load then reuses the
                // set's registers, and the loop carries no copy of a register
                // with a load in flight (which would wait for that load).
#pragma unroll
                for (int i = 0; i < B; ++i) asm volatile("" : "+v"(y[i]));
                uint32_t c[B / 8], sc;
#pragma unroll
                for (int i = 0; i < B / 8; ++i) asm volatile("v_mov_b32 %0, %1" : "=v"(c[i]) : "v"(sets[k].cw[i]));
                asm volatile("v_mov_b32 %0, %1" : "=v"(sc) : "v"(sets[k].s));
                issue(sets[k]);
                if (t < a.t1) block(y, c, sc);
                t += step;
            }
        }
    };
    if (first >= a.t1) {
        // no block for this thread
    } else if (a.axis == 0) {
        // row axis: block t = (v, j) holds B consecutive elements of view
        // row v, one vector load; its codes sit at t B / 2, its scale at t
        struct Set {
            StatsRaw<B, IN> raw;
            uint32_t cw[B / 8];
            uint32_t s;
        } sets[STATS_DEPTH(B, IF4)];
        auto load = [&](Set &d) {
            const int64_t idx = major * a.ldx + minor * B;
            if constexpr (IN == IN_BF16) {
                const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + idx);
#pragma unroll
                for (int c = 0; c < B / 8; ++c) d.raw.w[c] = p[c];
            } else {
                const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + idx);
#pragma unroll
                for (int c = 0; c < B / 4; ++c) d.raw.w[c] = p[c];
            }
            load_codes(lt * (B / 2), lt, d.cw, d.s);
        };
        auto unpack = [&](const Set &d, float (&y)[B]) {
            if constexpr (IN == IN_BF16) {
#pragma unroll
                for (int c = 0; c < B / 8; ++c) {
                    const uint32_t ws[4] = {d.raw.w[c].x, d.raw.w[c].y, d.raw.w[c].z, d.raw.w[c].w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const int i = 8 * c + 2 * h;
                        y[i] = u2f((ws[h] << 16) ^ sgn[i & 15]);
                        y[i + 1] = u2f((ws[h] & 0xFFFF0000u) ^ sgn[(i + 1) & 15]);
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < B / 4; ++c) {
                    const float4 w = d.raw.w[c];
                    y[4 * c] = u2f(f2u(w.x) ^ sgn[(4 * c) & 15]);
                    y[4 * c + 1] = u2f(f2u(w.y) ^ sgn[(4 * c + 1) & 15]);
                    y[4 * c + 2] = u2f(f2u(w.z) ^ sgn[(4 * c + 2) & 15]);
                    y[4 * c + 3] = u2f(f2u(w.w) ^ sgn[(4 * c + 3) & 15]);
                }
            }
        };
        run(sets, load, unpack);
    } else {
        // column axis: block t = (v, j) holds source elements x[j B + i][v];
        // consecutive lanes take consecutive v, so each of the B loads
        // coalesces.  The loaded values are kept as they arrive and unpacked
        // when the block is processed.
        struct Set {
            uint32_t h[B];
            uint32_t cw[B / 8];
            uint32_t s;
        } sets[STATS_DEPTH(B, IF4)];
        auto load = [&](Set &d) {
            const int64_t v = minor, j = major;
            if constexpr (IN == IN_BF16) {
                const uint16_t *p = static_cast<const uint16_t *>(a.x) + (j * B) * a.ldx + v;
#pragma unroll
                for (int i = 0; i < B; ++i) d.h[i] = p[i * a.ldx];
            } else {
                const uint32_t *p = static_cast<const uint32_t *>(a.x) + (j * B) * a.ldx + v;
#pragma unroll
                for (int i = 0; i < B; ++i) d.h[i] = p[i * a.ldx];
            }
            load_codes((v * a.L + j * B) / 2, v * nb_row + j, d.cw, d.s);
        };
        auto unpack = [&](const Set &d, float (&y)[B]) {
#pragma unroll
            for (int i = 0; i < B; ++i) y[i] = u2f((IN == IN_BF16 ? d.h[i] << 16 : d.h[i]) ^ sgn[i & 15]);
        };
        run(sets, load, unpack);
    }

    // The sums a format can make nonzero, reduced over the workgroup and
    // stored (or, after the first launch, added) at their places in the
    // 48-sum layout: 0..8, then the counts and bias sums of the NBIN bins
    // (the others are zero).  Each thread reads back only its own bins.
    constexpr int NV = 9 + 2 * NBIN;
    double out[NV];
    out[0] = (double)nblk * B;
#pragma unroll
    for (int k = 0; k < 6; ++k) out[1 + k] = acc[k];
    out[7] = (double)nblk;
    out[8] = (double)nint4;
#pragma unroll
    for (int q = 0; q < NBIN; ++q) {
        const uint64_t u = bins[q][tid];
        const double n = (double)(uint32_t)(u >> 48);
        out[9 + q] = n;
        out[9 + NBIN + q] = n * bin_grid<F>(q) - (double)(u & 0xFFFFFFFFFFFFull) * 0x1p-26;
    }
    double *dst = a.partials + (int64_t)blockIdx.x * NS;
    block_reduce_store<NV>(
        out, dst, [](int k) { return k < 9 ? k : (k < 9 + NBIN ? 16 + (k - 9) : 32 + (k - 9 - NBIN)); },
        a.accumulate != 0);
    // the sums no bin of this format touches: 9..15, and with 8 bins the
    // INT4-block counts 24..31 and bias sums 40..47
    if (tid < NS - NV) dst[tid < 7 ? 9 + tid : (tid < 15 ? 24 + (tid - 7) : 40 + (tid - 15))] = 0.0;
}

// Workgroups of the statistics grid: as many per compute unit of the current
// device as are resident at once, at most one per STATS_T blocks, at most
// STATS_WGS (the workspace rows).
template <typename K>
static int stats_grid(K kernel, int64_t nblocks)
{
    static const int per_cu = [kernel] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, STATS_T, 0) != hipSuccess || n < 1) n = 1;
        return n;
    }();
    int64_t g = (nblocks + STATS_T - 1) / STATS_T;
    const int64_t resident = (int64_t)cu_count() * per_cu;
    if (g > resident) g = resident;
    if (g > STATS_WGS) g = STATS_WGS;
    return g < 1 ? 1 : (int)g;
}

// One or more launches over consecutive ranges of blocks (each thread takes
// at most STATS_CHUNK elements per launch), the later ones adding to the
// partial sums, then the reduction.
template <typename K>
static hipError_t stats_run(K kernel, int B, StatsArgs a, hipStream_t st)
{
    const int64_t nblocks = a.V * (a.L / B);
    const int g = stats_grid(kernel, nblocks);
    const int64_t per_launch = (int64_t)g * STATS_T * (STATS_CHUNK / B);
    int64_t t0 = 0;
    do {
        a.t0 = t0;
        a.t1 = nblocks - t0 > per_launch ? t0 + per_launch : nblocks;
        a.accumulate = t0 > 0;
        launch_kernel(kernel, dim3((unsigned)g), dim3(STATS_T), st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        t0 = a.t1;
    } while (t0 < nblocks);
    launch_kernel(reduce_partials_kernel<NS>, dim3(NS), dim3(RED_T), st, a.partials, g, a.sums);
    return hipGetLastError();
}

template <int F, int S>
static hipError_t stats_pick(int in_dtype, int rht, const StatsArgs &a, hipStream_t st)
{
    constexpr int B = block_of(S);
    if (in_dtype == IN_BF16)
        return rht ? stats_run(stats_kernel<F, S, IN_BF16, true>, B, a, st)
                   : stats_run(stats_kernel<F, S, IN_BF16, false>, B, a, st);
    return rht ? stats_run(stats_kernel<F, S, IN_F32, true>, B, a, st)
               : stats_run(stats_kernel<F, S, IN_F32, false>, B, a, st);
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
    block_reduce_store<3>(acc, partials + (int64_t)blockIdx.x * 3, [](int k) { return k; });
}

hipError_t launch_eta(const float *zq, const float *z, int64_t M, int64_t N, int64_t ld, double *partials,
                      double *sums, hipStream_t st)
{
    launch_kernel(eta_kernel, dim3(ETA_WGS), dim3(256), st, zq, z, M, N, ld, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_kernel(reduce_partials_kernel<3>, dim3(3), dim3(RED_T), st, partials, ETA_WGS, sums);
    return hipGetLastError();
}

}  // namespace ufp4
