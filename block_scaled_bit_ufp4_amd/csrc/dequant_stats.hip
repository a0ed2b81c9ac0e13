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
// source columns), so the loads x[l][v] coalesce.  The next block's loads are
// issued before the current block is processed.
//
// The tensor-wide sums are binary64 registers; each block's terms are first
// summed in binary32 over its two halves (the element's products and the
// error e = x_hat - y are binary32 operations), then scaled and added in
// binary64.  The per-code counts and rounding-bias sums live in LDS bins
// private to each thread (no two lanes share a bin, so the LDS adds never
// conflict): counts as 32-bit integers, bias sums in binary64 (the LDS adds
// 32-bit integers and binary64 at full rate; its binary32 add is much
// slower).  Every sum is added in a fixed order, so the results are the same
// on every run; they differ from the oracle's element-order binary64 sums
// only by rounding: about 1e-7 relative for the whole-tensor sums, and for a
// bucket's bias sum at most 1.5 units in the last place of z per element
// (z = |y| / s from the rounded reciprocal), far below 1e-6 of its count.
// ---------------------------------------------------------------------------
constexpr int NS = 48;
constexpr int STATS_T = 256;
constexpr int stats_wg_per_cu(int B) { return B == 32 ? 3 : 4; }  // all resident: 16-blocks 4 waves/SIMD, 32-blocks 3

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

template <int F, int S, int IN, bool RHT>
__global__ __launch_bounds__(STATS_T) void stats_kernel(const StatsArgs a)
{
    constexpr int B = block_of(S);
    constexpr bool IF4 = F == FMT_IF4;
    constexpr int FG = IF4 ? FMT_E2M1 : F;
    constexpr int NBIN = IF4 ? 16 : 8;  // code k, or 8 + k in IF4's INT4 blocks
    constexpr bool FOLD = RHT && IN == IN_BF16;
    __shared__ double bias_bin[NBIN][STATS_T];
    __shared__ uint32_t count_bin[NBIN][STATS_T];
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < NBIN; ++q) {
        bias_bin[q][tid] = 0.0;
        count_bin[q][tid] = 0u;
    }
    double acc[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) acc[k] = 0.0;
    float alpha = 0.0f;
    if constexpr (S == SC_E4M3) alpha = *a.tensor_scale;
    uint32_t sgn[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sgn[i] = RHT ? ((a.smask >> i) & 1u) << 31 : 0u;
    const int64_t nb_row = a.L / B;
    const int64_t nblocks = a.V * nb_row;
    const int64_t step = (int64_t)gridDim.x * STATS_T;

    // Block t is block j of view row v: t = v nb_row + j (row axis) or
    // t = j V + v (column axis).  The position advances by a fixed step per
    // iteration, so it is kept as a (major, minor) pair and stepped without
    // divisions.
    const int64_t minor_n = a.axis == 0 ? nb_row : a.V;
    const int64_t d_major = step / minor_n, d_minor = step - d_major * minor_n;
    auto load = [&](int64_t major, int64_t minor, StatsRaw<B, IN> &r, uint32_t (&cw)[B / 8], uint32_t &sraw) {
        const int64_t v = a.axis == 0 ? major : minor, j = a.axis == 0 ? minor : major;
        if (a.axis == 0) {
            const int64_t idx = v * a.ldx + j * B;
            if constexpr (IN == IN_BF16) {
                const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + idx);
#pragma unroll
                for (int c = 0; c < B / 8; ++c) r.w[c] = p[c];
            } else {
                const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + idx);
#pragma unroll
                for (int c = 0; c < B / 4; ++c) r.w[c] = p[c];
            }
        } else {
            if constexpr (IN == IN_BF16) {
                const uint16_t *p = static_cast<const uint16_t *>(a.x) + (j * B) * a.ldx + v;
                uint32_t h[B];
#pragma unroll
                for (int i = 0; i < B; ++i) h[i] = p[i * a.ldx];
#pragma unroll
                for (int c = 0; c < B / 8; ++c)
                    r.w[c] = make_uint4(h[8 * c] | (h[8 * c + 1] << 16), h[8 * c + 2] | (h[8 * c + 3] << 16),
                                        h[8 * c + 4] | (h[8 * c + 5] << 16), h[8 * c + 6] | (h[8 * c + 7] << 16));
            } else {
                const float *p = static_cast<const float *>(a.x) + (j * B) * a.ldx + v;
#pragma unroll
                for (int c = 0; c < B / 4; ++c)
                    r.w[c] = make_float4(p[(4 * c) * a.ldx], p[(4 * c + 1) * a.ldx], p[(4 * c + 2) * a.ldx],
                                         p[(4 * c + 3) * a.ldx]);
            }
        }
        // the block's B / 2 code bytes as 32-bit words (codes are 4-byte aligned)
        const uint32_t *cp = reinterpret_cast<const uint32_t *>(a.codes + (v * a.L + j * B) / 2);
#pragma unroll
        for (int i = 0; i < B / 8; ++i) cw[i] = cp[i];
        const int64_t sidx = v * nb_row + j;
        if constexpr (S == SC_FP32)
            sraw = __float_as_uint(static_cast<const float *>(a.scales)[sidx]);
        else
            sraw = static_cast<const uint8_t *>(a.scales)[sidx];
    };

    int64_t t = (int64_t)blockIdx.x * STATS_T + tid;
    int64_t major = t / minor_n, minor = t - major * minor_n;
    StatsRaw<B, IN> raw;
    uint32_t cw[B / 8], sraw = 0;
    if (t < nblocks) load(major, minor, raw, cw, sraw);
    while (t < nblocks) {
        // unpack and transform the current block, then start the next one's loads
        float y[B];
        if constexpr (IN == IN_BF16) {
#pragma unroll
            for (int c = 0; c < B / 8; ++c) {
                const uint32_t ws[4] = {raw.w[c].x, raw.w[c].y, raw.w[c].z, raw.w[c].w};
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
                const float4 w = raw.w[c];
                y[4 * c] = u2f(f2u(w.x) ^ sgn[(4 * c) & 15]);
                y[4 * c + 1] = u2f(f2u(w.y) ^ sgn[(4 * c + 1) & 15]);
                y[4 * c + 2] = u2f(f2u(w.z) ^ sgn[(4 * c + 2) & 15]);
                y[4 * c + 3] = u2f(f2u(w.w) ^ sgn[(4 * c + 3) & 15]);
            }
        }
        uint32_t c_cur[B / 8];
#pragma unroll
        for (int i = 0; i < B / 8; ++i) c_cur[i] = cw[i];
        const uint32_t s_cur = sraw;
        const int64_t tn = t + step;
        minor += d_minor;
        major += d_major;
        if (minor >= minor_n) {
            minor -= minor_n;
            ++major;
        }
        if (tn < nblocks) load(major, minor, raw, cw, sraw);
        // the transform; for bf16 sources its final x 1/4 is folded into the
        // scale (y = v / 4 exactly, every partial sum being a multiple of
        // 2^-133), so the loop below works on v = 4y, 4 x_hat and 4e
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
        // z = |y| / s (IF4's INT4 blocks: |y| 7/6 / s) as one product with
        // the rounded reciprocal: within 1.5 units in the last place of the
        // correctly rounded quotient, far inside the bias sums' tolerance.
        // Scales outside [2^-75, 2^125] (where the reciprocal would leave the
        // normal range) take the true quotient.
        const float pre = int4 ? 7.0f / 6.0f : 1.0f;
        const float zinv = s == 0.0f ? 0.0f : pre / sk;
        float z[B];
#pragma unroll
        for (int i = 0; i < B; ++i) z[i] = fabsf(y[i]) * zinv;
        if constexpr (S != SC_E8M0) {
            const bool slow = s != 0.0f && !fast_div_ok(s);
            if (__builtin_amdgcn_ballot_w64(slow) != 0) {
                if (slow) {
#pragma unroll
                    for (int i = 0; i < B; ++i) z[i] = (fabsf(y[i]) * pre) / sk;
                }
            }
        }
        const float post = int4 ? 6.0f / 7.0f : 1.0f;
        const int bin0 = int4 ? 8 : 0;
        // The block's terms are summed in binary32 after scaling the block by
        // a power of two P near 1 / s (exact), so that squares of values up to
        // the binary32 maximum neither overflow nor lose precision; the sums
        // are scaled back exactly in binary64.  With s = 0 (an all-zero block,
        // or an E4M3 block scale that rounded to zero) P comes from the tensor
        // scale alpha, above every such block's values.
        const float pref = s != 0.0f ? s : (S == SC_E4M3 ? alpha : 1.0f);
        int pe = pref != 0.0f ? __builtin_amdgcn_frexp_expf(pref) : 0;
        pe = pe > 126 ? 126 : (pe < -126 ? -126 : pe);
        const float P = __builtin_amdgcn_ldexpf(1.0f, -pe);
        const float skp = sk * P;  // exact
        const double Pinv = __builtin_amdgcn_ldexp(1.0, pe), Pinv2 = Pinv * Pinv;
        // grid values of the codes: E2M1 codes by the hardware FP4 decode
        // (two per instruction, signed, exact), the uniform grids as k x step
        float gv[B];
        if constexpr (e2m1_codes(FG)) {
#pragma unroll
            for (int i = 0; i < B; i += 2) {
                const v2f d = decode2_e2m1(c_cur[i >> 3], (i & 7) >> 1);
                gv[i] = d.x;
                gv[i + 1] = d.y;
            }
        }
        // binary32 sums over the block's two halves, then binary64
        float p1[2] = {0.f, 0.f}, p2[2] = {0.f, 0.f}, p3[2] = {0.f, 0.f}, p4[2] = {0.f, 0.f}, p5[2] = {0.f, 0.f},
              p6[2] = {0.f, 0.f};
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int h = (2 * i) / B;
            const uint32_t sh = 4 * (i & 7);
            const uint32_t k = (c_cur[i >> 3] >> sh) & 7u;
            float gs;  // signed grid value
            if constexpr (e2m1_codes(FG)) {
                gs = gv[i];
                if constexpr (IF4) {
                    const float gi = u2f(f2u((float)k) | ((c_cur[i >> 3] << (28 - sh)) & 0x80000000u));
                    gs = int4 ? gi : gs;
                }
            } else {
                gs = u2f(f2u(grid_value<FG>(k)) | ((c_cur[i >> 3] << (28 - sh)) & 0x80000000u));
            }
            // P x_hat = (g s P) post with the code's sign (post = 1 is exact); x 4 when folded
            const float xk = (gs * skp) * post;
            const float v = y[i] * P;
            const float ek = xk - v;
            p1[h] = __builtin_fmaf(v, v, p1[h]);
            p2[h] = __builtin_fmaf(ek, ek, p2[h]);
            p3[h] += ek;
            p4[h] += u2f(f2u(ek) ^ (f2u(v) & 0x80000000u));  // sign(y) e (y = +-0 gives e = +-0)
            p5[h] = __builtin_fmaf(xk, v, p5[h]);
            p6[h] += fabsf(ek);
            const int bin = bin0 + (int)k;
            atomicAdd(&bias_bin[bin][tid], (double)(fabsf(gs) - z[i]));
            atomicAdd(&count_bin[bin][tid], 1u);
        }
        constexpr double F2 = FOLD ? 1.0 / 16.0 : 1.0, F1 = FOLD ? 0.25 : 1.0;  // exact
        const double G2 = F2 * Pinv2, G1 = F1 * Pinv;                             // exact
        acc[0] += (double)B;
        acc[1] = __builtin_fma((double)(p1[0] + p1[1]), G2, acc[1]);
        acc[2] = __builtin_fma((double)(p2[0] + p2[1]), G2, acc[2]);
        acc[3] = __builtin_fma((double)(p3[0] + p3[1]), G1, acc[3]);
        acc[4] = __builtin_fma((double)(p4[0] + p4[1]), G1, acc[4]);
        acc[5] = __builtin_fma((double)(p5[0] + p5[1]), G2, acc[5]);
        acc[6] = __builtin_fma((double)(p6[0] + p6[1]), G1, acc[6]);
        acc[7] += 1.0;
        if constexpr (IF4) acc[8] += int4 ? 1.0 : 0.0;
        t = tn;
    }
    double out[NS];
#pragma unroll
    for (int k = 0; k < 9; ++k) out[k] = acc[k];
#pragma unroll
    for (int k = 9; k < NS; ++k) out[k] = 0.0;
    // each thread reads back only its own bins (its own LDS adds are done in
    // order before these reads)
#pragma unroll
    for (int q = 0; q < NBIN; ++q) {
        out[16 + q] = (double)count_bin[q][tid];
        out[32 + q] = bias_bin[q][tid];
    }
    block_reduce_store<NS>(out, a.partials + (int64_t)blockIdx.x * NS);
}

// Workgroups of the statistics grid: as many per compute unit of the current
// device as are resident at once, at most one per STATS_T blocks, at most
// STATS_WGS (the workspace rows).
static int stats_grid(int64_t nblocks, int per_cu)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    int64_t g = (nblocks + STATS_T - 1) / STATS_T;
    const int64_t resident = (int64_t)cus * per_cu;
    if (g > resident) g = resident;
    if (g > STATS_WGS) g = STATS_WGS;
    return g < 1 ? 1 : (int)g;
}

template <int F, int S>
static hipError_t stats_pick(int in_dtype, int rht, const StatsArgs &a, hipStream_t st)
{
    const int64_t nblocks = a.V * (a.L / block_of(S));
    const int g = stats_grid(nblocks, stats_wg_per_cu(block_of(S)));
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
    launch_kernel(reduce_partials_kernel<NS>, dim3(1), dim3(256), st, a.partials, g, a.sums);
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
