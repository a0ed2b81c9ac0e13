// quantize.hip -- fused RHT + block quantization kernels for gfx950.
//
// What is computed: the 4-bit block quantizer of the pages -- an optional
// 16-wide random or deterministic Hadamard transform ("蚂蚁集团揭秘" section 四
// and section 六: Hadamard block = quantization block = 16, fused without
// intermediate storage; MXFP4 page: deterministic H16), a per-block amax
// scale (FP32 single level -- UFP4 recipe table of "当你的 GPU 学不会算账";
// E4M3 with an FP32 tensor scale and IF4's type flag -- IF4 page 3.1-3.2;
// E8M0 -- MXFP4 page), and rounding to E2M1 / E1M2 / INT4 by round-to-nearest-
// even or stochastic rounding (IF4 page 6.1; UFP4 recipe: dY only).
//
// Layout on the chip.  Row kernel: each lane owns one 16-element chunk of a
// view row per step (two 16-byte bf16 loads), so the butterflies, the block
// max and the scale stay in the lane; only E8M0's 32-element blocks combine a
// lane pair through DPP.  A 256-lane workgroup handles 2 x 256 consecutive
// chunks (16 KiB of bf16); codes leave as one 8-byte store per lane.
// Column kernel (the transposed bwd_dw operand): each lane loads 16 rows x 8
// columns (16 loads of 16 bytes, each wave instruction covering eight
// full 128-byte row segments), transforms and quantizes its 8 column blocks in
// registers and writes 8 bytes of codes per column; the 4 waves of a
// workgroup cover 512 rows of 64 columns, so every 128-byte line of the
// transposed code array is written by one workgroup.
//
// Arithmetic.  For bf16 sources the transform's final x 1/4 is exact (every
// partial sum is a multiple of 2^-133), so it is folded into the divisor:
// z = RN(y / s) = RN(v / 4s) with v the unscaled butterfly output.  The
// division is Markstein's reciprocal-and-correct sequence (exact inside the
// scale range checked per block, IEEE division outside it), and the codes come
// from the hardware FP4/FP8 converts, which equal the nearest-even definition.
#include "device.hpp"
#include "kernels.hpp"

namespace ufp4 {

constexpr int RT = 256;  // row kernel: threads per workgroup
constexpr int RU = 2;    // row kernel: 16-element chunks per lane (quantize, transform)
constexpr int RUA = 4;   // row kernel: chunks per lane in the amax pass (4 read cold fastest of 1-16)
// Outputs are written with non-temporal stores: no pass reads its own codes
// and scales back, and keeping them out of the caches leaves room for the
// input, which the next quantization of the same tensor re-reads.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void nt_store16(void *p, uint32_t x, uint32_t y, uint32_t z, uint32_t w)
{
    const u32x4 v = {x, y, z, w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
constexpr int CT = 256;  // column kernel: threads per workgroup
constexpr int CTC = 64;  // column kernel: source columns per workgroup
constexpr int CCG = CTC / 8;          // column kernel: 8-column groups, one per lane of a wave row
constexpr int CRB = 64 / CCG;         // column kernel: 16-row blocks per wave
constexpr int CTR = CT / 64 * CRB * 16; // column kernel: source rows per workgroup
constexpr int COL_GROUP = 8;  // column kernel: row tiles dispatched together

enum : int { MODE_QUANT = 0, MODE_AMAX = 1, MODE_RHT = 2 };

// ---------------------------------------------------------------------------
// Per-tensor and per-block constants
// ---------------------------------------------------------------------------
struct TensorConst {
    float alpha;   // two-level tensor scale
    float den;     // alpha * gridmax
    float inv_den; // RN(1 / den)
    bool den_fast;
};

template <int F, int S>
__device__ __forceinline__ TensorConst tensor_const(const float *amax)
{
    TensorConst t{0.f, 0.f, 0.f, false};
    if constexpr (S == SC_E4M3) {
        const float A = *amax;
        t.alpha = A / (grid_max(F) * 448.0f);
        t.den = t.alpha * grid_max(F);
        t.inv_den = t.den == 0.0f ? 0.0f : 1.0f / t.den;
        t.den_fast = fast_div_ok(t.den);
    }
    return t;
}

struct BlockScale {
    float s;        // effective scale (x_hat = value * s)
    float sd;       // divisor applied to the kernel's values (4 s when x 1/4 is folded)
    float invd;     // RN(1 / sd) where fast (0 otherwise)
    uint32_t byte;  // stored byte (E4M3 / E8M0)
    bool fast;      // Markstein division valid (or s == 0)
    bool sub;       // a scale that can leave |y| / s past the grid's top rounding boundary:
                    // a subnormal scale, an E4M3 byte in the subnormal range, or a
                    // subnormal E4M3 denominator alpha gridmax
};

// m: block amax of the transformed values y.  FOLD: the kernel holds 4y.
template <int F, int S, bool FOLD>
__device__ __forceinline__ BlockScale block_scale(float m, const TensorConst &t)
{
    BlockScale b;
    if constexpr (S == SC_E8M0) {
        int e = m == 0.0f ? -127 : __builtin_amdgcn_frexp_expf(m) - 3;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        b.s = __builtin_amdgcn_ldexpf(1.0f, e);
        b.sd = b.s;
        b.invd = __builtin_amdgcn_ldexpf(1.0f, -e - (FOLD ? 2 : 0));
        b.byte = (uint32_t)(e + 127);
        b.fast = true;
        b.sub = false;
        return b;
    } else {
        if constexpr (S == SC_FP32) {
            b.s = div_by_gridmax<F>(m);
            b.byte = 0;
        } else {
            float delta;
            if (t.den == 0.0f)
                delta = 0.0f;
            else if (t.den_fast && m >= 0x1p-100f)
                delta = div_fast(m, t.den, t.inv_den);
            else
                delta = m / t.den;
            b.byte = e4m3_encode_hw(delta);
            b.s = t.alpha * e4m3_decode_hw(b.byte);
        }
        // (a subnormal scale, or under E4M3 a subnormal alpha gridmax, keeps
        // too few bits for the bound on |z| that the clamp relies on)
        b.sub = b.s != 0.0f && b.s < 0x1p-126f;
        if constexpr (S == SC_E4M3)
            b.sub = b.sub || ((b.byte & 0x78u) == 0 && b.byte != 0) || (t.den != 0.0f && t.den < 0x1p-126f);
        b.sd = FOLD ? b.s * 4.0f : b.s;
        b.fast = b.s == 0.0f || (b.sd >= 0x1p-75f && b.sd <= 0x1p125f);
        // the reciprocal serves the fast quotients only (s and 1 / s normal there)
        const float inv = b.s != 0.0f && b.fast ? rcp_rn(b.s) : 0.0f;
        b.invd = FOLD ? inv * 0.25f : inv;
        return b;
    }
}

// Signed scaled values z_i = RN(y_i / s) for 8 kernel values v_i (v = 4y when
// FOLD).  The fast quotient can be off only for |v| < 2^-100, where |z| <
// 2^-25: RTNE gives code 0 there, and so does SR, which rounds up only from
// 2^-16 of a step above the lower point.
template <int S, bool FOLD, bool SR>
__device__ __forceinline__ void scaled8(const float *v, const BlockScale &b, float *z)
{
    if constexpr (S == SC_E8M0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = v[i] * b.invd;
        return;
    } else {
        if (b.fast) {
#pragma unroll
            for (int i = 0; i < 8; ++i) z[i] = sdiv_fast(v[i], b.sd, b.invd);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) z[i] = (FOLD ? v[i] * 0.25f : v[i]) / b.s;
        }
    }
}

// Codes of 8 elements for the non-IF4 formats.
template <int F, int S, bool FOLD, bool SR>
__device__ __forceinline__ uint32_t encode8(const float *v, const BlockScale &b, const uint32_t *w)
{
    float z[8];
    scaled8<S, FOLD, SR>(v, b, z);
    uint32_t packed;
    if constexpr (SR && F == FMT_E2M1) {
        packed = pack8_e2m1_sr(z, w);
    } else if constexpr (SR) {
        // The rounding must stay within the codes 0..7.  A normal FP32 scale
        // RN(m / gridmax) keeps |z| within 2^-22 of the grid maximum, where
        // stochastic rounding (which rounds up only from 2^-16 of a step)
        // always rounds down: only waves holding a subnormal FP32 scale
        // clamp.  Under E4M3 and E8M0 scales |z| can pass the maximum.
        if (S != SC_FP32 || __builtin_amdgcn_ballot_w64(b.sub) != 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) z[i] = __builtin_amdgcn_fmed3f(z[i], -grid_max(F), grid_max(F));
        }
        packed = pack8_uniform_sr<F>(z, w);
    } else if constexpr (F == FMT_E2M1) {
        packed = pack8_e2m1(z);
    } else if constexpr (e2m1_codes(F)) {
        // capped range: saturate at the cap (a grid point), then nearest even
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = __builtin_amdgcn_fmed3f(z[i], -grid_max(F), grid_max(F));
        packed = pack8_e2m1(z);
    } else {
        if constexpr (S != SC_E8M0) {
            // The rounding of the block scale can leave |z| above the grid
            // maximum.  Past the rounding boundary above it (gridmax + step /
            // 2, where the FP8 convert would leave the code range) only under
            // an E4M3 scale in its subnormal range (a normal one is within
            // 1/16 of Delta, so |z| <= gridmax x 16/15: 3.73 < 3.75 for E1M2,
            // 7.47 < 7.5 for INT4, where the convert's own rounding gives the
            // same code as the clamp) or a subnormal FP32 scale (a normal one
            // is RN(m / gridmax), within a unit in the last place).  Only
            // waves holding such a block clamp.
            if (__builtin_amdgcn_ballot_w64(b.sub) != 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) z[i] = __builtin_amdgcn_fmed3f(z[i], -grid_max(F), grid_max(F));
            }
        }
        packed = pack8_uniform<F>(z);
    }
    return b.s == 0.0f ? 0u : packed;
}

// ---------------------------------------------------------------------------
// Row kernel: one lane per 16-element chunk of a view row (two 16-byte bf16
// loads; each wave instruction covers 2 KiB, the pair of instructions all of
// it).  The transform and the block max stay in the lane; only the 32-element
// E8M0 blocks combine two lanes (DPP).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t row_offset(const RowArgs &a, int64_t ch)
{
    if (a.contiguous) return ch * 16;
    const int64_t L16 = a.L >> 4;
    const int64_t vr = ch / L16;
    return vr * a.ldx + (ch - vr * L16) * 16;
}

template <int IN>
struct Raw16;
template <>
struct Raw16<IN_BF16> {
    uint4 a, b;
};
template <>
struct Raw16<IN_F32> {
    float4 a, b, c, d;
};

template <int IN>
__device__ __forceinline__ Raw16<IN> load_raw(const RowArgs &a, int64_t ch)
{
    Raw16<IN> r;
    const int64_t off = row_offset(a, ch);
    if constexpr (IN == IN_BF16) {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + off);
        r.a = p[0];
        r.b = p[1];
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + off);
        r.a = p[0];
        r.b = p[1];
        r.c = p[2];
        r.d = p[3];
    }
    return r;
}

// Unpack 16 elements, applying the sign diagonal (sgn: sign bit per position).
template <int IN>
__device__ __forceinline__ void unpack16(const Raw16<IN> &r, float *v, const uint32_t *sgn)
{
    if constexpr (IN == IN_BF16) {
        const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
        // sign bits: adding 0x80000000 flips bit 31 only (the low half of w << 16 is zero)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = u2f((w[i] << 16) + sgn[2 * i]);
            v[2 * i + 1] = u2f((w[i] & 0xFFFF0000u) ^ sgn[2 * i + 1]);
        }
    } else {
        const float f[16] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w,
                             r.c.x, r.c.y, r.c.z, r.c.w, r.d.x, r.d.y, r.d.z, r.d.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = u2f(f2u(f[i]) ^ sgn[i]);
    }
}

// 16-point butterflies (spans 1, 2, 4, 8); the final x 1/4 unless FOLD.
template <bool RHT, bool FOLD>
__device__ __forceinline__ void transform16(float *v)
{
    if constexpr (RHT) {
        fwht8(v);
        fwht8(v + 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = v[i], q = v[i + 8];
            v[i] = p + q;
            v[i + 8] = p - q;
        }
        if constexpr (!FOLD) {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = v[i] * 0.25f;
        }
    }
}

__device__ __forceinline__ float absmax16(const float *v)
{
    float m = fmaxf(fabsf(v[0]), fabsf(v[1]));
#pragma unroll
    for (int i = 2; i < 16; i += 2) m = fmaxf(fmaxf(m, fabsf(v[i])), fabsf(v[i + 1]));
    return m;
}

// Quantize one transformed 16-element chunk held by this lane; returns the
// codes (low word: elements 0..7) and sets the scale byte / value.
// IF4 for one 16-element block, on signed values: z = RN(y / s) once; the
// E2M1 candidate's codes from the FP4 convert of z and its grid values from
// the FP4 decode; the INT4 candidate's levels from t = RN(z 7/6), rounded by
// the FP8 convert and read back by its decode.  Both errors in units of the
// scale: g - z and k 6/7 - z (one FMA; each error is odd in y, so its square
// equals the |y| form).  Each candidate's squares accumulate in element
// order, one FMA per element; INT4 iff strictly smaller.  Sets the flag in
// bit 7 of sbyte.
__device__ __forceinline__ void if4_chunk(const float *v, const BlockScale &bs, uint32_t &lo, uint32_t &hi,
                                          uint32_t &sbyte)
{
    constexpr float C76 = 7.0f / 6.0f;
    constexpr float C67 = 6.0f / 7.0f;
    float z[16], t[16];
    if (bs.fast) {
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = sdiv_fast(v[i], bs.s, bs.invd);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = v[i] / bs.s;
    }
    const uint32_t lof = pack8_e2m1(z), hif = pack8_e2m1(z + 8);
    float ef = 0.0f, ei = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const v2f g = decode2_e2m1(j < 4 ? lof : hif, j & 3);
        const float d0 = g.x - z[2 * j], d1 = g.y - z[2 * j + 1];
        ef = __builtin_fmaf(d0, d0, ef);
        ef = __builtin_fmaf(d1, d1, ef);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = z[i] * C76;
    // |t| <= 6 x 16/15 x 7/6 < 7.5 under a normal E4M3 block scale (see
    // encode8): only waves holding a subnormal one clamp
    if (__builtin_amdgcn_ballot_w64(bs.sub) != 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = __builtin_amdgcn_fmed3f(t[i], -7.0f, 7.0f);
    }
    // the levels k = RN(t), ties to even, through the FP8 convert (bytes
    // sign << 7 | |k|, the subnormal |k| 2^-9), read back exactly by the FP8
    // decode: one convert and one decode per pair instead of a rounding per
    // element, and the bytes are the INT4 codes once folded
    uint32_t kb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v2i16 w = {0, 0};
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, t[4 * q], t[4 * q + 1], 512.0f, false);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, t[4 * q + 2], t[4 * q + 3], 512.0f, true);
        kb[q] = __builtin_bit_cast(uint32_t, w);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const v2f k01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(kb[q], 512.0f, false);
        const v2f k23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(kb[q], 512.0f, true);
        const float k[4] = {k01.x, k01.y, k23.x, k23.y};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float d = __builtin_fmaf(k[j], C67, -z[4 * q + j]);
            ei = __builtin_fmaf(d, d, ei);
        }
    }
    const bool use_int = bs.s != 0.0f && ei < ef;
    if (use_int) {
        lo = fold_fp8_codes(kb[0], kb[1]);
        hi = fold_fp8_codes(kb[2], kb[3]);
    } else {
        lo = lof;
        hi = hif;
    }
    if (bs.s == 0.0f) lo = hi = 0;
    sbyte |= use_int ? 0x80u : 0u;
}

template <int F, int S, bool SR, bool FOLD>
__device__ __forceinline__ uint2 quant_chunk(const float *v, const TensorConst &tc, uint64_t n0, uint64_t sr_seed,
                                             uint32_t sr_stream, bool pair_max, uint32_t &sbyte, float &sval)
{
    float m = absmax16(v);
    if constexpr (S == SC_E8M0) {
        if (pair_max) m = fmaxf(m, xor1(m));  // the partner lane holds the other half of the block
    }
    if constexpr (FOLD) m = m * 0.25f;
    const BlockScale bs = block_scale<F == FMT_IF4 ? FMT_E2M1 : F, S, FOLD>(m, tc);
    sbyte = bs.byte;
    sval = bs.s;
    uint32_t lo = 0, hi = 0;
    if constexpr (F == FMT_IF4) {
        if4_chunk(v, bs, lo, hi, sbyte);
    } else {
        uint32_t w[16];
        if constexpr (SR) {
#pragma unroll
            for (int q = 0; q < 2; ++q) sr_words8(n0 + 8 * q, sr_seed, sr_stream, w + 8 * q);
        }
        lo = encode8<F, S, FOLD, SR>(v, bs, w);
        hi = encode8<F, S, FOLD, SR>(v + 8, bs, w + 8);
    }
    return make_uint2(lo, hi);
}

template <int MODE, int F, int S, bool SR, int IN, bool RHT, int OUT, int U>
__device__ __forceinline__ void row_chunk(const RowArgs &a, int64_t ch, float *v, const TensorConst &tc,
                                          float &lmax)
{
    // fold x 1/4 into the divisor for bf16 sources (exact), not for IF4
    constexpr bool FOLD = MODE == MODE_QUANT && RHT && IN == IN_BF16 && F != FMT_IF4;
    transform16<RHT, FOLD>(v);
    if constexpr (MODE == MODE_AMAX) {
        lmax = fmaxf(lmax, absmax16(v));
    } else if constexpr (MODE == MODE_RHT) {
        int64_t off;
        if (a.ldy == a.L) {
            off = ch * 16;
        } else {
            const int64_t L16 = a.L >> 4, vr = ch / L16;
            off = vr * a.ldy + (ch - vr * L16) * 16;
        }
        if constexpr (OUT == IN_F32) {
            // A whole wave of consecutive chunks in a contiguous output goes
            // through LDS, so each of its four stores writes 1 KiB contiguously
            // (per lane they would be 16-byte pieces 64 bytes apart); the
            // stores are non-temporal.  The wave's LDS write and read execute
            // in order: no barrier.
            __shared__ float4 stage[RT / 64][256];
            const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
            const int64_t ch0 = ch - l;  // the chunk of lane 0
            if (a.ldy == a.L && ch0 + 63 < a.n_ch) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    stage[w][4 * l + q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
                f32x4 *p = reinterpret_cast<f32x4 *>(static_cast<float *>(a.y) + ch0 * 16);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 t = stage[w][64 * q + l];
                    const f32x4 r = {t.x, t.y, t.z, t.w};
                    __builtin_nontemporal_store(r, p + 64 * q + l);
                }
            } else {
                float4 *p = reinterpret_cast<float4 *>(static_cast<float *>(a.y) + off);
#pragma unroll
                for (int q = 0; q < 4; ++q) p[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
            }
        } else {
            uint4 *p = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.y) + off);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                p[q] = make_uint4(to_bf16(v[8 * q]) | (to_bf16(v[8 * q + 1]) << 16),
                                  to_bf16(v[8 * q + 2]) | (to_bf16(v[8 * q + 3]) << 16),
                                  to_bf16(v[8 * q + 4]) | (to_bf16(v[8 * q + 5]) << 16),
                                  to_bf16(v[8 * q + 6]) | (to_bf16(v[8 * q + 7]) << 16));
        }
    } else {
        uint32_t sbyte;
        float sval;
        const uint2 codes = quant_chunk<F, S, SR, FOLD>(v, tc, (uint64_t)ch * 16, a.sr_seed, a.sr_stream, true,
                                                        sbyte, sval);
        const u32x2 cv = {codes.x, codes.y};
        __builtin_nontemporal_store(cv, reinterpret_cast<u32x2 *>(a.codes) + ch);
        if constexpr (S == SC_E8M0) {
            if ((ch & 1) == 0) __builtin_nontemporal_store((uint8_t)sbyte, static_cast<uint8_t *>(a.scales) + (ch >> 1));
        } else if constexpr (S == SC_E4M3) {
            __builtin_nontemporal_store((uint8_t)sbyte, static_cast<uint8_t *>(a.scales) + ch);
        } else {
            __builtin_nontemporal_store(sval, static_cast<float *>(a.scales) + ch);
        }
    }
}

template <int MODE, int F, int S, bool SR, int IN, bool RHT, int OUT, int U>
__global__ __launch_bounds__(RT) void row_kernel(const RowArgs a)
{
    const int tid = threadIdx.x;
    uint32_t sgn[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sgn[i] = RHT ? ((a.smask >> i) & 1u) << 31 : 0u;
    TensorConst tc{0.f, 0.f, 0.f, false};
    if constexpr (MODE == MODE_QUANT) tc = tensor_const<F == FMT_IF4 ? FMT_E2M1 : F, S>(a.amax);
    if constexpr (MODE == MODE_QUANT && S == SC_E4M3) {
        if (blockIdx.x == 0 && tid == 0) *a.tensor_scale = tc.alpha;
    }

    const int64_t base = (int64_t)blockIdx.x * (RT * U) + tid;
    float lmax = 0.0f;
    Raw16<IN> raw[U];
    if (base + (U - 1) * RT < a.n_ch) {
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = load_raw<IN>(a, base + u * RT);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v[16];
            unpack16<IN>(raw[u], v, sgn);
            row_chunk<MODE, F, S, SR, IN, RHT, OUT, U>(a, base + u * RT, v, tc, lmax);
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + u * RT < a.n_ch) raw[u] = load_raw<IN>(a, base + u * RT);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + u * RT < a.n_ch) {
                float v[16];
                unpack16<IN>(raw[u], v, sgn);
                row_chunk<MODE, F, S, SR, IN, RHT, OUT, U>(a, base + u * RT, v, tc, lmax);
            }
    }
    if constexpr (MODE == MODE_AMAX) {
        __shared__ float red[RT / 64];
        float m = lmax;
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        if (tid == 0) {
            float w = red[0];
            for (int i = 1; i < RT / 64; ++i) w = fmaxf(w, red[i]);
            a.partials[blockIdx.x] = w;
        }
    }
}

// ---------------------------------------------------------------------------
// Column kernel: the view is the transpose of the source.
// ---------------------------------------------------------------------------
template <int MODE, int F, int S, bool SR, int IN, bool RHT, int OUT>
__global__ __launch_bounds__(CT) void col_kernel(const ColArgs a)
{
    constexpr bool FOLD = MODE == MODE_QUANT && RHT && IN == IN_BF16 && F != FMT_IF4;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane % CCG, b = lane / CCG;
    // Tile order: groups of COL_GROUP row tiles, row tile fastest, so the
    // workgroups in flight write COL_GROUP x CTR / 2 contiguous code bytes of
    // each view row while still sharing the source rows they read.
    int ty, tx;
    {
        const int nx = (int)gridDim.x, ny = (int)gridDim.y;
        const int bid = (int)(blockIdx.y * gridDim.x + blockIdx.x);
        const int grp = bid / (COL_GROUP * nx), in = bid - grp * (COL_GROUP * nx);
        const int gy = min(COL_GROUP, ny - grp * COL_GROUP);
        ty = grp * COL_GROUP + in % gy;
        tx = in / gy;
    }
    const int64_t r0 = (int64_t)ty * CTR + wave * (CRB * 16) + b * 16;  // first source row of this lane
    const int64_t c0 = (int64_t)tx * CTC + g * 8;                // first source column
    const bool active = r0 < a.R && c0 < a.C;

    TensorConst tc{0.f, 0.f, 0.f, false};
    if constexpr (MODE == MODE_QUANT) tc = tensor_const<F == FMT_IF4 ? FMT_E2M1 : F, S>(a.amax);
    if constexpr (MODE == MODE_QUANT && S == SC_E4M3) {
        if (tx == 0 && ty == 0 && tid == 0) *a.tensor_scale = tc.alpha;
    }
    float lmax = 0.0f;

    // A whole tile (in bounds, with 16-byte aligned output rows) stages its
    // codes and scales in LDS; after a barrier the workgroup writes each view
    // row's 256 bytes of codes and its scales as whole lines (written per
    // lane, they would go out as scattered 32- and 16-byte pieces).
    constexpr bool STAGE = MODE == MODE_QUANT;
    constexpr int NB = CTR / 16;  // 16-row blocks in a tile
    constexpr int CP = NB + 1;    // padded pitch (in uint2) of a view row's codes
    __shared__ uint2 st_codes[STAGE ? CTC * CP : 1];
    __shared__ float st_scale[STAGE && S == SC_FP32 ? CTC * CP : 1];
    __shared__ __attribute__((aligned(16))) uint8_t st_sbyte[STAGE && S != SC_FP32 ? CTC * NB : 16];
    const bool staged = STAGE && (a.R % CTR) == 0 && (int64_t)(ty + 1) * CTR <= a.R &&
                        (int64_t)(tx + 1) * CTC <= a.C &&
                        (((uintptr_t)a.codes | (uintptr_t)a.scales) & 15) == 0;  // uniform in the workgroup

    // 16 rows x 8 columns, kept as loaded (bf16 pairs) until each column is
    // processed
    uint4 raw[16];
    if (active) {
        if constexpr (IN == IN_BF16) {
            const uint16_t *xp = static_cast<const uint16_t *>(a.x) + r0 * a.ldx + c0;
#pragma unroll
            for (int i = 0; i < 16; ++i) raw[i] = *reinterpret_cast<const uint4 *>(xp + i * a.ldx);
        }
    }

#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float v[16];
        if (active) {
            if constexpr (IN == IN_BF16) {
                // widen with the sign diagonal applied in the same instruction
                // (the shifted-out half is zero, so adding the sign bit flips it)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint32_t w = (j >> 1) == 0 ? raw[i].x : (j >> 1) == 1 ? raw[i].y : (j >> 1) == 2 ? raw[i].z : raw[i].w;
                    const uint32_t sg = RHT ? ((a.smask >> i) & 1u) << 31 : 0u;
                    v[i] = (j & 1) ? u2f((w & 0xFFFF0000u) ^ sg) : u2f((w << 16) + sg);
                }
            } else {
                const float *xp = static_cast<const float *>(a.x) + r0 * a.ldx + c0 + j;
#pragma unroll
                for (int i = 0; i < 16; ++i) v[i] = xp[i * a.ldx];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = 0.0f;
        }
        if (active && RHT) {
            if constexpr (IN != IN_BF16) {
#pragma unroll
                for (int i = 0; i < 16; ++i) v[i] = u2f(f2u(v[i]) ^ (((a.smask >> i) & 1u) << 31));
            }
            fwht8(v);
            fwht8(v + 8);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p = v[i], q = v[i + 8];
                v[i] = p + q;
                v[i + 8] = p - q;
            }
            if constexpr (!FOLD) {
#pragma unroll
                for (int i = 0; i < 16; ++i) v[i] = v[i] * 0.25f;
            }
        }
        const int64_t c = c0 + j;  // view row
        if constexpr (MODE == MODE_AMAX) {
            if (active) lmax = fmaxf(lmax, absmax16(v));
        } else if constexpr (MODE == MODE_RHT) {
            if (active) {
                const int64_t off = c * a.ldy + r0;
                if constexpr (OUT == IN_F32) {
                    float4 *p = reinterpret_cast<float4 *>(static_cast<float *>(a.y) + off);
#pragma unroll
                    for (int q = 0; q < 4; ++q) p[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
                } else {
                    uint4 *p = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.y) + off);
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        p[q] = make_uint4(to_bf16(v[8 * q]) | (to_bf16(v[8 * q + 1]) << 16),
                                          to_bf16(v[8 * q + 2]) | (to_bf16(v[8 * q + 3]) << 16),
                                          to_bf16(v[8 * q + 4]) | (to_bf16(v[8 * q + 5]) << 16),
                                          to_bf16(v[8 * q + 6]) | (to_bf16(v[8 * q + 7]) << 16));
                }
            }
        } else {
            float m = absmax16(v);
            if constexpr (S == SC_E8M0) {
                // the partner lane (the next 16-row block) holds the other 16 rows
                if constexpr (CCG == 8)
                    m = fmaxf(m, xor8(m));
                else
                    m = fmaxf(m, __shfl_xor(m, CCG));
            }
            if (!active) continue;
            if constexpr (FOLD) m = m * 0.25f;
            const BlockScale bs = block_scale<F == FMT_IF4 ? FMT_E2M1 : F, S, FOLD>(m, tc);
            uint32_t lo = 0, hi = 0;
            uint32_t sbyte = bs.byte;
            if constexpr (F == FMT_IF4) {
                if4_chunk(v, bs, lo, hi, sbyte);
            } else {
                uint32_t w[16];
                if constexpr (SR) {
                    const uint64_t n0 = (uint64_t)c * (uint64_t)a.R + (uint64_t)r0;
#pragma unroll
                    for (int q = 0; q < 2; ++q) sr_words8(n0 + 8 * q, a.sr_seed, a.sr_stream, w + 8 * q);
                }
                lo = encode8<F, S, FOLD, SR>(v, bs, w);
                hi = encode8<F, S, FOLD, SR>(v + 8, bs, w + 8);
            }
            if (staged) {
                const int cl = g * 8 + j, rb = wave * CRB + b;  // tile-local view row, 16-row block
                st_codes[cl * CP + rb] = make_uint2(lo, hi);
                if constexpr (S == SC_E8M0) {
                    if ((b & 1) == 0) st_sbyte[cl * NB + (rb >> 1)] = (uint8_t)sbyte;
                } else if constexpr (S == SC_E4M3) {
                    st_sbyte[cl * NB + rb] = (uint8_t)sbyte;
                } else {
                    st_scale[cl * CP + rb] = bs.s;
                }
                continue;
            }
            *reinterpret_cast<uint2 *>(a.codes + c * (a.R >> 1) + (r0 >> 1)) = make_uint2(lo, hi);
            if constexpr (S == SC_E8M0) {
                if ((b & 1) == 0) static_cast<uint8_t *>(a.scales)[c * (a.R >> 5) + (r0 >> 5)] = (uint8_t)sbyte;
            } else if constexpr (S == SC_E4M3) {
                static_cast<uint8_t *>(a.scales)[c * (a.R >> 4) + (r0 >> 4)] = (uint8_t)sbyte;
            } else {
                static_cast<float *>(a.scales)[c * (a.R >> 4) + (r0 >> 4)] = bs.s;
            }
        }
    }
    if (staged) {
        __syncthreads();
        const int64_t cv0 = (int64_t)tx * CTC;  // first view row of the tile
        const int64_t rs0 = (int64_t)ty * CTR;  // first source row
        // codes: CTC view rows x CTR / 2 bytes, CTR / 32 lanes of 16 bytes per
        // view row
        constexpr int CPARTS = CTR / 32;
#pragma unroll
        for (int q = 0; q < CTC * CPARTS / CT; ++q) {
            const int idx = q * CT + tid, cl = idx / CPARTS, part = idx % CPARTS;
            const uint2 u = st_codes[cl * CP + 2 * part], w = st_codes[cl * CP + 2 * part + 1];
            nt_store16(a.codes + (cv0 + cl) * (a.R >> 1) + (rs0 >> 1) + 16 * part, u.x, u.y, w.x, w.y);
        }
        if constexpr (S == SC_FP32) {
            // CTC view rows x NB scales (CTR / 4 bytes), CTR / 64 lanes of 16
            // bytes per view row
            constexpr int SPARTS = CTR / 64;
#pragma unroll
            for (int q = 0; q < CTC * SPARTS / CT; ++q) {
                const int idx = q * CT + tid, cl = idx / SPARTS, part = idx % SPARTS;
                const float *p = st_scale + cl * CP + 4 * part;
                nt_store16(static_cast<float *>(a.scales) + (cv0 + cl) * (a.R >> 4) + (rs0 >> 4) + 4 * part,
                           __float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]), __float_as_uint(p[3]));
            }
        } else if constexpr (S == SC_E4M3) {
            // CTC view rows x NB bytes, NB / 16 lanes of 16 bytes per view row
            constexpr int BPARTS = NB / 16;
            if (tid < CTC * BPARTS) {
                const int cl = tid / BPARTS, part = tid % BPARTS;
                const uint4 q4 = *reinterpret_cast<const uint4 *>(st_sbyte + cl * NB + 16 * part);
                nt_store16(static_cast<uint8_t *>(a.scales) + (cv0 + cl) * (a.R >> 4) + (rs0 >> 4) + 16 * part, q4.x,
                           q4.y, q4.z, q4.w);
            }
        } else {
            // E8M0: CTC view rows x NB / 2 bytes, one lane per view row
            if (tid < CTC) {
                uint8_t *dst = static_cast<uint8_t *>(a.scales) + (cv0 + tid) * (a.R >> 5) + (rs0 >> 5);
                if constexpr (NB / 2 == 16) {
                    const uint4 q4 = *reinterpret_cast<const uint4 *>(st_sbyte + tid * NB);
                    nt_store16(dst, q4.x, q4.y, q4.z, q4.w);
                } else {
                    static_assert(NB / 2 == 8, "E8M0 scale bytes per view row of a tile");
                    const uint2 q2 = *reinterpret_cast<const uint2 *>(st_sbyte + tid * NB);
                    const u32x2 v = {q2.x, q2.y};
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(dst));
                }
            }
        }
    }
    if constexpr (MODE == MODE_AMAX) {
        __shared__ float red[CT / 64];
        float m = lmax;
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (lane == 0) red[wave] = m;
        __syncthreads();
        if (tid == 0) {
            float w = red[0];
            for (int i = 1; i < CT / 64; ++i) w = fmaxf(w, red[i]);
            a.partials[(int64_t)ty * gridDim.x + tx] = w;
        }
    }
}

// One workgroup: the max of the per-tile partial maxima (exact, any order).
__global__ __launch_bounds__(1024) void amax_final_kernel(const float *partials, int64_t n, float *amax)
{
    __shared__ float red[16];
    // four maxima in turn, so four loads are in flight (max is exact and
    // order-free: any order gives the same result)
    float m4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int64_t i = threadIdx.x;
    for (; i + 3 * 1024 < n; i += 4 * 1024) {
#pragma unroll
        for (int u = 0; u < 4; ++u) m4[u] = fmaxf(m4[u], partials[i + u * 1024]);
    }
#pragma unroll
    for (int u = 0; u < 3; ++u)
        if (i + u * 1024 < n) m4[u] = fmaxf(m4[u], partials[i + u * 1024]);
    float m = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float w = red[0];
        for (int i = 1; i < 16; ++i) w = fmaxf(w, red[i]);
        *amax = w;
    }
}

int64_t amax_tiles(int axis, int64_t rows, int64_t cols)
{
    if (axis == 0) return (rows * cols / 16 + RT * RUA - 1) / (RT * RUA);
    return ((cols + CTC - 1) / CTC) * ((rows + CTR - 1) / CTR);
}

// ---------------------------------------------------------------------------
// Launch helpers: runtime options -> template instance.
// ---------------------------------------------------------------------------
template <int MODE, int F, int S, bool SR, int IN, bool RHT, int OUT>
static hipError_t launch_one(int axis, const RowArgs &ra, const ColArgs &ca, hipStream_t st)
{
    if (axis == 0) {
        if (ra.n_ch == 0) return hipSuccess;
        constexpr int U = MODE == MODE_AMAX ? RUA : RU;
        const int64_t wgs = (ra.n_ch + RT * U - 1) / (RT * U);
        launch_kernel((row_kernel<MODE, F, S, SR, IN, RHT, OUT, U>), dim3((unsigned)wgs), dim3(RT), st, ra);
    } else {
        if (ca.R == 0 || ca.C == 0) return hipSuccess;
        const dim3 grid((unsigned)((ca.C + CTC - 1) / CTC), (unsigned)((ca.R + CTR - 1) / CTR));
        launch_kernel((col_kernel<MODE, F, S, SR, IN, RHT, OUT>), grid, dim3(CT), st, ca);
    }
    return hipGetLastError();
}

template <int F, int S, bool SR, int IN, bool RHT>
static hipError_t pick_quant(int axis, const RowArgs &ra, const ColArgs &ca, hipStream_t st)
{
    return launch_one<MODE_QUANT, F, S, SR, IN, RHT, 0>(axis, ra, ca, st);
}

template <int F, int S, bool SR>
static hipError_t pick_in_rht(const LaunchSpec &sp, const RowArgs &ra, const ColArgs &ca, hipStream_t st)
{
    const bool rht = sp.rht != 0;
    if (sp.in_dtype == IN_BF16)
        return rht ? pick_quant<F, S, SR, IN_BF16, true>(sp.axis, ra, ca, st)
                   : pick_quant<F, S, SR, IN_BF16, false>(sp.axis, ra, ca, st);
    return rht ? pick_quant<F, S, SR, IN_F32, true>(sp.axis, ra, ca, st)
               : pick_quant<F, S, SR, IN_F32, false>(sp.axis, ra, ca, st);
}

template <int F>
static hipError_t pick_scale_sr(const LaunchSpec &sp, const RowArgs &ra, const ColArgs &ca, hipStream_t st)
{
    if constexpr (F == FMT_IF4) {
        return pick_in_rht<FMT_IF4, SC_E4M3, false>(sp, ra, ca, st);
    } else {
        if (sp.scale == SC_E8M0) {
            if constexpr (F == FMT_E2M1) return pick_in_rht<F, SC_E8M0, false>(sp, ra, ca, st);
            return hipErrorInvalidValue;
        }
        if constexpr (F >= FMT_E2M1_M4) {  // capped E2M1: RTNE only
            if (sp.sr) return hipErrorInvalidValue;
            return sp.scale == SC_FP32 ? pick_in_rht<F, SC_FP32, false>(sp, ra, ca, st)
                                       : pick_in_rht<F, SC_E4M3, false>(sp, ra, ca, st);
        }
        if (sp.scale == SC_FP32)
            return sp.sr ? pick_in_rht<F, SC_FP32, true>(sp, ra, ca, st) : pick_in_rht<F, SC_FP32, false>(sp, ra, ca, st);
        return sp.sr ? pick_in_rht<F, SC_E4M3, true>(sp, ra, ca, st) : pick_in_rht<F, SC_E4M3, false>(sp, ra, ca, st);
    }
}

hipError_t launch_quantize(const LaunchSpec &sp, const RowArgs &ra, const ColArgs &ca, hipStream_t st)
{
    switch (sp.format) {
    case FMT_E2M1: return pick_scale_sr<FMT_E2M1>(sp, ra, ca, st);
    case FMT_E1M2: return pick_scale_sr<FMT_E1M2>(sp, ra, ca, st);
    case FMT_INT4: return pick_scale_sr<FMT_INT4>(sp, ra, ca, st);
    case FMT_IF4: return pick_scale_sr<FMT_IF4>(sp, ra, ca, st);
    case FMT_E2M1_M4: return pick_scale_sr<FMT_E2M1_M4>(sp, ra, ca, st);
    case FMT_E2M1_M3: return pick_scale_sr<FMT_E2M1_M3>(sp, ra, ca, st);
    case FMT_E2M1_M2: return pick_scale_sr<FMT_E2M1_M2>(sp, ra, ca, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_amax(const LaunchSpec &sp, const RowArgs &ra, const ColArgs &ca, float *amax, hipStream_t st)
{
    const int64_t tiles = sp.axis == 0 ? (ra.n_ch + RT * RUA - 1) / (RT * RUA)
                                       : ((ca.C + CTC - 1) / CTC) * ((ca.R + CTR - 1) / CTR);
    hipError_t e = hipSuccess;
    if (tiles > 0) {
        const bool rht = sp.rht != 0;
        if (sp.in_dtype == IN_BF16)
            e = rht ? launch_one<MODE_AMAX, 0, 0, false, IN_BF16, true, 0>(sp.axis, ra, ca, st)
                    : launch_one<MODE_AMAX, 0, 0, false, IN_BF16, false, 0>(sp.axis, ra, ca, st);
        else
            e = rht ? launch_one<MODE_AMAX, 0, 0, false, IN_F32, true, 0>(sp.axis, ra, ca, st)
                    : launch_one<MODE_AMAX, 0, 0, false, IN_F32, false, 0>(sp.axis, ra, ca, st);
        if (e != hipSuccess) return e;
    }
    launch_kernel(amax_final_kernel, dim3(1), dim3(1024), st, sp.axis == 0 ? ra.partials : ca.partials, tiles,
                       amax);
    return hipGetLastError();
}

hipError_t launch_rht(const LaunchSpec &sp, int out_dtype, const RowArgs &ra, const ColArgs &ca, hipStream_t st)
{
    const bool rht = sp.rht != 0;
#define UFP4_RHT_CASE(INT, OUTT)                                                                     \
    if (sp.in_dtype == INT && out_dtype == OUTT)                                                     \
        return rht ? launch_one<MODE_RHT, 0, 0, false, INT, true, OUTT>(sp.axis, ra, ca, st)         \
                   : launch_one<MODE_RHT, 0, 0, false, INT, false, OUTT>(sp.axis, ra, ca, st);
    UFP4_RHT_CASE(IN_BF16, IN_F32)
    UFP4_RHT_CASE(IN_BF16, IN_BF16)
    UFP4_RHT_CASE(IN_F32, IN_F32)
    UFP4_RHT_CASE(IN_F32, IN_BF16)
#undef UFP4_RHT_CASE
    return hipErrorInvalidValue;
}

}  // namespace ufp4
