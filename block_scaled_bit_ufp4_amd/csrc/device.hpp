// device.hpp -- gfx950 device helpers of the 4-bit block quantizer.
//
// Number formats: E2M1 {0,.5,1,1.5,2,3,4,6} and E1M2 {0,.5,...,3.5}
// ("当你的 GPU 学不会算账" sections "E2M1：一块刻度不均的尺子" and "UFP4：换一把
// 尺子"); INT4 {0..7} and the E4M3 / UE8M0 scale formats (IF4 page, section 2.2
// format table; MXFP4 page, section on MXFP4).  Philox4x32-10 from Salmon et al.,
// "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
//
// Every function here computes exactly (bit for bit) the binary32 result the
// ABI header defines; the faster formulations are justified next to them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ufp4 {

enum : int { FMT_E2M1 = 0, FMT_E1M2 = 1, FMT_INT4 = 2, FMT_IF4 = 3, FMT_E2M1_M4 = 4, FMT_E2M1_M3 = 5, FMT_E2M1_M2 = 6 };
enum : int { SC_FP32 = 0, SC_E4M3 = 1, SC_E8M0 = 2 };
enum : int { IN_BF16 = 0, IN_F32 = 1 };

typedef short v2i16 __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr float grid_max(int f)
{
    return f == FMT_E1M2      ? 3.5f
           : f == FMT_INT4    ? 7.0f
           : f == FMT_E2M1_M4 ? 4.0f
           : f == FMT_E2M1_M3 ? 3.0f
           : f == FMT_E2M1_M2 ? 2.0f
                              : 6.0f;
}
// E2M1 codes: the full grid and the range-capped variants (points up to the cap)
__host__ __device__ constexpr bool e2m1_codes(int f) { return f == FMT_E2M1 || f >= FMT_E2M1_M4; }
__host__ __device__ constexpr int block_of(int scl) { return scl == SC_E8M0 ? 32 : 16; }

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// ---------------------------------------------------------------------------
// Cross-lane moves (DPP, wave64).  quad_perm [1,0,3,2] = lane ^ 1,
// quad_perm [2,3,0,1] = lane ^ 2, row_ror:8 = lane ^ 8 inside 16-lane rows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor1(float v)
{
    return u2f((uint32_t)__builtin_amdgcn_mov_dpp((int)f2u(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float xor2(float v)
{
    return u2f((uint32_t)__builtin_amdgcn_mov_dpp((int)f2u(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float xor8(float v)
{
    return u2f((uint32_t)__builtin_amdgcn_mov_dpp((int)f2u(v), 0x128, 0xF, 0xF, true));
}

// ---------------------------------------------------------------------------
// Philox4x32-10: ten rounds of two 32x32->64 multiplies by the SC'11
// constants; the key advances by the two Weyl increments between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox10(uint4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        // three-way xors in one instruction each (v_bitop3_b32, truth table 0x96)
        c = make_uint4(__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96), (uint32_t)p1,
                       __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96), (uint32_t)p0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// SR words of view elements n0..n0+7 (n0 a multiple of 8), one Philox block at
// counter n0 / 8: the 32-bit output words are read 16 bits at a time, low half
// first, and each element's 16 bits go to the top half of its word (the low
// half zero), where both stochastic-rounding converts read their random bits.
__device__ __forceinline__ void sr_words8(uint64_t n0, uint64_t seed, uint32_t stream, uint32_t *w)
{
    const uint64_t q = n0 >> 3;
    const uint4 r = philox10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), stream, 0u), (uint32_t)seed,
                             (uint32_t)(seed >> 32));
    const uint32_t o[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w[2 * j] = o[j] << 16;
        w[2 * j + 1] = o[j] & 0xFFFF0000u;
    }
}

// ---------------------------------------------------------------------------
// 16-point Walsh-Hadamard butterflies, spans 1, 2, 4 inside 8 registers.
// (a, b) -> (a + b, a - b), the same additions in the same order as the
// definition, so the results are identical whatever the lane layout.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fwht8(float *v)
{
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

// Full 16-point transform in registers (span 8 last), then x 1/4.
__device__ __forceinline__ void fwht16_local(float *v)
{
    fwht8(v);
    fwht8(v + 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = v[i], b = v[i + 8];
        v[i] = a + b;
        v[i + 8] = a - b;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = v[i] * 0.25f;
}

// ---------------------------------------------------------------------------
// Division.  z = RN(a / s) for a >= 0 as  q = a*inv, r = fma(-q, s, a),
// z = fma(r, inv, q)  with inv = RN(1/s): Markstein's correction step, exact
// when the residual r does not underflow.  Conditions used here: s in
// [2^-75, 2^125] and a >= 2^-100 (r is then a normal number); for a < 2^-100
// the quotient is below 2^-25, where every rounding gives code 0 (RTNE, and
// stochastic rounding, which rounds up only from 2^-16 of a step).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool fast_div_ok(float s) { return s >= 0x1p-75f && s <= 0x1p125f; }

// RN(1 / s) for s and 1 / s normal: the hardware reciprocal (within one unit
// in the last place) refined by one Newton step on the FMA.  On gfx950 this is
// the correctly rounded reciprocal for every binary32 significand (checked
// exhaustively against the IEEE division at exponents -75 to 124), at 3
// instructions against about 11 for the division.
__device__ __forceinline__ float rcp_rn(float s)
{
    const float r = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r);
}

__device__ __forceinline__ float div_fast(float a, float s, float inv)
{
    const float q = a * inv;
    const float r = __builtin_fmaf(-q, s, a);
    return __builtin_fmaf(r, inv, q);
}

// Signed form: RN(y / s) for either sign, q = y*inv, r = q*s - y (exact),
// z = q - r*inv.  Writing the correction as a subtraction keeps the sign of a
// zero quotient (y = -0 gives -0, as the division does).
__device__ __forceinline__ float sdiv_fast(float y, float s, float inv)
{
    const float q = y * inv;
    const float r = __builtin_fmaf(q, s, -y);
    return __builtin_fmaf(-r, inv, q);
}

// RN(m / G) for a constant G (the grid maximum), m >= 0.
template <int F>
__device__ __forceinline__ float div_by_gridmax(float m)
{
    constexpr float G = grid_max(F);
    constexpr float INV = 1.0f / G;
    if (m >= 0x1p-100f) return div_fast(m, G, INV);
    return m / G;
}

// ---------------------------------------------------------------------------
// E4M3FN (bias 7, max 448, subnormal step 2^-9): nearest, ties to even,
// saturating.  Input v >= 0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float v)
{
    if (!(v < 448.0f)) return 0x7Eu;
    if (v < 0x1p-6f) {
        // subnormal range: multiples of 2^-9; x 512 is exact, rint is RNE;
        // q = 8 is 2^-6, whose encoding 0x08 is the same integer
        return (uint32_t)__builtin_rintf(v * 512.0f);
    }
    // normal range: round the binary32 significand to 3 bits (nearest even)
    const uint32_t b = f2u(v);
    const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
    const uint32_t code = (r >> 20) - (120u << 3);
    return code > 0x7Eu ? 0x7Eu : code;
}

// The same encoding with the hardware FP8 convert (identical to e4m3_encode
// for every input below 464, verified exhaustively on gfx950; the clamp to
// 448 provides the saturation the convert does not).
__device__ __forceinline__ uint32_t e4m3_encode_hw(float v)
{
    v2i16 w = {0, 0};
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, fminf(v, 448.0f), 0.0f, 1.0f, false);
    return (uint32_t)(uint16_t)w[0] & 0xFFu;
}

// Decoding with the hardware FP8 convert (gfx950's FP8 is the OCP E4M3FN
// format); exact for every byte 0x00..0x7E.
__device__ __forceinline__ float e4m3_decode_hw(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

__device__ __forceinline__ float e4m3_decode(uint32_t b)
{
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 0) return (float)m * 0x1p-9f;
    return u2f(((e + 120u) << 23) | (m << 20));
}

// ---------------------------------------------------------------------------
// Magnitude codes, round to nearest even.  a >= 0 (a = |z|).
//   E1M2: k = rint(2a), clamped to 7: min(a, 3.5) * 2 + 2^23 rounds 2a to an
//         integer (RNE) in the low mantissa bits.
//   INT4: k = rint(a) clamped to 7, the same way.
//   E2M1: below 1 the step is 0.5 (k = rint(2a) in {0,1,2}); from 1 up the
//         code is the binary32 value rounded to one mantissa bit (RNE), read
//         off the exponent and that bit; clamped to 7 (saturation at 6).
// Each equals the nearest-grid-point definition with ties to the even code.
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ uint32_t rtne_code(float a)
{
    if constexpr (F == FMT_E1M2) {
        return f2u(__builtin_fmaf(fminf(a, 3.5f), 2.0f, 0x1p23f)) & 7u;
    } else if constexpr (F == FMT_INT4) {
        return f2u(fminf(a, 7.0f) + 0x1p23f) & 7u;
    } else {
        const uint32_t lo = f2u(__builtin_fmaf(fminf(a, 1.0f), 2.0f, 0x1p23f)) & 7u;
        const uint32_t b = f2u(fminf(a, 8.0f));
        const uint32_t r = b + 0x1FFFFFu + ((b >> 22) & 1u);
        const uint32_t hi = min((r >> 22) - 252u, 7u);
        return a < 1.0f ? lo : hi;
    }
}

// ---------------------------------------------------------------------------
// Hardware converts (verified on gfx950 against the software definitions for
// every finite binary32: the FP4 convert equals the nearest-even E2M1 code
// with saturation at 6; the FP8 convert with scale 2^8 (2^9) returns
// sign << 7 | rint(2|z|) (rint(|z|)) for |z| < 7.75 (15.5).  Both convert
// pairs: src0 to the low field.  The scale operand only contributes its
// power-of-two exponent (the convert divides by it).
// ---------------------------------------------------------------------------
// 8 signed scaled values -> 8 E2M1 codes (element i in bits 4i..4i+3).
__device__ __forceinline__ uint32_t pack8_e2m1(const float *z)
{
    uint32_t p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, z[0], z[1], 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, z[2], z[3], 1.0f, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, z[4], z[5], 1.0f, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, z[6], z[7], 1.0f, 3);
    return p;
}

// Two E2M1 codes (byte b of w: low nibble first) -> their values (exact;
// the scale operand 1.0 leaves them unscaled).
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2f decode2_e2m1(uint32_t w, int b)
{
    switch (b) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    }
}

// The FP8 convert's bytes of 8 values (d0: elements 0..3, d1: 4..7), each
// sign << 7 | k with k <= 7 (bits 3..6 clear), as 8 codes sign << 3 | k, byte j
// holding element 2j in its low nibble and 2j + 1 in its high one: v_perm
// gathers the even and the odd elements' bytes, then a 4-bit shift brings each
// byte's sign next to its k (right for the low nibbles, left for the high ones).
__device__ __forceinline__ uint32_t fold_fp8_codes(uint32_t d0, uint32_t d1)
{
    const uint32_t ev = __builtin_amdgcn_perm(d1, d0, 0x06040200u);  // elements 0, 2, 4, 6
    const uint32_t od = __builtin_amdgcn_perm(d1, d0, 0x07050301u);  // elements 1, 3, 5, 7
    return (((od << 4) | od) & 0xF0F0F0F0u) | ((ev | (ev >> 4)) & 0x0F0F0F0Fu);
}

// 8 signed scaled values on the uniform grids -> 8 codes: the FP8 convert
// gives bytes sign<<7 | k, folded into nibbles.  Requires |z| <= gridmax (+
// less than half a step).
template <int F>
__device__ __forceinline__ uint32_t pack8_uniform(const float *z)
{
    constexpr float SC = F == FMT_E1M2 ? 256.0f : 512.0f;
    v2i16 w0 = {0, 0}, w1 = {0, 0};
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, z[0], z[1], SC, false);
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, z[2], z[3], SC, true);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, z[4], z[5], SC, false);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, z[6], z[7], SC, true);
    return fold_fp8_codes(__builtin_bit_cast(uint32_t, w0), __builtin_bit_cast(uint32_t, w1));
}

// Stochastic rounding of 8 signed scaled values onto a uniform grid through
// the FP8 convert with stochastic rounding: the caller keeps |z| at or below
// the grid maximum, or so little above it that the rounding goes down (so
// 2|z|, or |z| for INT4, stays within the subnormal codes 0..7), and the
// convert returns sign << 7 | k with k = k_lo + 1 exactly when (w >> 12) +
// floor(frac 2^20) reaches 2^20, frac = t - k_lo (checked on gfx950 against
// that rule on 2^30 pairs per grid: z of every binary32 exponent and sign, w
// random or at the rounding threshold and one below).  The words w come from
// sr_words8, their low 16 bits zero: with h = w >> 16, (w >> 12) = 16 h, and
// 16 h + floor(frac 2^20) >= 2^20 holds exactly when h + floor(frac 2^16) >=
// 2^16, the 16-bit rule.  The bytes fold into nibbles as in pack8_uniform.
template <int F>
__device__ __forceinline__ uint32_t pack8_uniform_sr(const float *z, const uint32_t *w)
{
    constexpr float SC = F == FMT_E1M2 ? 256.0f : 512.0f;
    int d0 = 0, d1 = 0;
    d0 = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d0, z[0], w[0], SC, 0);
    d0 = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d0, z[1], w[1], SC, 1);
    d0 = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d0, z[2], w[2], SC, 2);
    d0 = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d0, z[3], w[3], SC, 3);
    d1 = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d1, z[4], w[4], SC, 0);
    d1 = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d1, z[5], w[5], SC, 1);
    d1 = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d1, z[6], w[6], SC, 2);
    d1 = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(d1, z[7], w[7], SC, 3);
    return fold_fp8_codes((uint32_t)d0, (uint32_t)d1);
}

// Stochastic rounding of 8 signed scaled values onto E2M1 through the packed
// FP4 convert with stochastic rounding.  That convert rounds its first value
// up when (seed >> 10) + floor(frac 2^22) reaches 2^22 (and feeds the second
// a rotated copy of the seed).  The words of sr_words8 have their low 16 bits
// clear, so seed >> 10 = 64 h with h = w >> 16, and 64 h + floor(frac 2^22) >=
// 2^22 holds exactly when h + floor(frac 2^16) >= 2^16: the 16-bit rule of the
// uniform grids.  One value per convert, the second 0 (code 0), into byte 0:
// this builtin does not keep the other bytes of its first operand (they come
// back as whatever the destination register held), so only byte 0 of each
// result is used and v_perm gathers them, the even elements' codes into the
// low nibbles of one word and the odd ones' into another, shifted up.
__device__ __forceinline__ uint32_t sr_fp4_byte0(float z, uint32_t w)
{
    const v2f p = {z, 0.0f};
    return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, w, 1.0f, 0);
}
__device__ __forceinline__ uint32_t gather_byte0(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3)
{
    // bytes [r0.b0, r1.b0, 0, 0] | [0, 0, r2.b0, r3.b0]
    return __builtin_amdgcn_perm(r1, r0, 0x0c0c0400u) | __builtin_amdgcn_perm(r3, r2, 0x04000c0cu);
}
__device__ __forceinline__ uint32_t pack8_e2m1_sr(const float *z, const uint32_t *w)
{
    uint32_t r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = sr_fp4_byte0(z[i], w[i]);
    const uint32_t e = gather_byte0(r[0], r[2], r[4], r[6]);
    const uint32_t o = gather_byte0(r[1], r[3], r[5], r[7]);
    return e | (o << 4);
}

// Grid value of a magnitude code.
template <int F>
__device__ __forceinline__ float grid_value(uint32_t k)
{
    if constexpr (F == FMT_E1M2) return (float)k * 0.5f;
    if constexpr (F == FMT_INT4) return (float)k;
    // E2M1: 0, .5, 1, 1.5, 2, 3, 4, 6
    const uint32_t e = k >> 1, m = k & 1u;
    return e == 0 ? (float)m * 0.5f : u2f(((e + 126u) << 23) | (m << 22));
}

// bf16 bits -> binary32
__device__ __forceinline__ float bf16lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }

// binary32 -> bf16 bits, nearest even (finite inputs)
__device__ __forceinline__ uint32_t to_bf16(float f)
{
    const uint32_t u = f2u(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace ufp4
