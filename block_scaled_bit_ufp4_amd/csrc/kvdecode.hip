// kvdecode.hip -- FP4 KV-cache decode attention for gfx950.
//
// "FP4 训练 vs FP4 推理：LLM 量化路线正在分叉" (reports.10n1j.top), UltraQuant
// section: decode attention with an FP8 query against an FP4 KV cache with
// UE8M0 group scales, run on CDNA4's native scaled MFMA; K and V are treated
// asymmetrically and K is Walsh-Hadamard rotated.  The definitions (groups of
// 32, the MX exponent rule, the rotation, the FP8 probabilities) are those of
// the ABI header.
//
// Both products run on v_mfma_scale_f32_16x16x128_f8f6f4 with an FP4 A operand
// and an FP8 B operand.  Its operand layout (measured on gfx950):
//   A (FP4): lane l holds row l%16 and the 32 consecutive K values
//            32(l/16) .. 32(l/16)+31 (low nibble first);
//   B (FP8): lane l holds column l%16, bytes 0..15 at K = 16(l/16) + i and
//            bytes 16..31 at K = 64 + 16(l/16) + (i - 16);
//   scales:  lane l supplies the exponent of row / column l%16 for the K block
//            l/16 (K = 32(l/16) .. +31), for either operand;
//   result:  lane l holds column l%16, rows 4(l/16) .. 4(l/16)+3.
//
// S^T = K Q^T: A rows are 16 tokens, A's K is the head dim (so one key group
// per lane and the key scale is the lane's own), B columns are the <= 16 query
// rows.  Eight MFMAs cover a 128-token page; MFMA j row rho holds token
//   tok(j, rho) = 64 (j / 4) + 16 (rho / 4) + 4 (j % 4) + rho % 4,
// so result lane (r, g = l/16) ends up with the scores of exactly the tokens
// that P V's B operand wants in that lane: byte 4j + i <-> MFMA j, result i.
// O^T = V^T P^T: A rows are 16 channels, A's K is the page's 128 tokens (one
// value group per lane), B is P.  MFMA n row rho is channel 8 rho + n, so a
// result lane holds 32 consecutive output channels.
//
// The cache is stored in exactly these operand layouts (see ufp4.h), so every
// load is a 16-byte (or 8-byte) lane load and each instruction reads 1 KiB
// (512 B) of contiguous memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace ufp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int KV_D = 128;
constexpr int KV_PAGE = 128;
constexpr int KV_K_CODES = 0;
constexpr int KV_K_SCALES = 8192;
constexpr int KV_V_CODES = 8704;
constexpr int KV_V_SCALES = 16896;
constexpr int KV_PAGE_BYTES = 17408;
// FP8 (MXFP8) baseline page: the same operands with 32-byte E4M3 lanes.
constexpr int KV8_K_CODES = 0;
constexpr int KV8_K_SCALES = 16384;
constexpr int KV8_V_CODES = 16896;
constexpr int KV8_V_SCALES = 33280;
constexpr int KV8_PAGE_BYTES = 33792;
constexpr int KV_NT = 2;     // cache-policy bits of a buffer load: non-temporal
constexpr int KV_WAVES = 8;  // waves of a decode workgroup (pages are dealt out round-robin)

// Token of score MFMA j, A row rho, inside a page.
__device__ __forceinline__ int page_token(int j, int rho)
{
    return 64 * (j >> 2) + 16 * (rho >> 2) + 4 * (j & 3) + (rho & 3);
}

__device__ __forceinline__ void load_bf16x32(const uint16_t *p, float *y)
{
    const uint4 *s = reinterpret_cast<const uint4 *>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint4 w = s[k];
        y[8 * k + 0] = bf16lo(w.x);
        y[8 * k + 1] = bf16hi(w.x);
        y[8 * k + 2] = bf16lo(w.y);
        y[8 * k + 3] = bf16hi(w.y);
        y[8 * k + 4] = bf16lo(w.z);
        y[8 * k + 5] = bf16hi(w.z);
        y[8 * k + 6] = bf16lo(w.w);
        y[8 * k + 7] = bf16hi(w.w);
    }
}

// Walsh-Hadamard transform over the 128 head-dim channels, spread over the
// four lanes l, l^16, l^32, l^48 (lane chunk c = l/16 holds channels
// 32c .. 32c+31).  Spans 1..16 inside the lane, then 32 (lane ^ 16) and 64
// (lane ^ 32); each butterfly (a, b) -> (a + b, a - b), a the lower channel.
__device__ __forceinline__ void wht128(float *y, int lane)
{
#pragma unroll
    for (int h = 1; h < 32; h <<= 1)
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if ((i & h) == 0) {
                const float a = y[i], b = y[i + h];
                y[i] = a + b;
                y[i + h] = a - b;
            }
#pragma unroll
    for (int s = 16; s <= 32; s <<= 1) {
        const bool upper = (lane & s) != 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float o = __shfl_xor(y[i], s);
            y[i] = upper ? o - y[i] : y[i] + o;
        }
    }
}

__device__ __forceinline__ float absmax32(const float *y)
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(y[i]));
    return m;
}

// UE8M0 exponent floor(log2 amax) - emax clamped below at -127 (amax >= 0,
// finite; zero and subnormal amax give -127 for every emax used here).
__device__ __forceinline__ int mx_exp(float amax, int emax)
{
    const int e = (int)((f2u(amax) >> 23) & 0xFFu) - 127 - emax;
    return e < -127 ? -127 : e;
}

// 2^-e as binary32 (e in [-127, 125]).
__device__ __forceinline__ float pow2_neg(int e) { return u2f((uint32_t)(127 - e) << 23); }

// 32 values -> 16 bytes of E2M1 codes (value i in nibble i).
__device__ __forceinline__ uint4 pack32_e2m1(const float *z)
{
    return make_uint4(pack8_e2m1(z), pack8_e2m1(z + 8), pack8_e2m1(z + 16), pack8_e2m1(z + 24));
}

// Four binary32 values -> four E4M3FN bytes (nearest even; callers keep
// |z| <= 448 so the convert never leaves the finite range).
__device__ __forceinline__ uint32_t pack4_e4m3(float z0, float z1, float z2, float z3)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(z0, z1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(z2, z3, w, true);
    return (uint32_t)w;
}

// MXFP8 of one query row chunk held by a lane (32 channels, already rotated):
// codes in the channel order, and the biased group exponent.
__device__ __forceinline__ uint32_t q_codes32(const float *y, uint32_t *codes)
{
    const int e = mx_exp(absmax32(y), 8);
    const float inv = pow2_neg(e);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = fminf(fmaxf(y[4 * k + i] * inv, -448.0f), 448.0f);
        codes[k] = pack4_e4m3(z[0], z[1], z[2], z[3]);
    }
    return (uint32_t)(e + 127);
}

// The query chunk of lane (row r = l%16, chunk c = l/16): rows >= G are zero.
// With rotation: H_128 q in binary32 times 1/128 (exact).
__device__ __forceinline__ void q_chunk(const uint16_t *q_rows, int G, int rotate, int lane, float *y)
{
    const int r = lane & 15, c = lane >> 4;
    if (r < G) {
        load_bf16x32(q_rows + (int64_t)r * KV_D + 32 * c, y);
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) y[i] = 0.0f;
    }
    if (rotate) {
        wht128(y, lane);
#pragma unroll
        for (int i = 0; i < 32; ++i) y[i] = y[i] * 0.0078125f;
    }
}

// FP8 A-operand order: lane (rho, g) holds K positions 16g .. 16g+15 and
// 64 + 16g .. 64 + 16g + 15.  cw holds this lane's 32 codes in contiguous
// order (positions 32c .. 32c+31 for c = lane / 16); the result gathers the
// two 16-byte halves from lanes (rho, g / 2) and (rho, 2 + g / 2).
__device__ __forceinline__ void fp8_operand_order(const uint32_t *cw, int lane, uint32_t *out)
{
    const int g = lane >> 4, h = g & 1;
    const int src1 = (lane & 15) + 16 * (g >> 1), src2 = src1 + 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a0 = (uint32_t)__shfl((int)cw[i], src1), a1 = (uint32_t)__shfl((int)cw[4 + i], src1);
        const uint32_t b0 = (uint32_t)__shfl((int)cw[i], src2), b1 = (uint32_t)__shfl((int)cw[4 + i], src2);
        out[i] = h ? a1 : a0;
        out[4 + i] = h ? b1 : b0;
    }
}

// ---------------------------------------------------------------------------
// Cache quantizer: one wave per 128-token page.
// ---------------------------------------------------------------------------
struct KvQuantArgs {
    const uint16_t *k, *v;
    int64_t sb, sh, st;  // element strides of batch entry, head, token
    const int32_t *lens;
    int64_t Hkv, L_cap, npages;
    int rotate;
    uint8_t *cache;
};

// The cache is written with non-temporal stores: the pass does not read it
// back, and a decode reads it later from HBM.
typedef unsigned int kv_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int kv_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void nt_store16(uint8_t *p, uint4 v)
{
    const kv_u32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<kv_u32x4 *>(p));
}
__device__ __forceinline__ void nt_store8(uint8_t *p, uint32_t lo, uint32_t hi)
{
    const kv_u32x2 x = {lo, hi};
    __builtin_nontemporal_store(x, reinterpret_cast<kv_u32x2 *>(p));
}

template <bool FP8>
__global__ __launch_bounds__(256) void kv_quantize_kernel(KvQuantArgs a)
{
    constexpr int PB = FP8 ? KV8_PAGE_BYTES : KV_PAGE_BYTES;
    const int lane = threadIdx.x & 63;
    const int64_t page = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t h = blockIdx.y, b = blockIdx.z;
    const int64_t len = min((int64_t)max(a.lens[b], 0), a.L_cap);
    if (page >= a.npages || page * KV_PAGE >= len) return;
    uint8_t *out = a.cache + ((b * a.Hkv + h) * a.npages + page) * PB;
    const int64_t t0 = page * KV_PAGE;

    // K: score-MFMA order, one 32-channel group per lane and instruction.
    {
        const uint16_t *src = a.k + b * a.sb + h * a.sh;
        const int rho = lane & 15, c = lane >> 4;
        uint32_t sc[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t t = t0 + page_token(j, rho);
            float y[32];
            if (t < len) {
                load_bf16x32(src + t * a.st + 32 * c, y);
            } else {
#pragma unroll
                for (int i = 0; i < 32; ++i) y[i] = 0.0f;
            }
            if (a.rotate) wht128(y, lane);
            uint32_t eb;
            if constexpr (FP8) {
                uint32_t cw[8], ow[8];
                eb = q_codes32(y, cw);
                fp8_operand_order(cw, lane, ow);
                uint8_t *dst = out + KV8_K_CODES + j * 2048 + lane * 16;
                nt_store16(dst, make_uint4(ow[0], ow[1], ow[2], ow[3]));
                nt_store16(dst + 1024, make_uint4(ow[4], ow[5], ow[6], ow[7]));
            } else {
                const int e = mx_exp(absmax32(y), 2);
                const float inv = pow2_neg(e);
#pragma unroll
                for (int i = 0; i < 32; ++i) y[i] = y[i] * inv;
                nt_store16(out + KV_K_CODES + j * 1024 + lane * 16, pack32_e2m1(y));
                eb = (uint32_t)(e + 127);
            }
            sc[j >> 2] |= eb << (8 * (j & 3));
        }
        nt_store8(out + (FP8 ? KV8_K_SCALES : KV_K_SCALES) + lane * 8, sc[0], sc[1]);
    }
    // V: lane (rho, g) holds channels 8 rho .. 8 rho + 7 of tokens 32g .. 32g+31.
    {
        const uint16_t *src = a.v + b * a.sb + h * a.sh;
        const int rho = lane & 15, g = lane >> 4;
        uint4 raw[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) {
            const int64_t t = t0 + 32 * g + u;
            raw[u] = t < len ? *reinterpret_cast<const uint4 *>(src + t * a.st + 8 * rho) : make_uint4(0, 0, 0, 0);
        }
        uint32_t sc[2] = {0u, 0u};
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            float y[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const uint32_t w = n < 2 ? raw[u].x : n < 4 ? raw[u].y : n < 6 ? raw[u].z : raw[u].w;
                y[u] = (n & 1) ? bf16hi(w) : bf16lo(w);
            }
            uint32_t eb;
            if constexpr (FP8) {
                uint32_t cw[8], ow[8];
                eb = q_codes32(y, cw);
                fp8_operand_order(cw, lane, ow);
                uint8_t *dst = out + KV8_V_CODES + n * 2048 + lane * 16;
                nt_store16(dst, make_uint4(ow[0], ow[1], ow[2], ow[3]));
                nt_store16(dst + 1024, make_uint4(ow[4], ow[5], ow[6], ow[7]));
            } else {
                const int e = mx_exp(absmax32(y), 2);
                const float inv = pow2_neg(e);
#pragma unroll
                for (int u = 0; u < 32; ++u) y[u] = y[u] * inv;
                nt_store16(out + KV_V_CODES + n * 1024 + lane * 16, pack32_e2m1(y));
                eb = (uint32_t)(e + 127);
            }
            sc[n >> 2] |= eb << (8 * (n & 3));
        }
        nt_store8(out + (FP8 ? KV8_V_SCALES : KV_V_SCALES) + lane * 8, sc[0], sc[1]);
    }
}

// ---------------------------------------------------------------------------
// Standalone MXFP8 query quantizer: one wave per 16 rows, natural layout.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void q_quantize_kernel(const uint16_t *q, int64_t rows, int rotate, uint8_t *codes,
                                                        uint8_t *scales)
{
    const int lane = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * 16;
    const int G = (int)min((int64_t)16, rows - r0);
    float y[32];
    q_chunk(q + r0 * KV_D, G, rotate, lane, y);
    uint32_t cw[8];
    const uint32_t s = q_codes32(y, cw);
    const int r = lane & 15, c = lane >> 4;
    if (r < G) {
        uint4 *dst = reinterpret_cast<uint4 *>(codes + (r0 + r) * KV_D + 32 * c);
        dst[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        dst[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
        scales[(r0 + r) * 4 + c] = (uint8_t)s;
    }
}

// ---------------------------------------------------------------------------
// Decode attention.
// ---------------------------------------------------------------------------
struct KvDecodeArgs {
    const uint16_t *q;      // [B][Hq][128] bf16
    const uint8_t *cache;   // [B][Hkv][npages] pages
    const int32_t *lens;    // [B]
    int64_t Hkv, L_cap, npages;
    int G, pps, nsplit, rotate;
    float c;                // sm_scale * log2(e), rounded to binary32
    float *out;             // [B][Hq][128] (nsplit == 1)
    float *ws_o;            // [B][Hkv][nsplit][G][128] unnormalised partial outputs
    float *ws_ml;           // [B][Hkv][nsplit][G][2]  (integer max m, sum l)
};

// Scaled MFMA with an FP4 (16-byte) or FP8 (32-byte) A operand and an FP8 B
// operand; sel_a picks the byte of scale_a.
__device__ __forceinline__ v4f mfma_kv(const v8i &a, const v8i &b, v4f acc, int sel_a, int scale_a, int scale_b)
{
    switch (sel_a) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, scale_a, 0, scale_b);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 1, scale_a, 0, scale_b);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 2, scale_a, 0, scale_b);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 3, scale_a, 0, scale_b);
    }
}

__device__ __forceinline__ v4f mfma_kv(v4u a, const v8i &b, v4f acc, int sel_a, int scale_a, int scale_b)
{
    const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    switch (sel_a) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, acc, 4, 0, 0, scale_a, 0, scale_b);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, acc, 4, 0, 1, scale_a, 0, scale_b);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, acc, 4, 0, 2, scale_a, 0, scale_b);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, acc, 4, 0, 3, scale_a, 0, scale_b);
    }
}

// One page's operands in registers: FP4 lanes hold 16 bytes per MFMA (v4u),
// FP8 lanes 32 bytes (v8i).
template <bool FP8>
struct Page {
    using Op = typename std::conditional<FP8, v8i, v4u>::type;
    Op kc[8], vc[8];
    v2u ks, vs;
};

// A lane's A operand for one MFMA.  FP4: 16 bytes at lane*16.  FP8: the
// instruction's 2 KiB hold the first 16 bytes of every lane, then the second
// 16 bytes, so each of the two loads reads 1 KiB of whole lines.
template <bool FP8>
__device__ __forceinline__ typename Page<FP8>::Op load_op(__amdgpu_buffer_rsrc_t rs, uint32_t v, int s)
{
    const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(rs, v, s, KV_NT);
    if constexpr (FP8) {
        const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(rs, v + 1024, s, KV_NT);
        return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
        return lo;
    }
}

// Loads of a page's keys (with their exponents) or values go through a buffer
// resource whose range ends at the split's last page: a page past it reads as
// zeros without touching memory, so the prefetch of the next page needs no
// branch.  The page offset is wave-uniform and goes in the scalar offset; the
// per-lane offsets stay fixed.  The cache is read once per step, so the loads
// are non-temporal (measured: 12 % faster on a cache larger than the
// last-level cache).
template <bool FP8>
__device__ __forceinline__ void load_keys(__amdgpu_buffer_rsrc_t rs, int64_t p, uint32_t v16, uint32_t v8,
                                          Page<FP8> &P)
{
    constexpr int PB = FP8 ? KV8_PAGE_BYTES : KV_PAGE_BYTES, STRIDE = FP8 ? 2048 : 1024;
    constexpr int CODES = FP8 ? KV8_K_CODES : KV_K_CODES, SCALES = FP8 ? KV8_K_SCALES : KV_K_SCALES;
    constexpr int PER4K = 4096 / STRIDE;  // instructions per 4 KiB of scalar offset
    const int sp = __builtin_amdgcn_readfirstlane((int)(p * PB));
#pragma unroll
    for (int j = 0; j < 8; ++j)
        P.kc[j] = load_op<FP8>(rs, v16 + (j % PER4K) * STRIDE, sp + CODES + (j / PER4K) * 4096);
    P.ks = __builtin_amdgcn_raw_buffer_load_b64(rs, v8, sp + SCALES, KV_NT);
}

template <bool FP8>
__device__ __forceinline__ void load_values(__amdgpu_buffer_rsrc_t rs, int64_t p, uint32_t v16, uint32_t v8,
                                            Page<FP8> &P)
{
    constexpr int PB = FP8 ? KV8_PAGE_BYTES : KV_PAGE_BYTES, STRIDE = FP8 ? 2048 : 1024;
    constexpr int CODES = FP8 ? KV8_V_CODES : KV_V_CODES, SCALES = FP8 ? KV8_V_SCALES : KV_V_SCALES;
    constexpr int PER4K = 4096 / STRIDE;
    const int sp = __builtin_amdgcn_readfirstlane((int)(p * PB));
#pragma unroll
    for (int n = 0; n < 8; ++n)
        P.vc[n] = load_op<FP8>(rs, v16 + (n % PER4K) * STRIDE, sp + CODES + (n / PER4K) * 4096);
    P.vs = __builtin_amdgcn_raw_buffer_load_b64(rs, v8, sp + SCALES, KV_NT);
}

// Running softmax state of one wave: integer running maximum, the lane's
// share of the normaliser, and the output accumulators (lane (r, g): O[n][i]
// is channel 32g + 8i + n of query row r).
struct DecodeState {
    float m_run, l_lane;
    v4f O[8];
};

// Scores of a page, x[j][i] for token page_token(j, 4g + i) (masked past the
// length), and their maximum in this lane.
template <typename KOp>
__device__ __forceinline__ float page_scores(const KOp *kc, v2u ks, const v8i &qb, int qs, int64_t p, int64_t len,
                                             float c, int g, float (&x)[8][4])
{
    float mloc = -INFINITY;
    const int64_t tbase = p * KV_PAGE + 16 * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const v4f s = mfma_kv(kc[j], qb, (v4f){0.0f, 0.0f, 0.0f, 0.0f}, j & 3, (int)(j < 4 ? ks.x : ks.y), qs);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = tbase + 64 * (j >> 2) + 4 * (j & 3) + i;
            x[j][i] = t < len ? s[i] * c : -INFINITY;
            mloc = fmaxf(mloc, x[j][i]);
        }
    }
    return mloc;
}

// Softmax update of one page and its E4M3 probabilities: the operand pb and
// the biased exponent ps this lane supplies.
__device__ __forceinline__ void page_softmax(float (&x)[8][4], float mloc, int g, DecodeState &st, v8i &pb, int &ps)
{
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(st.m_run, ceilf(mloc));
    const float alpha = ldexpf(1.0f, (int)fmaxf(st.m_run - m_new, -1000.0f));
    st.m_run = m_new;
    st.l_lane *= alpha;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.O[n] *= alpha;

    // probabilities, their sum, and the E4M3 operand with one exponent per
    // 32-token block (block 0/1: first halves of lane groups 0,1 / 2,3;
    // block 2/3: second halves)
    float a1 = 0.0f, a2 = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[j][i] = __builtin_amdgcn_exp2f(x[j][i] - m_new);
            st.l_lane += x[j][i];
            if (j < 4)
                a1 = fmaxf(a1, x[j][i]);
            else
                a2 = fmaxf(a2, x[j][i]);
        }
    a1 = fmaxf(a1, __shfl_xor(a1, 16));
    a2 = fmaxf(a2, __shfl_xor(a2, 16));
    const int e1 = mx_exp(a1, 7), e2 = mx_exp(a2, 7);
    const float inv1 = pow2_neg(e1), inv2 = pow2_neg(e2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float inv = j < 4 ? inv1 : inv2;
        pb[j] = (int)pack4_e4m3(x[j][0] * inv, x[j][1] * inv, x[j][2] * inv, x[j][3] * inv);
    }
    // lane group g supplies block g: groups 0 and 3 hold it (e1, e2), groups
    // 1 and 2 take it from the partner group 3 (its e1) or 0 (its e2)
    const int recv = __shfl_xor(g >= 2 ? e1 : e2, 32);
    const int keep = g == 0 ? e1 : e2;
    const int swap = -(int)((unsigned)(g - 1) < 2u);
    ps = ((recv & swap) | (keep & ~swap)) + 127;
}

// O += V^T P^T for one page.
template <typename VOp>
__device__ __forceinline__ void page_pv(const VOp *vc, v2u vs, const v8i &pb, int ps, DecodeState &st)
{
#pragma unroll
    for (int n = 0; n < 8; ++n) st.O[n] = mfma_kv(vc[n], pb, st.O[n], n & 3, (int)(n < 4 ? vs.x : vs.y), ps);
}

template <bool FP8>
__global__ __launch_bounds__(64 * KV_WAVES) __attribute__((amdgpu_waves_per_eu(2))) void kv_decode_kernel(KvDecodeArgs a)
{
    constexpr int PB = FP8 ? KV8_PAGE_BYTES : KV_PAGE_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t q_lds[16 * KV_D + 64];
    __shared__ float o_lds[KV_WAVES][16][KV_D];
    __shared__ float ml_lds[KV_WAVES][16][2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x;
    const int64_t h = blockIdx.y, b = blockIdx.z;
    const int r = lane & 15, g = lane >> 4;
    const int64_t Hq = a.Hkv * a.G;

    const int64_t len = min((int64_t)max(a.lens[b], 0), a.L_cap);
    const int64_t npg = (len + KV_PAGE - 1) / KV_PAGE;
    const int64_t p0 = (int64_t)split * a.pps;
    const int64_t p1 = max(p0, min(p0 + a.pps, npg));
    const uint8_t *seq = a.cache + (b * a.Hkv + h) * a.npages * PB;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(seq), (short)0, (int)(p1 * PB), 0x00020000);

    int64_t p = p0 + wave;
    const uint32_t v16 = (uint32_t)lane * 16u, v8 = (uint32_t)lane * 8u;
    // the first page, in the loop's order (keys with their scales, then
    // values), so the loop's waits count the same outstanding loads on every
    // entry
    Page<FP8> cur;
    load_keys(rs, p, v16, v8, cur);
    __builtin_amdgcn_sched_barrier(0);
    load_values(rs, p, v16, v8, cur);
    __builtin_amdgcn_sched_barrier(0);

    // Query operand: wave 0 quantizes (contiguous chunks), all waves read it
    // back in the B-operand order.
    if (wave == 0) {
        float y[32];
        q_chunk(a.q + (b * Hq + h * a.G) * KV_D, a.G, a.rotate, lane, y);
        uint32_t cw[8];
        const uint32_t s = q_codes32(y, cw);
        uint4 *dst = reinterpret_cast<uint4 *>(q_lds + r * KV_D + 32 * g);
        dst[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        dst[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
        q_lds[16 * KV_D + r * 4 + g] = (uint8_t)s;
    }
    __syncthreads();
    v8i qb;
    {
        const uint4 lo = *reinterpret_cast<const uint4 *>(q_lds + r * KV_D + 16 * g);
        const uint4 hi = *reinterpret_cast<const uint4 *>(q_lds + r * KV_D + 64 + 16 * g);
        qb = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    const int qs = q_lds[16 * KV_D + r * 4 + g];

    DecodeState st;
    st.m_run = -INFINITY;
    st.l_lane = 0.0f;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.O[n] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    // One register set: the next page's keys load once the score MFMAs have
    // read the current ones, its values once P V has, so about one page per
    // wave is in flight at all times.
    while (p < p1) {
        float x[8][4];
        const float mloc = page_scores(cur.kc, cur.ks, qb, qs, p, len, a.c, g, x);
        __builtin_amdgcn_sched_barrier(0);
        load_keys(rs, p + KV_WAVES, v16, v8, cur);
        __builtin_amdgcn_sched_barrier(0);
        v8i pb;
        int ps;
        page_softmax(x, mloc, g, st, pb, ps);
        page_pv(cur.vc, cur.vs, pb, ps, st);
        __builtin_amdgcn_sched_barrier(0);
        load_values(rs, p + KV_WAVES, v16, v8, cur);
        __builtin_amdgcn_sched_barrier(0);
        p += KV_WAVES;
    }
    const float m_run = st.m_run, l_lane = st.l_lane;
    v4f O[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) O[n] = st.O[n];

    float l_row = l_lane + __shfl_xor(l_lane, 16);
    l_row += __shfl_xor(l_row, 32);
    // lane (r, g): O[n][i] = output channel 32g + 8i + n of query row r
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 *d = reinterpret_cast<float4 *>(&o_lds[wave][r][32 * g + 8 * i]);
        d[0] = make_float4(O[0][i], O[1][i], O[2][i], O[3][i]);
        d[1] = make_float4(O[4][i], O[5][i], O[6][i], O[7][i]);
    }
    if (g == 0) {
        ml_lds[wave][r][0] = m_run;
        ml_lds[wave][r][1] = l_row;
    }
    __syncthreads();

    // merge the waves: thread t -> row t/32, channels 4 (t%32) .. +3
    const int t = threadIdx.x, row = t >> 5, d0 = (t & 31) * 4;
    if (row >= a.G) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < KV_WAVES; ++w) M = fmaxf(M, ml_lds[w][row][0]);
    float o[4] = {0, 0, 0, 0}, lsum = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < KV_WAVES; ++w) {
            const float f = ldexpf(1.0f, (int)fmaxf(ml_lds[w][row][0] - M, -1000.0f));
            lsum += ml_lds[w][row][1] * f;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] += o_lds[w][row][d0 + k] * f;
        }
    }
    if (a.nsplit == 1) {
        const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
        *reinterpret_cast<float4 *>(a.out + ((b * Hq + h * a.G + row) * KV_D + d0)) =
            make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    } else {
        const int64_t slot = ((b * a.Hkv + h) * a.nsplit + split) * a.G + row;
        *reinterpret_cast<float4 *>(a.ws_o + slot * KV_D + d0) = make_float4(o[0], o[1], o[2], o[3]);
        if ((t & 31) == 0) {
            a.ws_ml[slot * 2 + 0] = M;
            a.ws_ml[slot * 2 + 1] = lsum;
        }
    }
}

// Combine the splits of one query row: grid B * Hq, 128 threads (channels).
__global__ __launch_bounds__(128) void kv_combine_kernel(KvDecodeArgs a)
{
    const int64_t bq = blockIdx.x;
    const int64_t Hq = a.Hkv * a.G;
    const int64_t b = bq / Hq, hq = bq % Hq, h = hq / a.G, row = hq % a.G;
    const int d = threadIdx.x;
    const int64_t slot0 = (b * a.Hkv + h) * a.nsplit * a.G + row;
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.ws_ml[(slot0 + (int64_t)s * a.G) * 2]);
    float o = 0.0f, lsum = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < a.nsplit; ++s) {
            const int64_t slot = slot0 + (int64_t)s * a.G;
            const float f = ldexpf(1.0f, (int)fmaxf(a.ws_ml[slot * 2] - M, -1000.0f));
            lsum += a.ws_ml[slot * 2 + 1] * f;
            o += a.ws_o[slot * KV_D + d] * f;
        }
    }
    a.out[bq * KV_D + d] = lsum > 0.0f ? o / lsum : 0.0f;
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
hipError_t launch_kv_quantize(const uint16_t *k, const uint16_t *v, int64_t B, int64_t Hkv, int64_t L_cap, int fp8,
                              int64_t sb, int64_t sh, int64_t st, const int32_t *lens, int rotate, uint8_t *cache,
                              hipStream_t s)
{
    KvQuantArgs a{k, v, sb, sh, st, lens, Hkv, L_cap, L_cap / KV_PAGE, rotate, cache};
    const dim3 grid((unsigned)((a.npages + 3) / 4), (unsigned)Hkv, (unsigned)B);
    if (fp8)
        launch_kernel(kv_quantize_kernel<true>, grid, dim3(256), s, a);
    else
        launch_kernel(kv_quantize_kernel<false>, grid, dim3(256), s, a);
    return hipGetLastError();
}

hipError_t launch_q_quantize(const uint16_t *q, int64_t rows, int rotate, uint8_t *codes, uint8_t *scales, hipStream_t s)
{
    launch_kernel(q_quantize_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(64), s, q, rows, rotate, codes, scales);
    return hipGetLastError();
}

hipError_t launch_kv_decode(const uint16_t *q, const uint8_t *cache, const int32_t *lens, int64_t B, int64_t Hkv, int G,
                            int fp8, int64_t L_cap, float c, int rotate, int pps, int nsplit, float *out, float *ws_o,
                            float *ws_ml, hipStream_t s)
{
    KvDecodeArgs a{q, cache, lens, Hkv, L_cap, L_cap / KV_PAGE, G, pps, nsplit, rotate, c, out, ws_o, ws_ml};
    const dim3 grid((unsigned)nsplit, (unsigned)Hkv, (unsigned)B);
    if (fp8)
        launch_kernel(kv_decode_kernel<true>, grid, dim3(64 * KV_WAVES), s, a);
    else
        launch_kernel(kv_decode_kernel<false>, grid, dim3(64 * KV_WAVES), s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit == 1) return e;
    launch_kernel(kv_combine_kernel, dim3((unsigned)(B * Hkv * G)), dim3(128), s, a);
    return hipGetLastError();
}

}  // namespace ufp4
