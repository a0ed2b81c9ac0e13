// gemm.hip -- block-scaled GEMM on CDNA4 matrix cores.
//
// Z = A B^T with both operands K-major.  The MXFP4 path feeds E2M1 codes
// with their UE8M0 block scales straight into the scaled MFMA (FP4 tensors
// with UE8M0 group scales on the native scaled-MFMA path: "FP4 训练 vs FP4
// 推理", UltraQuant; MXFP4 blocks of 32 sharing an E8M0 exponent: MXFP4
// page).  The bf16 path multiplies bf16 operands on the bf16 MFMA (the
// software route for E1M2/INT4 that FP4-only hardware needs: same page, "保留
// FP4 计算，用软件模拟 E1M2 / INT4 路径").  Both accumulate in binary32.
//
// Both paths move operands as bytes: a K-major row supplies 64 bytes per
// pipeline stage (128 E2M1 codes or 32 bf16 values), and one 32x32 MFMA step
// consumes 32 bytes of each of 32 rows, lane l holding row l mod 32 and the
// 16-byte half l / 32 (32 FP4 codes of one 32-element scale block, or 8 bf16).
// Workgroup tile 256 x 256, 4 waves of 128 x 128 (4 x 4 MFMA tiles of 32 x 32,
// 256 fp32 accumulators per lane), two LDS stages of 256 rows x 64 bytes per
// operand with the 16-byte chunks of each row XOR-swizzled so the 16-byte
// fragment reads are free of bank conflicts.  Workgroups are ordered so that
// the eight XCDs each work on a compact band of output tiles.
#include "device.hpp"
#include "kernels.hpp"

namespace ufp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int GBM = 256;   // workgroup tile rows (M)
constexpr int GBN = 256;   // workgroup tile columns (N)
constexpr int GKB = 64;    // bytes of K per row per stage
constexpr int GT = 256;    // threads
constexpr int GROUP_M = 8; // tile-row group of the raster order

// byte offset of 16-byte chunk c of row r in a stage (64 bytes per row)
__device__ __forceinline__ int lds_off(int r, int c) { return r * GKB + ((c ^ ((r >> 2) & 3)) << 4); }

// tile index -> (tile row, tile column): XCD-contiguous bands, then a grouped
// raster inside each band
__device__ __forceinline__ void tile_of(int bid, int MT, int NT, int &tm, int &tn)
{
    const int T = MT * NT;
    int t = bid;
    if ((T & 7) == 0) t = (bid & 7) * (T >> 3) + (bid >> 3);
    const int per_group = GROUP_M * NT;
    const int g = t / per_group;
    const int first_m = g * GROUP_M;
    const int gsz = min(MT - first_m, GROUP_M);
    const int r = t - g * per_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

template <bool FP4>
__global__ __launch_bounds__(GT, 1) void gemm_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA,
                                                     const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB,
                                                     int M, int N, int64_t kbytes, int64_t lda, int64_t ldb,
                                                     int64_t lds_a, int64_t lds_b, float *__restrict__ C, int64_t ldc)
{
    __shared__ __attribute__((aligned(16))) uint8_t As[2][GBM * GKB];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][GBN * GKB];
    __shared__ uint32_t Ss[2][2][GBM];  // scales: [stage][A/B][row], 4 E8M0 bytes (two 64-deep steps x 2 halves)

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, h = lane >> 5;
    int tm, tn;
    tile_of(blockIdx.x, M / GBM, N / GBN, tm, tn);
    const int64_t m0 = (int64_t)tm * GBM, n0 = (int64_t)tn * GBN;

    // global -> register staging: 4 chunks of A and 4 of B per thread; thread
    // t handles chunk q = t + 256 i (row q / 4, 16-byte chunk q % 4)
    const int srow = tid >> 2, sc = tid & 3;
    const uint8_t *ga = A + (m0 + srow) * lda + sc * 16;
    const uint8_t *gb = B + (n0 + srow) * ldb + sc * 16;
    const int64_t a_step = 64 * lda, b_step = 64 * ldb;  // rows advance by 64 per i
    const uint8_t *gsa = FP4 ? SA + (m0 + tid) * lds_a : nullptr;
    const uint8_t *gsb = FP4 ? SB + (n0 + tid) * lds_b : nullptr;

    uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
    uint32_t rsa = 0, rsb = 0;
#define UFP4_GLOAD(kb)                                                              \
    do {                                                                            \
        ra0 = *reinterpret_cast<const uint4 *>(ga + (kb));                          \
        ra1 = *reinterpret_cast<const uint4 *>(ga + a_step + (kb));                 \
        ra2 = *reinterpret_cast<const uint4 *>(ga + 2 * a_step + (kb));             \
        ra3 = *reinterpret_cast<const uint4 *>(ga + 3 * a_step + (kb));             \
        rb0 = *reinterpret_cast<const uint4 *>(gb + (kb));                          \
        rb1 = *reinterpret_cast<const uint4 *>(gb + b_step + (kb));                 \
        rb2 = *reinterpret_cast<const uint4 *>(gb + 2 * b_step + (kb));             \
        rb3 = *reinterpret_cast<const uint4 *>(gb + 3 * b_step + (kb));             \
        if constexpr (FP4) {                                                        \
            rsa = *reinterpret_cast<const uint32_t *>(gsa + ((kb) >> 4));           \
            rsb = *reinterpret_cast<const uint32_t *>(gsb + ((kb) >> 4));           \
        }                                                                           \
    } while (0)
#define UFP4_LSTORE(st)                                                                             \
    do {                                                                                            \
        *reinterpret_cast<uint4 *>(&As[st][lds_off(srow, sc)]) = ra0;                               \
        *reinterpret_cast<uint4 *>(&As[st][lds_off(srow + 64, sc)]) = ra1;                          \
        *reinterpret_cast<uint4 *>(&As[st][lds_off(srow + 128, sc)]) = ra2;                         \
        *reinterpret_cast<uint4 *>(&As[st][lds_off(srow + 192, sc)]) = ra3;                         \
        *reinterpret_cast<uint4 *>(&Bs[st][lds_off(srow, sc)]) = rb0;                               \
        *reinterpret_cast<uint4 *>(&Bs[st][lds_off(srow + 64, sc)]) = rb1;                          \
        *reinterpret_cast<uint4 *>(&Bs[st][lds_off(srow + 128, sc)]) = rb2;                         \
        *reinterpret_cast<uint4 *>(&Bs[st][lds_off(srow + 192, sc)]) = rb3;                         \
        if constexpr (FP4) {                                                                        \
            Ss[st][0][tid] = rsa;                                                                   \
            Ss[st][1][tid] = rsb;                                                                   \
        }                                                                                           \
    } while (0)

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    const int nk = (int)(kbytes / GKB);
    UFP4_GLOAD(0);
    UFP4_LSTORE(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int s = kt & 1;
        if (kt + 1 < nk) UFP4_GLOAD((int64_t)(kt + 1) * GKB);
        // scale words of this wave's rows: byte b holds the E8M0 scale of the
        // stage's 32-element block b; step kk, half h uses block 2 kk + h
        uint32_t wsa[4], wsb[4];
        if constexpr (FP4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wsa[i] = Ss[s][0][wm * 128 + i * 32 + r32] >> (8 * h);
                wsb[i] = Ss[s][1][wn * 128 + i * 32 + r32] >> (8 * h);
            }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            uint4 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ra_ = wm * 128 + i * 32 + r32;
                const int rb_ = wn * 128 + i * 32 + r32;
                fa[i] = *reinterpret_cast<const uint4 *>(&As[s][lds_off(ra_, 2 * kk + h)]);
                fb[i] = *reinterpret_cast<const uint4 *>(&Bs[s][lds_off(rb_, 2 * kk + h)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (FP4) {
                        const v8i a8 = {(int)fa[i].x, (int)fa[i].y, (int)fa[i].z, (int)fa[i].w, 0, 0, 0, 0};
                        const v8i b8 = {(int)fb[j].x, (int)fb[j].y, (int)fb[j].z, (int)fb[j].w, 0, 0, 0, 0};
                        const int sa_ = (int)((wsa[i] >> (16 * kk)) & 0xFFu);
                        const int sb_ = (int)((wsb[j] >> (16 * kk)) & 0xFFu);
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], 4, 4, 0, sa_,
                                                                                     0, sb_);
                    } else {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fa[i]),
                                                                           __builtin_bit_cast(v8bf, fb[j]),
                                                                           acc[i][j], 0, 0, 0);
                    }
                }
        }
        if (kt + 1 < nk) UFP4_LSTORE(s ^ 1);
        __syncthreads();
    }

#undef UFP4_GLOAD
#undef UFP4_LSTORE

    // epilogue: accumulator element e of lane l is C[8(e/4) + 4h + e%4][l%32]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t rbase = m0 + wm * 128 + i * 32 + 4 * h;
            const int64_t col = n0 + wn * 128 + j * 32 + r32;
#pragma unroll
            for (int e = 0; e < 16; ++e) C[(rbase + 8 * (e >> 2) + (e & 3)) * ldc + col] = acc[i][j][e];
        }
}

hipError_t launch_gemm_mxfp4(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb, int64_t M,
                             int64_t N, int64_t K, float *c, int64_t ldc, hipStream_t st)
{
    const dim3 grid((unsigned)((M / GBM) * (N / GBN)));
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(GT), 0, st, a, sa, b, sb, (int)M, (int)N, K / 2, K / 2, K / 2,
                       K / 32, K / 32, c, ldc);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *b, int64_t M, int64_t N, int64_t K, int64_t lda,
                            int64_t ldb, float *c, int64_t ldc, hipStream_t st)
{
    const dim3 grid((unsigned)((M / GBM) * (N / GBN)));
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(GT), 0, st, reinterpret_cast<const uint8_t *>(a), nullptr,
                       reinterpret_cast<const uint8_t *>(b), nullptr, (int)M, (int)N, K * 2, lda * 2, ldb * 2,
                       (int64_t)0, (int64_t)0, c, ldc);
    return hipGetLastError();
}

}  // namespace ufp4
