// gemm.hip -- block-scaled GEMM on CDNA4 matrix cores.
//
// Z = A B^T with both operands K-major.  The MXFP4 path feeds E2M1 codes
// with their UE8M0 block scales straight into the scaled MFMA (FP4 tensors
// with UE8M0 group scales on the native scaled-MFMA path: "FP4 训练 vs FP4
// 推理", UltraQuant; MXFP4 blocks of 32 sharing an E8M0 exponent: MXFP4
// page).  The bf16 path multiplies bf16 operands on the bf16 MFMA (the
// software route for E1M2/INT4 that FP4-only hardware needs: same page, "保留
// FP4 计算，用软件模拟 E1M2 / INT4 路径").  Both accumulate in binary32.
#include "device.hpp"
#include "kernels.hpp"

namespace ufp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// 32x32 output tile per wave; 2 x 2 waves per workgroup (64 x 64).
// Operand fragments: lane l holds row/column (l mod 32) and the K slice
// [32 (l / 32), +32) of a 64-deep MXFP4 step (16 bytes of codes and the
// slice's E8M0 scale), or [8 (l / 32), +8) of a 16-deep bf16 step.
// Accumulator element i of lane l is C[8 (i / 4) + 4 (l / 32) + i mod 4][l mod 32].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_mxfp4_kernel(const uint8_t *__restrict__ a, const uint8_t *__restrict__ sa,
                                                         const uint8_t *__restrict__ b, const uint8_t *__restrict__ sb,
                                                         int64_t K, float *__restrict__ c, int64_t ldc)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
    const int r = lane & 31, h = lane >> 5;
    const uint8_t *ap = a + (m0 + r) * (K >> 1) + h * 16;
    const uint8_t *bp = b + (n0 + r) * (K >> 1) + h * 16;
    const uint8_t *sap = sa + (m0 + r) * (K >> 5) + h;
    const uint8_t *sbp = sb + (n0 + r) * (K >> 5) + h;
    v16f acc = {};
    for (int64_t k = 0; k < K; k += 64) {
        const uint4 av = *reinterpret_cast<const uint4 *>(ap + (k >> 1));
        const uint4 bv = *reinterpret_cast<const uint4 *>(bp + (k >> 1));
        const int s_a = sap[k >> 5];
        const int s_b = sbp[k >> 5];
        v8i A = {(int)av.x, (int)av.y, (int)av.z, (int)av.w, 0, 0, 0, 0};
        v8i B = {(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, 4, 4, 0, s_a, 0, s_b);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t row = m0 + 8 * (i >> 2) + 4 * h + (i & 3);
        c[row * ldc + n0 + r] = acc[i];
    }
}

__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
                                                        int64_t K, int64_t lda, int64_t ldb, float *__restrict__ c,
                                                        int64_t ldc)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
    const int r = lane & 31, h = lane >> 5;
    const uint16_t *ap = a + (m0 + r) * lda + h * 8;
    const uint16_t *bp = b + (n0 + r) * ldb + h * 8;
    v16f acc = {};
    for (int64_t k = 0; k < K; k += 16) {
        const uint4 av = *reinterpret_cast<const uint4 *>(ap + k);
        const uint4 bv = *reinterpret_cast<const uint4 *>(bp + k);
        const v8bf A = __builtin_bit_cast(v8bf, av);
        const v8bf B = __builtin_bit_cast(v8bf, bv);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t row = m0 + 8 * (i >> 2) + 4 * h + (i & 3);
        c[row * ldc + n0 + r] = acc[i];
    }
}

hipError_t launch_gemm_mxfp4(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb, int64_t M,
                             int64_t N, int64_t K, float *c, int64_t ldc, hipStream_t st)
{
    const dim3 grid((unsigned)(N / 64), (unsigned)(M / 64));
    hipLaunchKernelGGL(gemm_mxfp4_kernel, grid, dim3(256), 0, st, a, sa, b, sb, K, c, ldc);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *b, int64_t M, int64_t N, int64_t K, int64_t lda,
                            int64_t ldb, float *c, int64_t ldc, hipStream_t st)
{
    const dim3 grid((unsigned)(N / 64), (unsigned)(M / 64));
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(256), 0, st, a, b, K, lda, ldb, c, ldc);
    return hipGetLastError();
}

}  // namespace ufp4
