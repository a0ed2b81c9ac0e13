// gemm.hip -- block-scaled GEMM on CDNA4 matrix cores.
//
// Z = A B^T with both operands K-major.  The MXFP4 path feeds E2M1 codes
// with their UE8M0 block scales straight into the scaled MFMA (FP4 tensors
// with UE8M0 group scales on the native scaled-MFMA path: "FP4 训练 vs FP4
// 推理", UltraQuant; MXFP4 blocks of 32 sharing an E8M0 exponent: MXFP4
// page).  The bf16 path multiplies bf16 operands on the bf16 MFMA: matrix
// cores with no E1M2/INT4 input take those formats through software, as the
// UFP4 section of the same page describes.  Both accumulate in binary32.
//
// Both paths move operands as bytes: a K-major row supplies 64 bytes per
// pipeline stage (128 E2M1 codes or 32 bf16 values), and one 32x32 MFMA step
// consumes 32 bytes of each of 32 rows, lane l holding row l mod 32 and the
// 16-byte half l / 32 (32 FP4 codes of one 32-element scale block, or 8 bf16).
// Workgroup tile 256 x 256: four waves (one per SIMD) of 128 x 128 (4 x 4
// MFMA tiles of 32 x 32, 256 fp32 accumulators per lane) over a ring of four
// LDS stages (256 rows x 64 bytes per operand plus scales), filled by
// asynchronous global -> LDS copies three stages ahead of the
// multiplications.  The
// 16-byte chunks of each row are XOR-swizzled so the 16-byte fragment reads
// are free of bank conflicts.  The grid is persistent, one workgroup per
// compute unit, each taking its tiles in turn through the same ring; tiles
// are ordered so that the eight XCDs each work on a compact band of them.
#include "device.hpp"
#include "kernels.hpp"

namespace ufp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int GBM = 256;   // workgroup tile rows (M)
constexpr int GBN = 256;   // workgroup tile columns (N)
constexpr int GKB = 64;    // bytes of K per row per stage
constexpr int GROUP_M = 4; // tile-row group of the raster order

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

typedef __attribute__((address_space(3))) void lds_void;

// LDS: a ring of four stage slots, each an A tile (256 rows x 64 B) then a B
// tile, then room for the E8M0 scales of a group of four stages, used in
// slot 0 only (it receives the first stage of every group): 16 bytes per A
// row and per B row, byte 4 j + b scaling block b of the group's stage j.
// They are stored row by row ([row][16 B], one 16-byte copy per row), or
// stage by stage ([j][row][4 B]) where K is not a multiple of four stages.
constexpr int ST_A = 0;
constexpr int ST_B = GBM * GKB;
constexpr int SG_A = 2 * GBM * GKB;         // 32 KiB of operand data
constexpr int SG_B = SG_A + 16 * GBM;
constexpr int ST_BYTES = SG_B + 16 * GBN;   // 40 KiB; four slots fill the 160 KiB of LDS
constexpr int GNS = 4;                      // stage slots

// s_waitcnt with only the vector-memory counter limited to n (n < 64)
#define UFP4_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// s_waitcnt: vector-memory counter at most n and no LDS access outstanding
#define UFP4_WAIT_VM_LDS(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))
// Compiler-level fence: no memory access moves across it, and no wait is
// emitted for it (the waits are explicit).
#define UFP4_CFENCE() asm volatile("" ::: "memory")
#define UFP4_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Wave layout: GWM x GWN waves, each owning TM x TN MFMA tiles of 32 x 32.
constexpr int GWM = 2, GWN = 2;
constexpr int TM = 4, TN = 4;
constexpr int GW = GWM * GWN;      // waves per workgroup, one per SIMD
constexpr int GTH = 64 * GW;
constexpr int ROWS_PER_WAVE = GBM / GW;  // tile rows of A and of B each wave copies
static_assert(GWM * TM * 32 == GBM && GWN * TN * 32 == GBN && GBM == GBN, "tile shape");
static_assert(ROWS_PER_WAVE == 64, "one scale row per lane");

// copies each wave issues: operand data of one stage, scales of one group
constexpr int DATA_COPIES = 2 * (ROWS_PER_WAVE / 16);
constexpr int scale_copies(bool fp4, bool pad) { return fp4 ? (pad ? 8 : 2) : 0; }
// Both paths issue each stage's operand copy in two halves at two points of
// the step (see gemm_step).  That shortens the bf16 step by about a fifth at
// 8192^3; the FP4 step gains fewer cycles and loses part of them to the clock
// (it runs at the board's power limit), 2-3 % net in an A/B in one process.
constexpr bool split_copies(bool) { return true; }

// Asynchronous global -> LDS copy of one stage's operand data, shared by the
// waves: wave w copies tile rows 64 w .. 64 w + 63 of A and of B, 16 rows
// (1 KiB) per instruction; lane l of the instruction for rows R0..R0+15 lands
// at LDS byte R0 * 64 + 16 l, so it fetches the logical chunk (l mod 4) ^ f(row)
// of row R0 + l / 4 and chunk c of row r ends up at lds_off(r, c).  The copies
// are buffer loads: the tile's base sits in the buffer descriptor, the stage's
// K offset in the scalar offset, and each lane's row offset in a vector
// register that stays the same for every stage, so no vector register is
// rewritten while a copy that reads it is in flight.
struct CopyOffsets {
    uint32_t a[ROWS_PER_WAVE / 16], b[ROWS_PER_WAVE / 16];  // operand data
    uint32_t sa, sb;                                        // scale rows
};

__device__ __forceinline__ CopyOffsets copy_offsets(int64_t lda, int64_t ldb, int64_t lds_a, int64_t lds_b, int wave,
                                                    int lane)
{
    CopyOffsets o;
#pragma unroll
    for (int i = 0; i < ROWS_PER_WAVE / 16; ++i) {
        const int row = ROWS_PER_WAVE * wave + 16 * i + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 2) & 3);
        o.a[i] = (uint32_t)(row * lda + 16 * c);
        o.b[i] = (uint32_t)(row * ldb + 16 * c);
    }
    const int srow = ROWS_PER_WAVE * wave + lane;
    o.sa = (uint32_t)(srow * lds_a);
    o.sb = (uint32_t)(srow * lds_b);
    return o;
}

// raw buffer over a tile's rows: base address, no stride, no range limit
// (every offset the kernel forms is inside the operand)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_buffer(const uint8_t *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, -1, 0x00020000);
}

// Buffer descriptors of one output tile: its A rows, B rows and (FP4) their
// scale rows.
struct TileBufs {
    __amdgpu_buffer_rsrc_t a, b, sa, sb;
};

template <bool FP4>
__device__ __forceinline__ TileBufs tile_bufs(const uint8_t *A, const uint8_t *B, const uint8_t *SA,
                                              const uint8_t *SB, int64_t lda, int64_t ldb, int64_t lds_a,
                                              int64_t lds_b, int64_t m0, int64_t n0)
{
    return TileBufs{tile_buffer(A + m0 * lda), tile_buffer(B + n0 * ldb), tile_buffer(FP4 ? SA + m0 * lds_a : A),
                    tile_buffer(FP4 ? SB + n0 * lds_b : B)};
}

// One stage's copies into slot st; with SCALES, also the scales of stages
// s0 .. s0 + 3 (each clamped to the last stage) into the slot's scale area:
// wave w copies the 16 bytes of rows 64 w .. 64 w + 63, one row per lane, of
// A's and B's scale rows; stage by stage (4 bytes a row) where K is not a
// multiple of four stages.  PART 0 and 1 copy only the first or the second
// half of each wave's operand rows (and PART 1 no scales); PART 2 copies
// everything.  (All copies of a call go through one restrict
// pointer: the compiler tells LDS copies apart by the alias scopes of their
// destinations and tracks only a few such scopes.)
template <bool SCALES, bool PAD, int PART = 2>
__device__ __forceinline__ void copy_stage(uint8_t *__restrict__ st, __amdgpu_buffer_rsrc_t At,
                                           __amdgpu_buffer_rsrc_t Bt, __amdgpu_buffer_rsrc_t SAt,
                                           __amdgpu_buffer_rsrc_t SBt, const CopyOffsets &o, int kb, int s0, int nk,
                                           int wave)
{
#pragma unroll
    for (int i = (PART == 1 ? ROWS_PER_WAVE / 32 : 0); i < (PART == 0 ? ROWS_PER_WAVE / 32 : ROWS_PER_WAVE / 16);
         ++i) {
        const int R0 = ROWS_PER_WAVE * wave + 16 * i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(At, (lds_void *)(st + ST_A + R0 * GKB), 16, o.a[i], kb, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(Bt, (lds_void *)(st + ST_B + R0 * GKB), 16, o.b[i], kb, 0, 0);
    }
    if constexpr (SCALES && !PAD && PART != 1) {
        const int s = min(s0, nk - 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(SAt, (lds_void *)(st + SG_A + 16 * ROWS_PER_WAVE * wave), 16, o.sa,
                                                 4 * s, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(SBt, (lds_void *)(st + SG_B + 16 * ROWS_PER_WAVE * wave), 16, o.sb,
                                                 4 * s, 0, 0);
    } else if constexpr (SCALES && PART != 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = min(s0 + j, nk - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                SAt, (lds_void *)(st + SG_A + 4 * GBM * j + 4 * ROWS_PER_WAVE * wave), 4, o.sa, 4 * s, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                SBt, (lds_void *)(st + SG_B + 4 * GBN * j + 4 * ROWS_PER_WAVE * wave), 4, o.sb, 4 * s, 0, 0);
        }
    }
}

// Operand fragments of one 32-element K step (kk = 0 or 1 of a stage): lane
// (r32, h) holds the 16-byte chunk 2 kk + h of its row in each of the wave's
// A and B tiles.
struct Frags {
    uint4 a[TM], b[TN];
};

__device__ __forceinline__ void read_frags(Frags &f, const uint8_t *__restrict__ st, int kk, int wm, int wn, int r32,
                                           int h)
{
#pragma unroll
    for (int i = 0; i < TM; ++i)
        f.a[i] = *reinterpret_cast<const uint4 *>(st + ST_A + lds_off((wm * TM + i) * 32 + r32, 2 * kk + h));
#pragma unroll
    for (int j = 0; j < TN; ++j)
        f.b[j] = *reinterpret_cast<const uint4 *>(st + ST_B + lds_off((wn * TN + j) * 32 + r32, 2 * kk + h));
}

// keep (m = ~0) or zero (m = 0) the A fragments: a product with zero A adds
// exact zeros
__device__ __forceinline__ void mask_frags(Frags &f, uint32_t m)
{
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        f.a[i].x &= m;
        f.a[i].y &= m;
        f.a[i].z &= m;
        f.a[i].w &= m;
    }
}

// Scale words of a group for the lane's rows, word j for the group's stage j,
// shifted right by 8 h: the MFMA of step kk then takes byte 2 kk of it (block
// 2 kk + h of the stage), chosen by the scale operand's byte select.
struct ScaleGroup {
    uint4 a[TM], b[TN];
};

__device__ __forceinline__ uint4 shr4(uint4 v, int sh) { return uint4{v.x >> sh, v.y >> sh, v.z >> sh, v.w >> sh}; }

template <bool PAD>
__device__ __forceinline__ void read_scales(ScaleGroup &g, const uint8_t *__restrict__ sg, int wm, int wn, int r32,
                                            int h)
{
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = (wm * TM + i) * 32 + r32;
        if constexpr (!PAD) {
            g.a[i] = *reinterpret_cast<const uint4 *>(sg + SG_A + 16 * row);
        } else {
            const uint32_t *p = reinterpret_cast<const uint32_t *>(sg + SG_A) + row;
            g.a[i] = uint4{p[0], p[GBM], p[2 * GBM], p[3 * GBM]};
        }
        g.a[i] = shr4(g.a[i], 8 * h);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int row = (wn * TN + j) * 32 + r32;
        if constexpr (!PAD) {
            g.b[j] = *reinterpret_cast<const uint4 *>(sg + SG_B + 16 * row);
        } else {
            const uint32_t *p = reinterpret_cast<const uint32_t *>(sg + SG_B) + row;
            g.b[j] = uint4{p[0], p[GBN], p[2 * GBN], p[3 * GBN]};
        }
        g.b[j] = shr4(g.b[j], 8 * h);
    }
}

__device__ __forceinline__ int word_of(const uint4 &v, int j)
{
    return (int)(j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w);
}

// the MFMAs of K step KK of the group's stage j
template <bool FP4, int KK>
__device__ __forceinline__ void mfma_step(v16f (&acc)[TM][TN], const Frags &f, const ScaleGroup &g, int j)
{
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int n = 0; n < TN; ++n) {
            if constexpr (FP4) {
                const v8i a8 = {(int)f.a[i].x, (int)f.a[i].y, (int)f.a[i].z, (int)f.a[i].w, 0, 0, 0, 0};
                const v8i b8 = {(int)f.b[n].x, (int)f.b[n].y, (int)f.b[n].z, (int)f.b[n].w, 0, 0, 0, 0};
                acc[i][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][n], 4, 4, 2 * KK,
                                                                             word_of(g.a[i], j), 2 * KK,
                                                                             word_of(g.b[n], j));
            } else {
                acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, f.a[i]),
                                                                   __builtin_bit_cast(v8bf, f.b[n]), acc[i][n], 0, 0,
                                                                   0);
            }
        }
}

// The main loop over a ring of four LDS stages.  Step k multiplies stage k in
// two K steps.  The first runs on fragments read during the previous step
// while the second's fragments are read; between the two, the wave waits for
// those reads and for its own copies of stage k + 1, and meets the other
// waves at the barrier: stage k + 1 is then complete in LDS and no wave reads
// stage k any more, so its slot takes the copy of stage k + 4 (three steps of
// copy latency hidden) while stage k + 1's first fragments are read under the
// second K step.  Slot 0 receives the first stage of each group of four, and
// with it the group's scales, which the wave reads into registers one step
// ahead of the group.  Every step has the same shape: past the last stage
// the copy fetches the next tile's first stages (on a workgroup's last tile
// it re-reads the last stage into the free slot, and the reads of "stage
// k + 1" go unused); the steps that round the count up to a multiple of
// four multiply zeroed fragments.  So the body has no branches around
// matrix work and the scheduling barriers hold the order within it.  Restrict
// slot pointers tell the compiler which slot each access touches, so the
// copies into the other slots stay in flight.  The copies are split: the
// barrier's copy takes the first half of each wave's rows of stage k + 4
// (with the group's scales at position 0), and the second half follows at the start of the next step,
// into the same slot (pv there): every wave has passed the barrier behind
// its last read of that slot, and the copies in flight at each wait are
// still the four halves of stages k + 2 and k + 3.
template <bool FP4, bool PAD>
__device__ __forceinline__ void gemm_step(v16f (&acc)[TM][TN], Frags &f0, Frags &f1, ScaleGroup &g,
                                          uint8_t *__restrict__ cur, const uint8_t *__restrict__ nx,
                                          uint8_t *__restrict__ pv, const TileBufs &tc, const TileBufs &tn,
                                          const CopyOffsets &o, int k, int nk, int nk4, int j, int wave, int wm,
                                          int wn, int r32, int h)
{
    // j = k mod 4, a constant at each call (one function for the four
    // positions: the compiler then keeps the slots' alias scopes apart)
    constexpr int SC = scale_copies(FP4, PAD);
    constexpr int CP = split_copies(FP4) ? 0 : 2;
    // ring stage s is this tile's stage s (clamped to its last) below nk4 and
    // the next tile's stage s - nk4 from there (wave-uniform choices)
    const bool n3 = k + 3 >= nk4, n4 = k + 4 >= nk4;
    const int s3 = n3 ? k + 3 - nk4 : k + 3, s4 = n4 ? k + 4 - nk4 : k + 4;
    const TileBufs b3 = n3 ? tn : tc, b4 = n4 ? tn : tc;
    if constexpr (split_copies(FP4))
        copy_stage<false, PAD, 1>(pv, b3.a, b3.b, b3.sa, b3.sb, o, min(s3, nk - 1) * GKB, 0, nk, wave);
    read_frags(f1, cur, 1, wm, wn, r32, h);
    if constexpr (PAD) mask_frags(f1, k < nk ? ~0u : 0u);  // a step past the end adds exact zeros
    mfma_step<FP4, 0>(acc, f0, g, j);
    // the second K step's fragment reads go out first, under these MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
    UFP4_SCHED_FENCE();
    // the copies issued at the two previous steps (stages k + 2, k + 3) may
    // still be in flight; the group's scales went with the copy at position 0
    if (j == 1 || j == 2)
        UFP4_WAIT_VM_LDS(2 * DATA_COPIES + SC);
    else
        UFP4_WAIT_VM_LDS(2 * DATA_COPIES);
    UFP4_CFENCE();
    __builtin_amdgcn_s_barrier();
    UFP4_CFENCE();
    UFP4_SCHED_FENCE();
    if (FP4 && j == 0)
        copy_stage<true, PAD, CP>(cur, b4.a, b4.b, b4.sa, b4.sb, o, min(s4, nk - 1) * GKB, s4, nk, wave);
    else
        copy_stage<false, PAD, CP>(cur, b4.a, b4.b, b4.sa, b4.sb, o, min(s4, nk - 1) * GKB, 0, nk, wave);
    read_frags(f0, nx, 0, wm, wn, r32, h);
    ScaleGroup gn;
    if (FP4 && j == 3) read_scales<PAD>(gn, nx, wm, wn, r32, h);
    if constexpr (PAD) mask_frags(f0, k + 1 < nk || k + 1 >= nk4 ? ~0u : 0u);
    mfma_step<FP4, 1>(acc, f1, g, j);
    UFP4_SCHED_FENCE();
    if (FP4 && j == 3) g = gn;
}

// The output tiles of a workgroup, one after another through one ring: the
// copies that would re-read a tile's last stage past its end (steps nk4 - 4
// .. nk4 - 1, nk4 = nk rounded up to whole groups of four) fetch the next
// tile's stages 0 .. 3 into the slots that tile's steps use, so only the
// first tile waits for a prologue, and the fragments and scales read at a
// tile's last step are the next tile's first.
template <bool FP4, bool PAD>
__device__ __forceinline__ void gemm_tiles(uint8_t *__restrict__ P0, uint8_t *__restrict__ P1,
                                           uint8_t *__restrict__ P2, uint8_t *__restrict__ P3, const uint8_t *A,
                                           const uint8_t *B, const uint8_t *SA, const uint8_t *SB, int MT, int NT,
                                           int64_t lda, int64_t ldb, int64_t lds_a, int64_t lds_b, int nk,
                                           float *__restrict__ C, int64_t ldc, int wave, int lane, int wm, int wn,
                                           int r32, int h)
{
    const int T = MT * NT, G = (int)gridDim.x;
    const int nk4 = (nk + 3) & ~3;
    const CopyOffsets o = copy_offsets(lda, ldb, lds_a, lds_b, wave, lane);
    int t = (int)blockIdx.x, tm, tn;
    tile_of(t, MT, NT, tm, tn);
    TileBufs tc = tile_bufs<FP4>(A, B, SA, SB, lda, ldb, lds_a, lds_b, (int64_t)tm * GBM, (int64_t)tn * GBN);

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};
    Frags f0, f1;
    ScaleGroup g{};
    if (nk > 0) {
        // prologue of the first tile: stages 0 .. 3 (the last stage again
        // where there are fewer) and the scales of the first group
        copy_stage<FP4, PAD>(P0, tc.a, tc.b, tc.sa, tc.sb, o, 0, 0, nk, wave);
        copy_stage<false, PAD>(P1, tc.a, tc.b, tc.sa, tc.sb, o, min(1, nk - 1) * GKB, 0, nk, wave);
        copy_stage<false, PAD>(P2, tc.a, tc.b, tc.sa, tc.sb, o, min(2, nk - 1) * GKB, 0, nk, wave);
        if constexpr (split_copies(FP4)) {
            // stage 3's second half goes out at the start of step 0
            copy_stage<false, PAD, 0>(P3, tc.a, tc.b, tc.sa, tc.sb, o, min(3, nk - 1) * GKB, 0, nk, wave);
            UFP4_WAIT_VM(2 * DATA_COPIES + DATA_COPIES / 2);
        } else {
            copy_stage<false, PAD>(P3, tc.a, tc.b, tc.sa, tc.sb, o, min(3, nk - 1) * GKB, 0, nk, wave);
            UFP4_WAIT_VM(3 * DATA_COPIES);
        }
        UFP4_CFENCE();
        __builtin_amdgcn_s_barrier();
        UFP4_CFENCE();
        read_frags(f0, P0, 0, wm, wn, r32, h);
        if constexpr (FP4) read_scales<PAD>(g, P0, wm, wn, r32, h);
    }
    for (;;) {
        const int64_t m0 = (int64_t)tm * GBM, n0 = (int64_t)tn * GBN;
        const bool more = t + G < T;
        int tm2 = tm, tn2 = tn;
        if (more) tile_of(t + G, MT, NT, tm2, tn2);
        // the last tile's steps past its end re-read its own stages
        const TileBufs tx = more ? tile_bufs<FP4>(A, B, SA, SB, lda, ldb, lds_a, lds_b, (int64_t)tm2 * GBM,
                                                  (int64_t)tn2 * GBN)
                                 : tc;
#define UFP4_STEP(J, CUR, NX, PV) \
    gemm_step<FP4, PAD>(acc, f0, f1, g, CUR, NX, PV, tc, tx, o, kt + (J), nk, nk4, J, wave, wm, wn, r32, h)
        // whole groups of four steps; the steps past the end multiply zeros
        for (int kt = 0; kt < nk; kt += 4) {
            UFP4_STEP(0, P0, P1, P3);
            UFP4_STEP(1, P1, P2, P0);
            UFP4_STEP(2, P2, P3, P1);
            UFP4_STEP(3, P3, P0, P2);
        }
#undef UFP4_STEP
        // epilogue: accumulator element e of lane l is C[8(e/4) + 4h + e%4][l%32].
        // The output is written once and not read back here, so its stores
        // are non-temporal: they do not displace operand lines that the
        // workgroups still running read from L2 (the bf16 GEMM gains 2-3 % at
        // 8192^3).
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t rbase = m0 + (wm * TM + i) * 32 + 4 * h;
                const int64_t col = n0 + (wn * TN + j) * 32 + r32;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    __builtin_nontemporal_store(acc[i][j][e], &C[(rbase + 8 * (e >> 2) + (e & 3)) * ldc + col]);
                acc[i][j] = v16f{};
            }
        if (!more) break;
        t += G;
        tm = tm2;
        tn = tn2;
        tc = tx;
    }
    // no copy may still be writing LDS when the workgroup ends
    UFP4_WAIT_VM(0);
}

// Persistent grid: workgroup w computes output tiles w, w + G, w + 2G, ...
// (G = the grid size, at most one workgroup per compute unit; a multiple of
// 8 keeps each workgroup's tiles in its XCD's band).
template <bool FP4, bool PAD>
__global__ __launch_bounds__(GTH, 1) void gemm_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA,
                                                      const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB,
                                                      int M, int N, int64_t kbytes, int64_t lda, int64_t ldb,
                                                      int64_t lds_a, int64_t lds_b, float *__restrict__ C, int64_t ldc)
{
    __shared__ __attribute__((aligned(16))) uint8_t ring[GNS][ST_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / GWN, wn = wave % GWN;
    const int r32 = lane & 31, h = lane >> 5;
    gemm_tiles<FP4, PAD>(ring[0], ring[1], ring[2], ring[3], A, B, SA, SB, M / GBM, N / GBN, lda, ldb, lds_a, lds_b,
                         (int)(kbytes / GKB), C, ldc, wave, lane, wm, wn, r32, h);
}
#undef UFP4_WAIT_VM
#undef UFP4_WAIT_VM_LDS
#undef UFP4_CFENCE
#undef UFP4_SCHED_FENCE

// Workgroups of the persistent grid: one per compute unit of the current
// device (the kernel's LDS ring fills a CU), at most one per tile.
static unsigned gemm_grid(int64_t tiles)
{
    const int n = cu_count();
    return (unsigned)(tiles < n ? tiles : n);
}

hipError_t launch_gemm_mxfp4(const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb, int64_t M,
                             int64_t N, int64_t K, float *c, int64_t ldc, hipStream_t st)
{
    const dim3 grid(gemm_grid((M / GBM) * (N / GBN)));
    const int64_t nk = K / 2 / GKB;
    // whole groups of four stages with 16-byte aligned scale rows take the
    // 16-byte scale copies; any other K the per-stage ones
    const bool pad = (nk % 4) != 0 || ((uintptr_t)sa | (uintptr_t)sb | (uint64_t)(K / 32)) % 16 != 0;
    if (pad)
        launch_kernel((gemm_kernel<true, true>), grid, dim3(GTH), st, a, sa, b, sb, (int)M, (int)N, K / 2,
                           K / 2, K / 2, K / 32, K / 32, c, ldc);
    else
        launch_kernel((gemm_kernel<true, false>), grid, dim3(GTH), st, a, sa, b, sb, (int)M, (int)N, K / 2,
                           K / 2, K / 2, K / 32, K / 32, c, ldc);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *b, int64_t M, int64_t N, int64_t K, int64_t lda,
                            int64_t ldb, float *c, int64_t ldc, hipStream_t st)
{
    const dim3 grid(gemm_grid((M / GBM) * (N / GBN)));
    const uint8_t *a8 = reinterpret_cast<const uint8_t *>(a), *b8 = reinterpret_cast<const uint8_t *>(b);
    if (((K * 2 / GKB) % 4) != 0)
        launch_kernel((gemm_kernel<false, true>), grid, dim3(GTH), st, a8, nullptr, b8, nullptr, (int)M,
                           (int)N, K * 2, lda * 2, ldb * 2, (int64_t)0, (int64_t)0, c, ldc);
    else
        launch_kernel((gemm_kernel<false, false>), grid, dim3(GTH), st, a8, nullptr, b8, nullptr, (int)M,
                           (int)N, K * 2, lda * 2, ldb * 2, (int64_t)0, (int64_t)0, c, ldc);
    return hipGetLastError();
}

}  // namespace ufp4
