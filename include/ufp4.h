/*
 * ufp4.h -- C ABI of libufp4, a 4-bit block quantizer and block-scaled GEMM
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes follows these pages:
 *   [UFP4-ZC] "当你的 GPU 学不会算账：FP4 训练里那个被忽视了 30 年的几何陷阱"
 *             (zhichai.net): the E2M1 and E1M2 grids (sections "E2M1：一块刻度
 *             不均的尺子", "UFP4：换一把尺子"), the UFP4 recipe table (RHT on
 *             fwd_y/bwd_dx/bwd_dw, stochastic rounding on dY, 1x16 blocks,
 *             single FP32 scale), the attenuation identity Z_q = a_A a_B Z + noise
 *             (section "复利效应的反向版本").
 *   [UFP4-TW] "蚂蚁集团揭秘：为什么给AI'降精度省电'会悄悄让它越来越笨？"
 *             (techwalker.com): RTNE rounding (section 二), RHT (section 四),
 *             the recipe (section 五), fused 16-wide RHT + quantize (section 六).
 *   [MXFP4]   "AMD全新研究揭示：FP4训练不稳定性源于结构误差而非随机性不足"
 *             (cannews.ca): MXFP4 = 32-element blocks sharing an E8M0 exponent;
 *             deterministic Hadamard H16.
 *   [IF4]     "低精度量化技术：IF4自适应数据类型的原理与应用" (bxzpzcl.cn):
 *             block scaling (2.1), the format table (2.2), IF4's type flag in
 *             the E4M3 scale's sign bit with 7/6 and 6/7 INT4 scaling (3.1.1),
 *             the two-level scale alpha = max|X|/(6x448),
 *             Delta = max|X_block|/(alpha x 6) (3.2), stochastic rounding (6.1).
 *   [UQ]      "FP4 训练 vs FP4 推理" (reports.10n1j.top): FP4 tensors with UE8M0
 *             group scales on CDNA4's native scaled-MFMA path; UltraQuant's
 *             FP8-query x FP4-KV decode attention (asymmetric K/V,
 *             Walsh-Hadamard rotation).
 *
 * Conventions shared by every call
 *   - Device pointers are HIP device memory owned by the caller; the library
 *     allocates nothing, keeps no pointer after a call returns and has no
 *     global state except, per host thread, the last HIP error and a pending
 *     ufp4_time_next_launch request, and, per process, each device's
 *     compute-unit count (read once by the first GEMM or statistics call on
 *     that device, never changed after), the resident workgroups per compute
 *     unit of each statistics kernel (one occupancy query per kernel, the first
 *     time it runs) and the device address of ufp4_amax_noalloc's built-in
 *     scratch array (looked up once per device).  Calls are reentrant and
 *     can be captured in a HIP graph (no allocation, no memset); calls of
 *     ufp4_amax_noalloc that overlap on one device share its scratch.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; results are ordered by the stream.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     validation error nothing is written and a negative code is returned.
 *   - Inputs must be finite.  Outputs for NaN/Inf inputs are unspecified.
 *   - Element types: UFP4_BF16 (bfloat16) or UFP4_F32 (binary32).
 *
 * Quantization view
 *   A quantization runs along rows (UFP4_ROW) or down columns (UFP4_COL) of a
 *   row-major source x[rows][ldx].  Its "view" has V rows of L elements and the
 *   blocks run along view rows:
 *     UFP4_ROW: V = rows, L = cols, view(v, l) = x[v][l]
 *     UFP4_COL: V = cols, L = rows, view(v, l) = x[l][v]   (the transpose)
 *   so a column quantization of x is bit-identical to the row quantization of
 *   x^T.  Each GEMM operand is quantized along its contraction axis.
 *   Stored layout (row-major, contiguous):
 *     codes  uint8[V][L/2]: byte j holds elements 2j (low nibble) and 2j+1
 *            (high nibble); a nibble is sign<<3 | magnitude code k (0..7)
 *     scales float[V][L/16] (UFP4_SCALE_FP32), uint8[V][L/16] (UFP4_SCALE_E4M3,
 *            E4M3FN byte; for IF4 bit 7 is the type flag, 1 = INT4), or
 *            uint8[V][L/32] (UFP4_SCALE_E8M0, biased exponent, value 2^(b-127))
 *     tensor_scale float[1]: alpha of the two-level scale (E4M3 only)
 *   Magnitude codes: E2M1 k -> {0,.5,1,1.5,2,3,4,6}; E1M2 k -> k/2; INT4 k -> k.
 *
 * Arithmetic (identical to the CPU oracle, bit for bit)
 *   binary32 with round-to-nearest-even, no contraction, denormals kept.
 *   y    = RHT(x): per 16-element chunk of a view row, v = d (.) x, a 16-point
 *          Walsh-Hadamard butterfly with spans 1,2,4,8 in that order, then x 1/4.
 *          d_i = -1 iff bit i of Philox4x32-10 word 0 at key = rht_seed,
 *          counter = (0, 0, 0x52485400, 0); d = +1 for UFP4_RHT_DETERMINISTIC.
 *   m    = max |y| over the block.
 *   FP32 scale: s = m / gridmax (gridmax 6, 3.5, 7 for E2M1, E1M2, INT4).
 *   E4M3 scale: alpha = A / (gridmax x 448), A = max |y| over the tensor;
 *          Delta = m / (alpha x gridmax) rounded to E4M3FN (nearest, ties to
 *          even, saturating at 448); s = alpha x Delta_q.
 *   E8M0 scale: s = 2^E, E = floor(log2 m) - 2 clamped to [-127, 127]
 *          (m = 0 gives E = -127).
 *   z    = y / s (correctly rounded); s = 0 gives code 0.
 *   RTNE: nearest grid point, ties to the even code, saturating at gridmax.
 *   SR:   k = k_lo + 1 when h + floor(frac 2^16) >= 2^16, else k_lo (frac =
 *          position of |z| in its cell; 16 random bits h per element): h is
 *          half n mod 2 (low half first) of Philox4x32-10 word (n/2) mod 4 at
 *          key = sr_seed, counter = (lo32(n/8), hi32(n/8), sr_stream, 0),
 *          n = v L + l the element's index in the view.
 *   IF4:  z = y/s; FP4 candidate = RTNE of z on E2M1 (grid value g); INT4
 *          candidate k = rint(z x 7/6) clamped to 7, dequantized as (k x s) x 6/7;
 *          errors in units of s, g - z and k x 6/7 - z (one fused multiply-add);
 *          the candidate with the smaller binary32 sum of squared errors (each
 *          square fused into the running sum, in element order) wins, ties to FP4.
 *   Dequantization: x_hat = v x s (IF4 INT4 blocks: (k x s) x 6/7).
 */
#ifndef UFP4_H
#define UFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ------------------------------------------------------- */
#define UFP4_OK 0
#define UFP4_ERR_INVALID_ARG (-1) /* null pointer, unknown enum value, bad dtype     */
#define UFP4_ERR_SHAPE (-2)       /* sizes not multiples of the block / tile rules  */
#define UFP4_ERR_ALIGN (-3)       /* pointer not 16-byte aligned, ld not multiple of 8 */
#define UFP4_ERR_UNSUPPORTED (-4) /* combination of options the library does not run */
#define UFP4_ERR_WORKSPACE (-5)   /* workspace missing or smaller than required      */
#define UFP4_ERR_HIP (-6)         /* a HIP launch failed; see ufp4_last_hip_error()  */

/* ---- enumerations ------------------------------------------------------ */
/* Formats.  UFP4_E2M1_MAX4/3/2: E2M1 codes with the range capped at 4, 3 or
 * 2 (the grid's points up to the cap, saturating there; at 2 the points are
 * uniform): [UFP4-ZC] "UFP4：换一把尺子", the attempt to emulate a uniform grid
 * on E2M1.  FP32 or E4M3 block scales (gridmax = the cap), RTNE only. */
enum { UFP4_E2M1 = 0, UFP4_E1M2 = 1, UFP4_INT4 = 2, UFP4_IF4 = 3, UFP4_E2M1_MAX4 = 4, UFP4_E2M1_MAX3 = 5,
       UFP4_E2M1_MAX2 = 6 };
enum { UFP4_SCALE_FP32 = 0, UFP4_SCALE_E4M3 = 1, UFP4_SCALE_E8M0 = 2 };
enum { UFP4_RHT_NONE = 0, UFP4_RHT_RANDOM = 1, UFP4_RHT_DETERMINISTIC = 2 };
enum { UFP4_RTNE = 0, UFP4_SR = 1 };
enum { UFP4_ROW = 0, UFP4_COL = 1 };
enum { UFP4_BF16 = 0, UFP4_F32 = 1 };
enum { UFP4_GEMM_NATIVE_MXFP4 = 0, UFP4_GEMM_DEQUANT_BF16 = 1 };
enum { UFP4_OP_STATS = 0, UFP4_OP_QGEMM = 1, UFP4_OP_ETA = 2, UFP4_OP_AMAX = 3 };
enum { UFP4_KV_FP4 = 0, UFP4_KV_FP8 = 1 }; /* KV-cache element format (see the KV section) */

/* Supported combinations (anything else returns UFP4_ERR_UNSUPPORTED):
 *   E2M1 with FP32/16, E4M3/16 or E8M0/32; E1M2 and INT4 with FP32/16 or E4M3/16;
 *   IF4 with E4M3/16 only.  SR with E2M1, E1M2, INT4 under FP32 or E4M3 scales.
 *   The RHT is 16 wide; a 32-element block holds two transformed chunks. */
typedef struct ufp4_config {
    int32_t format;     /* UFP4_E2M1 / E1M2 / INT4 / IF4 / E2M1_MAX4 / MAX3 / MAX2 */
    int32_t scale;      /* UFP4_SCALE_*                                        */
    int32_t block;      /* 16 (FP32, E4M3) or 32 (E8M0)                        */
    int32_t rht;        /* UFP4_RHT_*                                          */
    int32_t rounding;   /* UFP4_RTNE / UFP4_SR                                 */
    int32_t axis;       /* UFP4_ROW / UFP4_COL                                 */
    uint64_t rht_seed;  /* key of the sign diagonal                            */
    uint64_t sr_seed;   /* key of the stochastic-rounding stream               */
    uint32_t sr_stream; /* third Philox counter word (0 row, 1 column by convention) */
    uint32_t reserved;  /* must be 0                                           */
} ufp4_config;

/* A quantized tensor.  rows/cols are the LOGICAL SOURCE shape; buffers hold
 * the view layout described above.  All pointers are device memory owned by
 * the caller. */
typedef struct ufp4_qtensor {
    uint8_t *codes;
    void *scales;
    float *tensor_scale; /* required for UFP4_SCALE_E4M3, ignored otherwise */
    int64_t rows;
    int64_t cols;
    ufp4_config cfg;
} ufp4_qtensor;

/* Statistics report ([UFP4-ZC] SQNR and signal factor; [UFP4-TW] 二 per-cell
 * bias; [IF4] 6.2 FP4/INT4 shares).  Filled on the host from the sums. */
typedef struct ufp4_stats_report {
    double n;             /* elements                                          */
    double sqnr_db;       /* 10 log10(sum y^2 / sum (x_hat - y)^2)                */
    double alpha;         /* sum x_hat y / sum y^2 (signal factor)                */
    double mse;           /* sum (x_hat - y)^2 / n                                */
    double mean_err;      /* sum (x_hat - y) / n                                  */
    double mean_shrink;   /* sum sign(y)(x_hat - y) / n (< 0: shrinkage)          */
    double int4_share;    /* IF4: INT4 blocks / blocks                            */
    double counts[2][8];  /* [type][k]: magnitude-code counts (type 1 = IF4 INT4)  */
    double bucket_bias[2][8]; /* mean (g[k] - |z|) per code, grid units (NaN if empty) */
} ufp4_stats_report;

#define UFP4_NSUMS 48
/* Layout of the 48 binary64 sums written by ufp4_stats:
 *  [0] n  [1] sum y^2  [2] sum e^2  [3] sum e  [4] sum sign(y) e  [5] sum x_hat y
 *  [6] sum |e|  [7] blocks  [8] INT4 blocks
 *  [16 + 8t + k] count of code k in blocks of type t; [32 + 8t + k] sum (g_t[k] - |z|)
 *  with e = x_hat - y (binary64 of binary32 values). */

/* ---- calls --------------------------------------------------------------- */

/* Standalone 16-wide RHT ([UFP4-TW] 六: the unfused variant, transform then
 * quantize).  Writes y = view of RHT(x) as y[V][ldy] in y_dtype (UFP4_F32 keeps
 * every bit; UFP4_BF16 rounds to nearest even).  Sizes: L multiple of 16;
 * x, y 16-byte aligned; ldx, ldy multiples of 8 (element counts); for UFP4_COL
 * also cols multiple of 8.  rht_kind UFP4_RHT_NONE copies (and converts). */
int ufp4_rht(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int axis, int rht_kind,
             uint64_t rht_seed, void *y, int y_dtype, int64_t ldy, void *stream);

/* Tensor amax after the transform named by cfg (rht, rht_seed, axis): writes
 * max |y| to amax[0] (device float).  Needed before a UFP4_SCALE_E4M3
 * quantization ([IF4] 3.2: alpha = max|X| / (6 x 448)).  Two launches: one
 * partial maximum per workgroup into ws, then one workgroup reduces them (no
 * atomics; the result is exact and order-free).  ws: device workspace of
 * ufp4_workspace_size(UFP4_OP_AMAX, rows, cols, cfg) bytes.  Several devices
 * can combine their amax with a MAX all-reduce before quantizing their shards. */
int ufp4_amax(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, const ufp4_config *cfg,
              float *amax, void *ws, size_t ws_bytes, void *stream);

/* ufp4_amax without a workspace argument, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation.  The partial maxima go to a scratch array
 * built into the library: 256 KiB of device memory on each device the library
 * runs on, held until the process ends; its address is looked up once per
 * device on the first call there.  The call allocates nothing.  Sizes: the
 * pass may need at most 65536 partial maxima, i.e. rows x cols up to 2^30
 * along rows, or ceil(cols/64) x ceil(rows/512) <= 65536 down columns;
 * larger tensors return UFP4_ERR_WORKSPACE before anything is enqueued.
 * Every call on one device shares that device's scratch: calls that may
 * overlap on one device (other streams, other host threads) race and must
 * be ordered by the caller.  Otherwise as ufp4_amax (same result, bit for
 * bit). */
int ufp4_amax_noalloc(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, const ufp4_config *cfg,
                      float *amax, void *stream);

/* Block quantization (all steps fused in one kernel: load, signs, FWHT, block
 * amax, scale, RTNE/SR or IF4 selection, nibble packing, stores).
 * Definitions: the fused 16-wide RHT + quantize of [UFP4-TW] 六; the per-block
 * scale of [UFP4-ZC]'s recipe table (single FP32 scale per 1x16 block), of
 * [IF4] 3.2 (E4M3 block scale under the FP32 tensor scale alpha) or of [MXFP4]
 * (E8M0 per 32); rounding to the grids of [UFP4-ZC] "E2M1：一块刻度不均的尺子"
 * and "UFP4：换一把尺子" by RTNE ([UFP4-TW] 二) or stochastic rounding
 * ([IF4] 6.1; [UFP4-TW] 五: dY only); IF4's per-block choice ([IF4] 3.1.1).
 * out->codes, out->scales (and out->tensor_scale for E4M3) must point to
 * buffers of the sizes above; out->rows/cols/cfg are filled in by the call.
 * amax: device float from ufp4_amax (required for E4M3, ignored otherwise).
 * Shapes: L multiple of the block; UFP4_COL also needs cols multiple of 8;
 * x 16-byte aligned, ldx multiple of 8 and >= cols. */
int ufp4_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, const ufp4_config *cfg,
                  const float *amax, ufp4_qtensor *out, void *stream);

/* Dequantization ([IF4] 3.1.1: code x scale, x 6/7 for INT4 blocks) of the
 * view: y[V][ldy] in y_dtype.  inverse_rht != 0 undoes the transform (FWHT x
 * 1/4, then the signs), giving the source orientation of each view row. */
int ufp4_dequantize(const ufp4_qtensor *q, int inverse_rht, void *y, int y_dtype, int64_t ldy, void *stream);

/* Quantization statistics of q against the source x it was made from (same
 * dtype/ldx as the quantize call): the SQNR and the signal factor alpha of
 * x_hat = alpha y + noise ([UFP4-ZC] "治病药反而喂养了病菌" and "复利效应的反向
 * 版本"), the mean shrinkage and the rounding bias per grid cell ([UFP4-ZC]
 * "E2M1：一块刻度不均的尺子"; [UFP4-TW] 二) and IF4's INT4 share ([IF4] 6.2).
 * Writes UFP4_NSUMS doubles to sums (device), layout above.
 * ws: device workspace of ufp4_workspace_size(UFP4_OP_STATS, ...) bytes. */
int ufp4_stats(const void *x, int x_dtype, int64_t ldx, const ufp4_qtensor *q, double *sums, void *ws,
               size_t ws_bytes, void *stream);

/* Host-only: derive the report from sums copied to the host. */
void ufp4_stats_finalize(const double *sums_host, ufp4_stats_report *report);

/* Block-scaled GEMM Z = deq(A) deq(B)^T, fp32 output c[M][ldc], on the
 * operands' views: A is a's view (M x K) and B is b's view (N x K), so both
 * are quantized along K -- a row quantization of an M x K matrix, or a
 * column quantization of a K x M one (the transposed operands of the
 * backward GEMMs [UFP4-ZC] recipe table).  Same rht kind and seed (a shared
 * sign diagonal keeps A B^T).
 * mode UFP4_GEMM_NATIVE_MXFP4: E2M1/E8M0/32 operands on CDNA4's scaled MFMA
 *   ([UQ]; [MXFP4]); products exact, fp32 accumulation.
 * mode UFP4_GEMM_DEQUANT_BF16: any operands; x_hat rounded to bf16 (nearest
 *   even), bf16 MFMA, fp32 accumulation ([UQ]: software E1M2/INT4).  IF4's
 *   INT4 blocks dequantize with the 6/7 factor, so a product of two INT4
 *   blocks carries 36/49 and a mixed one 6/7 ([IF4] 4.1, the MAC unit's
 *   scaling by operand types).
 * Sizes: M, N multiples of 256; K multiple of 128; ldc multiple of 4, >= N;
 * 256 operand rows must span less than 4 GiB (K below about 16.7 million
 * elements), else UFP4_ERR_SHAPE.
 * ws: UFP4_GEMM_DEQUANT_BF16 needs ufp4_workspace_size(UFP4_OP_QGEMM, M + N,
 * K, cfg) bytes, whatever the operands' format; UFP4_GEMM_NATIVE_MXFP4 needs
 * none (ws may be NULL). */
int ufp4_qgemm(const ufp4_qtensor *a, const ufp4_qtensor *b, int mode, float *c, int64_t ldc, void *ws,
               size_t ws_bytes, void *stream);

/* Plain bf16 GEMM Z = A B^T, fp32 accumulation and output (the unquantized
 * product the attenuation eta is measured against).  A[M][lda], B[N][ldb] bf16;
 * M, N multiples of 256, K multiple of 64; lda, ldb multiples of 8; 256 rows
 * of A or B must span less than 4 GiB (lda, ldb below about 8.4 million),
 * else UFP4_ERR_SHAPE. */
int ufp4_gemm_bf16(const void *a, const void *b, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                   float *c, int64_t ldc, void *stream);

/* Attenuation sums ([UFP4-ZC] "复利效应的反向版本": eta = <Zq,Z>/<Z,Z>):
 * writes sums[0] = <Zq,Z>, sums[1] = <Z,Z>, sums[2] = ||Zq - Z||^2 (binary64,
 * device) for M x N fp32 matrices with row stride ld.
 * ws: ufp4_workspace_size(UFP4_OP_ETA, ...) bytes. */
int ufp4_eta(const float *zq, const float *z, int64_t M, int64_t N, int64_t ld, double *sums, void *ws,
             size_t ws_bytes, void *stream);

/* ---- FP4 KV cache and decode attention ([UQ], UltraQuant) ---------------
 * [UQ] describes decode attention with an FP8 query against a 4-bit KV cache
 * with UE8M0 group scales on CDNA4's native scaled MFMA, K and V treated
 * asymmetrically and K Walsh-Hadamard rotated; it gives no formulas.  These
 * calls compute (head dim D = 128, groups of 32, binary32 unless stated):
 *   MX rule: a group's exponent is E = floor(log2 amax) - emax, clamped to
 *     [-127, 127] (amax = 0 gives -127), stored biased (E + 127); elements
 *     are rounded to nearest-even after scaling by 2^-E and saturate at the
 *     format's maximum (E2M1: emax 2, max 6; E4M3FN: emax 8, max 448).
 *   Rotation: H_128, the Walsh-Hadamard matrix of order 128 (entries
 *     (-1)^popcount(i & j)), applied by butterflies with spans 1, 2, ..., 64
 *     in that order, each (a, b) -> (a + b, a - b).
 *   K (per token): MXFP4 of H k (rotate) or of k, groups along the head dim.
 *   V (per channel): MXFP4 over 32 consecutive tokens, no rotation.
 *   Q (per query row): MXFP8 (E4M3) of (H q) / 128 (rotate) or of q, groups
 *     along the head dim; (H q / 128) . (H k) = q . k.
 *   Scores s_t = <Q', K'_t> of the dequantized operands (fp32 accumulation),
 *     x_t = s_t c with c = sm_scale log2(e) rounded to binary32, tokens
 *     t < len.  p_t = 2^(x_t - m) for an integer m >= max x_t.
 *   P: per 32-token block, E = floor(log2 max p) - 7 (one above the MX rule,
 *     so the block maximum is never clamped), p' = E4M3(p 2^-E) 2^E.
 *   out = sum_t p'_t V'_t / sum_t p_t (fp32 accumulation); len = 0 gives 0.
 *     Any integer m gives the same result (the block exponents absorb 2^m),
 *     so the splits of a long cache combine by exact power-of-two rescaling.
 *   UFP4_KV_FP8: the FP8 KV cache [UQ] measures against, read as the same
 *     cache in MXFP8 (E4M3 elements with the MX rule above, same groups,
 *     rotation and probabilities).
 *
 * Cache layout: [B][Hkv][L_cap/128] pages of 17408 bytes, one per 128 tokens.
 * A page holds the operands of v_mfma_scale_f32_16x16x128_f8f6f4 in register
 * order (lane l, rho = l % 16, g = l / 16):
 *   [0, 8192)      K codes: 16 bytes at j*1024 + l*16 (j = 0..7) = channels
 *                  32g .. 32g+31 (low nibble first) of token
 *                  64(j/4) + 16(rho/4) + 4(j%4) + rho%4 of the page;
 *   [8192, 8704)   K exponents: byte j at l*8 + j, for the same token and
 *                  channel group;
 *   [8704, 16896)  V codes: 16 bytes at n*1024 + l*16 (n = 0..7) = tokens
 *                  32g .. 32g+31 (low nibble first) of channel 8 rho + n;
 *   [16896, 17408) V exponents: byte n at l*8 + n, same channel and tokens.
 * Tokens len .. (end of the last page) are stored as zeros; pages past the
 * last one holding a token are not written.
 * UFP4_KV_FP8 pages hold 33792 bytes.  K codes (E4M3): 16 bytes at
 * j*2048 + l*16 for the token's channels 16g .. 16g+15 and 16 bytes at
 * j*2048 + 1024 + l*16 for channels 64+16g .. 64+16g+15; K exponents at
 * 16384 + l*8 (byte j: the token's channel group g).  V codes at
 * 16896 + n*2048 + l*16 (tokens 16g .. 16g+15 of channel 8 rho + n) and
 * 16896 + n*2048 + 1024 + l*16 (tokens 64+16g .. +15); V exponents at
 * 33280 + l*8 (byte n: tokens 32g .. 32g+31).
 */

/* Bytes of a cache for B sequences, Hkv KV heads, capacity L_cap tokens
 * (a multiple of 128, below 8.1 million: one sequence's pages stay under
 * 2 GiB), head dim D (128), format UFP4_KV_FP4 or UFP4_KV_FP8.  0 for
 * unsupported sizes or formats. */
size_t ufp4_kv_cache_bytes(int64_t B, int64_t Hkv, int64_t L_cap, int64_t D, int kv_format);

/* Quantize K and V (bf16, device) into the cache.  Element (b, h, t, d) is at
 * k[b*stride_b + h*stride_h + t*stride_t + d] (strides in elements, multiples
 * of 8; k, v, cache 16-byte aligned).  lens: device int32[B], tokens per
 * sequence (clamped to [0, L_cap]).  rotate_k: 1 applies H_128 to K (the
 * decode must be called with the same value and format).  Errors: SHAPE
 * (L_cap not a multiple of 128, Hkv < 1, stride_t < D), UNSUPPORTED
 * (D != 128), ALIGN, INVALID_ARG (null pointer, rotate_k not 0/1, unknown
 * format). */
int ufp4_kv_cache_quantize(const void *k, const void *v, int64_t B, int64_t Hkv, int64_t L_cap, int64_t D,
                           int kv_format, int64_t stride_b, int64_t stride_h, int64_t stride_t, const int32_t *lens,
                           int rotate_k, uint8_t *cache, void *stream);

/* The query quantization of the decode on its own: rows x 128 bf16 (device,
 * contiguous) -> codes uint8[rows][128] (E4M3FN, sign in bit 7) and scales
 * uint8[rows][4] (biased exponents). */
int ufp4_kv_q_quantize(const void *q, int64_t rows, int64_t D, int rotate, uint8_t *codes, uint8_t *scales,
                       void *stream);

/* Workspace bytes of ufp4_kv_decode (0 when the cache is not split). */
size_t ufp4_kv_decode_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L_cap,
                                     int64_t pages_per_split);

/* One decode step: q bf16 [B][Hq][128] (query heads h*G .. h*G+G-1 read KV
 * head h, G = Hq/Hkv <= 16), the cache and lens as written by
 * ufp4_kv_cache_quantize, out fp32 [B][Hq][128].  pages_per_split: pages of
 * one workgroup (0 = chosen from the sizes); with more than one split a
 * second kernel combines them and ws must hold
 * ufp4_kv_decode_workspace_size(...) bytes.  Errors as above, plus
 * WORKSPACE, INVALID_ARG for a non-finite sm_scale. */
int ufp4_kv_decode(const void *q, const uint8_t *cache, const int32_t *lens, int64_t B, int64_t Hq, int64_t Hkv,
                   int64_t D, int kv_format, int64_t L_cap, float sm_scale, int rotate, int64_t pages_per_split,
                   float *out, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for op (UFP4_OP_*) on a rows x cols source (QGEMM: rows = M+N,
 * cols = K, the dequantize-to-bf16 mode's need for any format; ETA: rows = M,
 * cols = N).  cfg may be NULL except for AMAX (whose size depends on the axis). */
size_t ufp4_workspace_size(int op, int64_t rows, int64_t cols, const ufp4_config *cfg);

/* Text of an error code (static storage). */
const char *ufp4_strerror(int code);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int ufp4_last_hip_error(void);

/* Library version, (major << 16) | minor. */
int ufp4_version(void);

/* Timing aid.  The next kernel this library launches from the calling thread
 * records its own start and end on start_event and stop_event (hipEvent_t
 * handles the caller created; hipExtLaunchKernel attaches them to the
 * dispatch itself, so no separate event commands run around it).  The events
 * bracket the dispatch: on MI355X they read a few microseconds longer than
 * the kernel's duration in a profiler's kernel trace, and the timed launch
 * starts after a short gap.  For ufp4_quantize that kernel is the
 * quantize kernel, for ufp4_amax the amax pass, for ufp4_qgemm in
 * UFP4_GEMM_NATIVE_MXFP4 mode the GEMM.  The request is consumed by that
 * launch; passing two NULLs clears a pending one.  Per thread, no other
 * effect.  Returns UFP4_OK, or UFP4_ERR_INVALID_ARG if exactly one is NULL. */
int ufp4_time_next_launch(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif
#endif /* UFP4_H */
