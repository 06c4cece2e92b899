/*
 * mxq.h — MX-FP8 block quantization and (grouped) GEMM on AMD MI355X (gfx950).
 *
 * C ABI of libmxq.so.  Every pointer argument marked "device" is an address in
 * GPU memory; the library never allocates, frees or keeps any caller buffer.
 * All calls are asynchronous on the given HIP stream (NULL = the default
 * stream) and never synchronize the host, except mxq_validate_offsets.
 * Arguments are checked on the host before anything is launched; a failed
 * check returns an error code and launches nothing.  There is no fallback
 * to a higher-precision GEMM on any error.
 *
 * Pages cited (by title and section):
 *   [HP329]  "DeepSeek-V3 16B FSDP2 MXFP8/HiF8 训练设计" (hyper-parallel #329)
 *   [FPBLOG] "Transformer 与 LLM（06）：浮点格式、数值稳定性与混合精度"
 *   [TTNPU]  "低精度训练特性（MXFP8 / HiFloat8）" (torchtitan-npu)
 *
 * Data formats
 *   BF16 input   : uint16 bit patterns, row-major.
 *   E4M3 code    : uint8, 1 sign / 4 exponent / 3 mantissa bits, bias 7, no
 *                  Inf, S.1111.111 is NaN, largest value 448 ([FPBLOG] §二.2).
 *   E8M0 scale   : uint8 biased exponent, value 2^(c-127), 0xFF = NaN.  One
 *                  scale per 32 consecutive values along the blocked dimension
 *                  ([HP329] §3 table; [TTNPU] block size 32).
 *   MX rule      : per block, e = max(floor(log2(amax)) - 8, -127) (an all-zero
 *                  block takes -127), code_i = RNE_E4M3(x_i * 2^-e) with
 *                  magnitudes >= 448 saturated to 448; a block holding NaN or
 *                  Inf gets scale 0xFF and codes 0x7F.
 *   Per-tensor   : s = amax/448 in FP32 if amax is finite and > 0, else 1.0
 *                  ([HP329] §3.2); code_i = RNE_E4M3(fp32(x_i) / s) with the
 *                  same saturation; NaN inputs give 0x7F | sign.
 *
 * GEMM contract ([HP329] §8 direction table, §13.4): C = A · Bᵀ where A is
 * [M, K] and B is [N, K], both quantized along K (the contraction dim), so the
 * forward, dgrad and wgrad products are all this one call on the operand copy
 * whose 32-blocks run along that pass's contraction dim.  Products of the
 * dequantized operands are summed into FP32 accumulators and the result is
 * written once as BF16 (round to nearest even) or FP32 ([FPBLOG] §五.1).
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#define MXQ_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXQ_OK = 0,
  MXQ_ERR_NULL = 1,        /* a required pointer is NULL                        */
  MXQ_ERR_SHAPE = 2,       /* a size is negative, inconsistent or not a multiple
                              of what the operation needs                       */
  MXQ_ERR_ALIGN = 3,       /* a pointer or leading dimension is not 16-byte
                              aligned where the kernels load/store 16 bytes     */
  MXQ_ERR_ARG = 4,         /* an enum argument is out of range                  */
  MXQ_ERR_WORKSPACE = 5,   /* workspace too small (see mxq_workspace_size)      */
  MXQ_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed        */
  MXQ_ERR_OFFSETS = 7      /* mxq_validate_offsets found bad group offsets      */
} mxq_status;

typedef enum { MXQ_OUT_BF16 = 0, MXQ_OUT_FP32 = 1 } mxq_out_dtype;

/* Human-readable name of a status code (static string). */
MXQ_API const char* mxq_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
MXQ_API int mxq_version(void);

/* ------------------------------------------------------------------------ *
 * Quantization                                                              *
 * ------------------------------------------------------------------------ */

/*
 * Row-wise (1x32) MX quantization ([HP329] §3 table, "1×32 block"; [TTNPU]
 * "线性层低精度": every 32 elements share one scale).
 *   x     : device, BF16 [M, K], row stride ldx elements.
 *   q     : device, E4M3 [M, K], row stride ldq bytes.
 *   scale : device, E8M0 [M, K/32], row stride lds bytes.
 * Requires K % 32 == 0, ldx >= K, ldq >= K, lds >= K/32, ldx % 8 == 0,
 * ldq % 16 == 0, x and q 16-byte aligned.  M == 0 or K == 0 is a no-op.
 */
MXQ_API int mx_quantize_rowwise(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        uint8_t* q, int64_t ldq, uint8_t* scale, int64_t lds,
                        hipStream_t stream);

/*
 * Several row-wise MX quantizations in one launch, e.g. a Linear's input and
 * weight, whose forward product reads both row copies ([HP329] §8 direction
 * table).  Each item receives exactly the codes and scales that
 * mx_quantize_rowwise gives it, under the same requirements; an item with
 * M == 0 or K == 0 is skipped.
 *   items : host array of n items, read during the call only.
 *   n     : 1 .. MXQ_ROWWISE_BATCH_MAX (else MXQ_ERR_SHAPE).
 * The first item that fails a check decides the returned status and nothing
 * is launched.  Items must not write overlapping memory.
 */
#define MXQ_ROWWISE_BATCH_MAX 4
typedef struct mxq_rowwise_item {
  const uint16_t* x;    /* device, BF16 [M, K], row stride ldx elements */
  int64_t M, K, ldx;
  uint8_t* q;           /* device, E4M3 [M, K], row stride ldq bytes */
  int64_t ldq;
  uint8_t* scale;       /* device, E8M0 [M, K/32], row stride lds bytes */
  int64_t lds;
} mxq_rowwise_item;
MXQ_API int mx_quantize_rowwise_batch(const mxq_rowwise_item* items, int32_t n,
                                      hipStream_t stream);

/*
 * Column-wise (32x1) MX quantization with transposed output ([HP329] §3 table
 * "32×1 block", §3.1 row and col copies are distinct physical data), in its
 * grouped form for the MoE wgrad operands ([TTNPU] "MoE 专家层低精度": the
 * weight gradient quantizes per expert group).
 *   x        : device, BF16 [M, K], row stride ldx elements.
 *   offsets  : device int64 [E+1] or NULL.  Group g owns rows
 *              [offsets[g], offsets[g+1]); offsets must be non-decreasing with
 *              offsets[0] == 0 and offsets[E] == M.  NULL means one group of
 *              all M rows (E is then ignored).
 *   qT       : device, E4M3 [K, ldqT]: row k holds column k of x, blocked by
 *              32 along M.  Each group is padded with zero rows to a multiple
 *              of 32, so group g occupies columns [poff[g], poff[g+1]) with
 *              poff[g+1] - poff[g] = ceil(m_g/32)*32.
 *   M_cap    : number of output columns written.  The padded total is
 *              known only on the device, so M_cap must be >= its bound
 *              M + 31*E (M rounded up to 32 when offsets is NULL), else
 *              MXQ_ERR_SHAPE (M == 0 needs nothing).  Columns in
 *              [padded total, M_cap) are zero-filled (codes and scales).
 *   scaleT   : device, E8M0 [K, ldsT], ldsT >= M_cap/32.
 *   offsets_padded : device int64 [E+1] receiving poff, or NULL.
 * Requires K % 8 == 0, M_cap % 32 == 0, ldqT >= M_cap, ldqT % 16 == 0,
 * ldx % 8 == 0, x and qT 16-byte aligned.  Offsets that break the rules
 * above give unspecified codes but never an access outside the buffers.
 */
MXQ_API int mx_quantize_colwise(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        const int64_t* offsets, int32_t E,
                        uint8_t* qT, int64_t ldqT, int64_t M_cap,
                        uint8_t* scaleT, int64_t ldsT,
                        int64_t* offsets_padded, hipStream_t stream);

/*
 * Dual-axis MX quantization: the row-wise copy of mx_quantize_rowwise and the
 * (grouped) column-wise copy of mx_quantize_colwise from one read of x
 * ([HP329] §3.1: an MX weight keeps row data + scale and col data + scale;
 * §8.1: both are produced once from the master copy after the optimizer step,
 * while activations and gradients are quantized on the fly and feed both the
 * dgrad and the wgrad products).  Every output is bit-identical to the
 * corresponding single-axis call.
 *   x, M, K, ldx, offsets, E                 : as for mx_quantize_colwise.
 *   q, ldq, scale, lds                        : as for mx_quantize_rowwise.
 *   qT, ldqT, M_cap, scaleT, ldsT, offsets_padded : as for mx_quantize_colwise.
 * Requires the conditions of both calls (K % 32 == 0, ldq % 16 == 0, q
 * 16-byte aligned, and those of mx_quantize_colwise).  M == 0 writes only the
 * zero padding of the column copy; K == 0 or M_cap == 0 is a no-op.
 */
MXQ_API int mx_quantize_dual(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                     const int64_t* offsets, int32_t E,
                     uint8_t* q, int64_t ldq, uint8_t* scale, int64_t lds,
                     uint8_t* qT, int64_t ldqT, int64_t M_cap,
                     uint8_t* scaleT, int64_t ldsT,
                     int64_t* offsets_padded, hipStream_t stream);

/*
 * Several dual-axis MX quantizations in one launch, each with its own groups,
 * e.g. a product's activation and its expert weights, whose forward product
 * reads both row copies and whose backward products read the column copies
 * ([HP329] §8 direction table; §8.1 activations and weights each keep both
 * copies).  Each item receives exactly the outputs mx_quantize_dual gives it,
 * under the same requirements; an item with K == 0 or M_cap == 0 is skipped.
 *   items : host array of n items, read during the call only.
 *   n     : 1 .. MXQ_DUAL_BATCH_MAX (else MXQ_ERR_SHAPE).
 * The first item that fails a check decides the returned status and nothing
 * is launched.  Items must not write overlapping memory.
 */
#define MXQ_DUAL_BATCH_MAX 4
typedef struct mxq_dual_item {
  const uint16_t* x;         /* device, BF16 [M, K], row stride ldx elements */
  int64_t M, K, ldx;
  const int64_t* offsets;    /* device int64 [E+1] or NULL, as for mx_quantize_colwise */
  int32_t E;
  uint8_t* q;                /* row copy: E4M3 [M, K], row stride ldq bytes */
  int64_t ldq;
  uint8_t* scale;            /* row copy: E8M0 [M, K/32], row stride lds bytes */
  int64_t lds;
  uint8_t* qT;               /* column copy: E4M3 [K, ldqT], M_cap columns written */
  int64_t ldqT, M_cap;
  uint8_t* scaleT;           /* column copy: E8M0 [K, ldsT] */
  int64_t ldsT;
  int64_t* offsets_padded;   /* device int64 [E+1] receiving poff, or NULL */
} mxq_dual_item;
MXQ_API int mx_quantize_dual_batch(const mxq_dual_item* items, int32_t n, hipStream_t stream);

/*
 * Per-tensor current-scaling FP8 E4M3 ([HP329] §3.2 current scaling: FP32
 * scale s = amax / 448 when amax is finite and non-zero, else s = 1;
 * [FPBLOG] §七.2 first pass finds amax, second pass quantizes).
 *   x         : device, BF16 [n], contiguous, 16-byte aligned.
 *   q         : device, E4M3 [n], 16-byte aligned.
 *   scale     : device float[1] receiving s.
 *   workspace : device scratch of at least
 *               mxq_workspace_size(MXQ_WS_PER_TENSOR, n, 0, 0, 0) bytes.
 */
MXQ_API int fp8_quantize_per_tensor(const uint16_t* x, int64_t n, uint8_t* q, float* scale,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * fp8_quantize_per_tensor with the tensor's amax given instead of found by a
 * first pass over x ([FPBLOG] §七.2: the amax pass is current scaling's extra
 * read, and the producing matmul's epilogue can supply the amax, as
 * fp8_gemm_per_tensor_amax does).
 *   amax  : device float[1]; the scale is the rule above applied to it
 *           (s = amax / 448 in FP32 when amax is finite and > 0, else 1; a NaN
 *           or infinite amax turns NaN codes into 0x7F | sign and saturates
 *           +-Inf, as the two-pass call does).  The codes and scale equal
 *           fp8_quantize_per_tensor's when amax is the true max |x|.
 *   x, q  : as for fp8_quantize_per_tensor; scale: device float[1] receiving s.
 * No workspace.  n == 0 writes only the scale.
 */
MXQ_API int fp8_quantize_per_tensor_amax(const uint16_t* x, int64_t n, const float* amax,
                                 uint8_t* q, float* scale, hipStream_t stream);

/*
 * Per-group (per-expert) current-scaling FP8 E4M3 ([HP329] §3 format table:
 * a grouped tensor keeps one FP32 scale per leading group; §3.2: 3-D grouped
 * weights take a per-leading-group scale, each from the rule above; [TTNPU]
 * MoE expert layers, HiFloat8 mode: each expert group shares one scale).
 * Rows [offsets[e], offsets[e+1]) of x form group e:
 *   s_e = amax_e / 448 in FP32 if amax_e is finite and > 0, else 1.0 (an
 *   empty group gets 1.0); code = RNE_E4M3(fp32(x) / s_e), saturating, as
 *   for fp8_quantize_per_tensor.
 * A 3-D weight [E, N, K] is the [E*N, K] matrix with offsets e*N.
 *   x         : device, BF16 [M, K], row stride ldx elements; K % 8 == 0,
 *               ldx % 8 == 0, 16-byte aligned.
 *   offsets   : device int64 [E+1], 1 <= E <= 256, offsets[0] = 0,
 *               non-decreasing, offsets[E] = M (rows outside [offsets[0],
 *               offsets[E]) get unspecified codes; nothing is accessed out of
 *               bounds for malformed offsets).
 *   q         : device, E4M3 [M, K], row stride ldq bytes (% 8 == 0),
 *               8-byte aligned.
 *   scales    : device float[E] receiving s_e.
 *   workspace : device scratch of at least
 *               mxq_workspace_size(MXQ_WS_PER_GROUP, M, E, 0, 0) bytes.
 * Three kernels: row maxima, group scales, encoding (two reads of x).
 */
MXQ_API int fp8_quantize_per_group(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                           const int64_t* offsets, int32_t E,
                           uint8_t* q, int64_t ldq, float* scales,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fp8_quantize_per_group for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument and no allocation.  The row and group
 * maxima go to a 1 MiB device array inside the library, one per GPU, held
 * until the process ends; its address is looked up on the first call on each
 * device (the current device must be the stream's).  Limit: M + E <= 262144
 * (MXQ_ERR_SHAPE beyond).  Calls that overlap on one GPU (concurrent streams
 * or host threads) share that array and race; serialize them.
 *   x, M, K, ldx, offsets, E, q, ldq, scales : as fp8_quantize_per_group,
 *   with the same results bit for bit.
 */
MXQ_API int fp8_quantize_per_group_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   const int64_t* offsets, int32_t E,
                                   uint8_t* q, int64_t ldq, float* scales, hipStream_t stream);

/*
 * Transposed copy of the per-group current-scaling quantization, for the
 * products that contract over x's rows: the weight gradient over each
 * expert's tokens, the data gradient over a weight's output rows.  [HP329]
 * §3: with FP32 per-tensor / per-group scales the quantized data do not
 * depend on the GEMM direction, only the operand layout does, so the codes
 * and scales equal fp8_quantize_per_group's; the layout is that of
 * mx_quantize_colwise: group e's rows become columns
 * [offsets_padded[e], offsets_padded[e] + count_e) of qT, each group padded
 * with zero columns to a multiple of 32, columns past the padded total
 * zero-filled.
 *   x, offsets, E, scales, workspace : as fp8_quantize_per_group.
 *   qT            : device, E4M3 [K, M_cap], row stride ldqT bytes (% 16 == 0),
 *                   16-byte aligned; M_cap % 32 == 0 and M_cap >= M + 31*E
 *                   (the bound of the padded total; else MXQ_ERR_SHAPE).
 *   offsets_padded: device int64 [E+1] receiving the padded offsets, or NULL.
 */
MXQ_API int fp8_quantize_per_group_colwise(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   const int64_t* offsets, int32_t E,
                                   uint8_t* qT, int64_t ldqT, int64_t M_cap, float* scales,
                                   int64_t* offsets_padded, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * fp8_quantize_per_group and fp8_quantize_per_group_colwise with each
 * group's amax given instead of found by a pass over x ([FPBLOG] §七.2: the
 * amax pass is current scaling's extra read, and the producing matmul's
 * epilogue can supply the amax; fp8_grouped_gemm_per_group_swiglu does).
 *   amax : device float[E], amax[e] = max |x| over group e's rows (NaN if
 *          the group holds a NaN; 0 for an empty group).  The scale rule is
 *          the one above applied to amax[e]; the codes equal the plain
 *          entry's when amax[e] is the group's true max |x|.
 * The other arguments, layouts and errors are those of the plain entries;
 * the workspace needs only mxq_workspace_size(MXQ_WS_PER_GROUP, 0, E, 0, 0)
 * bytes (no row maxima).
 */
MXQ_API int fp8_quantize_per_group_amax(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                const int64_t* offsets, int32_t E, const float* amax,
                                uint8_t* q, int64_t ldq, float* scales,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);
MXQ_API int fp8_quantize_per_group_colwise_amax(const uint16_t* x, int64_t M, int64_t K,
                                        int64_t ldx, const int64_t* offsets, int32_t E,
                                        const float* amax, uint8_t* qT, int64_t ldqT,
                                        int64_t M_cap, float* scales, int64_t* offsets_padded,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/*
 * Both per-group copies from one encoding pass (the per-expert counterpart of
 * mx_quantize_dual): the row-major codes of fp8_quantize_per_group and the
 * transposed, group-padded codes of fp8_quantize_per_group_colwise, with the
 * same group scales, after one amax pass over x.
 *   amax     : device float[E] of the groups' amaxes, as for
 *              fp8_quantize_per_group_amax (then there is no amax pass and the
 *              workspace needs mxq_workspace_size(MXQ_WS_PER_GROUP, 0, E, 0, 0)
 *              bytes), or NULL.
 *   q, ldq   : device E4M3 [M, K] (ldq % 8 == 0, 8-byte aligned).
 *   qT, ldqT, M_cap, scales, offsets_padded : as fp8_quantize_per_group_colwise.
 *   workspace: mxq_workspace_size(MXQ_WS_PER_GROUP, M, E, 0, 0) bytes.
 * Rows outside every group are not written; M_cap >= M + 31*E is required
 * (MXQ_ERR_SHAPE otherwise), so every row lands in both copies.
 */
MXQ_API int fp8_quantize_per_group_dual(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                const int64_t* offsets, int32_t E, const float* amax,
                                uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT,
                                int64_t M_cap, float* scales, int64_t* offsets_padded,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * GEMMs                                                                     *
 * ------------------------------------------------------------------------ */

/*
 * Accumulation of the E4M3 products.
 *  MXQ_ACC_MFMA_FP8 : the gfx950 block-scaled FP8 MFMA.  The matrix unit sums
 *     each run of 8 consecutive-k products after aligning them to the largest
 *     exponent sum in the run, keeping 13 bits below it (smaller products are
 *     truncated toward zero), then adds the run sums in FP32.
 *     Fast; outside the contract's |C - Y| <= 1e-5*S + 1e-6 when a run mixes
 *     a large product with much smaller ones (outlier-heavy activations).
 *  MXQ_ACC_FP32 : every product exact, summed in FP32 ("Transformer 与 LLM
 *     （06）" §五.1: FP8 inputs, FP32 accumulation).  Each 32-block of codes is
 *     widened to BF16 with its E8M0 scale folded in (v_cvt_scalef32_pk_bf16_fp8:
 *     exact for scale codes 3..246, i.e. every block of finite BF16 values
 *     whose largest magnitude is at least 2^-116; smaller blocks may lose
 *     bits below 2^-133) and multiplied on the BF16 matrix instruction, whose
 *     products are exact and whose sums stay within FP32 accuracy (measured
 *     error <= 1e-6 S at K = 2048).  Meets the contract's rule; at most half
 *     the FP8 mode's throughput (BF16 matrix peak).  Accepted by mx_gemm,
 *     fp8_gemm_per_tensor, mx_grouped_gemm, mx_grouped_gemm_wgrad and the
 *     per-group-scaled grouped GEMMs; fp8_gemm_blockwise returns MXQ_ERR_ARG
 *     for it (that recipe promotes per block on the FP8 unit by design).
 */
typedef enum { MXQ_ACC_MFMA_FP8 = 0, MXQ_ACC_FP32 = 1 } mxq_accum;

/*
 * Dense MX GEMM  C[M, N] = A[M, K] · B[N, K]ᵀ  ([HP329] §13.4
 * low_precision_matmul; [TTNPU] quant matmul).
 *   a, b         : device E4M3 codes, row strides lda, ldb bytes (>= K).
 *   a_scale, b_scale : device E8M0 [M, K/32] / [N, K/32], row strides
 *                  ldsa, ldsb bytes (>= K/32).
 *   c            : device output [M, N], row stride ldc elements, BF16 or FP32.
 * Requires K % 32 == 0; lda, ldb % 16 == 0; a, b 16-byte aligned; ldc >= N;
 * (M rows of lda bytes and the scale rows) addressable with 32-bit offsets
 * per 256-row tile.  Scale pointers and strides have no alignment rule;
 * when ldsa and ldsb are both multiples of 16 the scales are fetched in
 * 16-byte windows (much less load traffic), otherwise byte by byte.
 * K == 0 writes zeros; M == 0 or N == 0 is a no-op.
 */
MXQ_API int mx_gemm(const uint8_t* a, const uint8_t* a_scale, int64_t lda, int64_t ldsa,
            const uint8_t* b, const uint8_t* b_scale, int64_t ldb, int64_t ldsb,
            int64_t M, int64_t N, int64_t K,
            void* c, int64_t ldc, int out_dtype, int accum, hipStream_t stream);

/*
 * Per-tensor FP8 GEMM  C = s_a * s_b * (Q_a · Q_bᵀ)  ([HP329] §3.2 current
 * scaling with FP32 scales; [TTNPU] HiFloat8 mode: per-tensor quantization
 * then quant matmul).  a_scale, b_scale: device float[1] each.  Same shapes,
 * strides and requirements as mx_gemm without the block scales.
 */
MXQ_API int fp8_gemm_per_tensor(const uint8_t* a, const float* a_scale, int64_t lda,
                        const uint8_t* b, const float* b_scale, int64_t ldb,
                        int64_t M, int64_t N, int64_t K,
                        void* c, int64_t ldc, int out_dtype, int accum,
                        hipStream_t stream);

/*
 * fp8_gemm_per_tensor that also takes the current-scaling amax of its output
 * in the epilogue ([FPBLOG] §七.2: the amax can come from the producing
 * matmul, so quantizing C per tensor needs no amax pass; [HP329] §3.2 current
 * scaling).  Same arguments and requirements as fp8_gemm_per_tensor, plus
 *   c_amax : device float[1], 4-byte aligned.  Cleared, then set to the
 *            largest |C| over the M x N outputs as stored (rounded to the
 *            output type): NaN if an output is NaN, else +Inf if one is
 *            infinite; 0 when M, N or K is 0.
 * fp8_quantize_per_tensor_amax(C, ..., c_amax, ...) then gives exactly the
 * codes and scale of fp8_quantize_per_tensor(C, ...).
 */
MXQ_API int fp8_gemm_per_tensor_amax(const uint8_t* a, const float* a_scale, int64_t lda,
                             const uint8_t* b, const float* b_scale, int64_t ldb,
                             int64_t M, int64_t N, int64_t K,
                             void* c, int64_t ldc, int out_dtype, int accum, float* c_amax,
                             hipStream_t stream);

/*
 * Blockwise FP8, the comparison recipe ([FPBLOG] §七.3, DeepSeek-V3): E4M3
 * codes with one FP32 scale per 1x128 activation block (per row, per 128
 * columns) or 128x128 weight block, each block quantized by the current-
 * scaling rule of fp8_quantize_per_tensor (scale = amax/448 in FP32 if amax
 * is finite and > 0, else 1.0; codes RNE_E4M3(fp32(x)/scale), saturating).
 *   x, w    : device BF16 [M, K] / [N, K], row strides ldx / ldw (multiples
 *             of 8), 16-byte aligned; K % 128 == 0.
 *   q       : device E4M3 codes, same shape, row stride ldq (multiple of 8).
 *   scales  : device float, activations [M, K/128], weights [ceil(N/128),
 *             K/128] (the last block row may cover fewer than 128 rows), row
 *             stride lds (floats).
 */
MXQ_API int fp8_quantize_blockwise_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               uint8_t* q, int64_t ldq, float* scales, int64_t lds,
                               hipStream_t stream);
MXQ_API int fp8_quantize_blockwise_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* q, int64_t ldq, float* scales, int64_t lds,
                                  hipStream_t stream);

/*
 * Blockwise FP8 GEMM ([FPBLOG] §七.3: each 128-wide slice of the contraction
 * is multiplied by its blocks' s_a * s_w when it is promoted into the FP32
 * sum):  C[m, n] = Σ_b a_scales[m, b] * b_scales[n/128, b] * Σ_{k in block b} Q_a[m,k] Q_b[n,k].
 * Each 64-wide half of a block is formed on the FP8 matrix unit with unit
 * scales and added to the FP32 accumulators times the two scales (FMA).
 *   a, a_scales : codes [M, K] (lda) and float [M, K/128] (ldsa, floats),
 *                 from fp8_quantize_blockwise_act.
 *   b, b_scales : codes [N, K] (ldb) and float [ceil(N/128), K/128] (ldsb),
 *                 from fp8_quantize_blockwise_weight.
 *   c           : device [M, N] BF16 or FP32, row stride ldc.
 * Requires K % 128 == 0, lda/ldb multiples of 16 with 16-byte aligned codes,
 * 4-byte aligned scales; accum == MXQ_ACC_MFMA_FP8 (else MXQ_ERR_ARG).
 */
MXQ_API int fp8_gemm_blockwise(const uint8_t* a, const float* a_scales, int64_t lda, int64_t ldsa,
                       const uint8_t* b, const float* b_scales, int64_t ldb, int64_t ldsb,
                       int64_t M, int64_t N, int64_t K,
                       void* c, int64_t ldc, int out_dtype, int accum,
                       hipStream_t stream);

/*
 * Grouped MX GEMM with variable M (MoE forward and dgrad; [HP329] §5.2
 * routed experts, §13.4 low_precision_grouped_matmul with group_list;
 * [TTNPU] grouped matmul).
 *   For each group e with rows [offsets[e], offsets[e+1]):
 *     C[rows, :] = A[rows, :] · B_eᵀ
 *   a, a_scale  : device, [M, K] codes / [M, K/32] scales, row strides lda, ldsa.
 *   b, b_scale  : device, per expert e an [N, K] code matrix at
 *                 b + e*b_estride (row stride ldb) and its [N, K/32] scales at
 *                 b_scale + e*bs_estride (row stride ldsb).  A contiguous
 *                 [E, N, K] tensor has b_estride = N*ldb, bs_estride = N*ldsb;
 *                 the column-quantized weights of mx_quantize_colwise (one
 *                 group per expert) have b_estride = rows per expert and
 *                 bs_estride = rows per expert / 32.
 *   offsets     : device int64 [E+1], as for mx_quantize_colwise.
 *   c           : device [M, N], row stride ldc.
 * Rows of empty groups do not exist; nothing else is written.
 * Same alignment requirements as mx_gemm; b_estride % 16 == 0.
 */
MXQ_API int mx_grouped_gemm(const uint8_t* a, const uint8_t* a_scale, int64_t lda, int64_t ldsa,
                    const uint8_t* b, const uint8_t* b_scale, int64_t ldb, int64_t ldsb,
                    int64_t b_estride, int64_t bs_estride,
                    const int64_t* offsets, int32_t E,
                    int64_t M, int64_t N, int64_t K,
                    void* c, int64_t ldc, int out_dtype, int accum,
                    hipStream_t stream);

/*
 * Routed experts' gate/up product with SwiGLU and the MX quantization of its
 * output in the epilogue (the producer of the down matmul's operands:
 * [HP329] §5.2 gate_up weight [E, 2F, H] and grouped SwiGLU, §3 row and
 * column copies; [TTNPU] grouped MX quant for the expert wgrad; [FPBLOG]
 * §七.2 quantization bookkeeping folded into the producing matmul).
 *   For each group e with rows [offsets[e], offsets[e+1]):
 *     GU = A[rows, :] · B_eᵀ  (FP32 sums), g = GU[:, :F], u = GU[:, F:],
 *     h  = silu(g) * u,  silu(x) = x / (1 + e^-x), in FP32,
 *   and h is MX-quantized as mx_quantize_dual would quantize it, from the FP32
 *   values (no BF16 rounding in between).
 *   a, a_scale  : device, [M, K] codes / [M, K/32] scales (row copy), strides lda, ldsa.
 *   b, b_scale  : device, per expert e the [2F, K] gate_up codes (gate rows
 *                 [0, F), up rows [F, 2F)) at b + e*b_estride, row stride ldb,
 *                 and its scales at b_scale + e*bs_estride, row stride ldsb.
 *   offsets     : device int64 [E+1] expert row ranges.
 *   gu          : device BF16 [M, 2F] (row stride ldgu) receiving the gate/up
 *                 product (for the SwiGLU backward), or NULL to skip it.
 *   hq, hs      : device, h's row copy: codes [M, F] (stride ldhq), scales
 *                 [M, F/32] (stride ldhs).
 *   hqT, hsT    : device, h's grouped column copy: codes [F, M_cap] (stride
 *                 ldhqT), scales [F, M_cap/32] (stride ldhsT); each group zero-
 *                 padded to a multiple of 32 rows, as mx_quantize_colwise with
 *                 offsets; M_cap >= M + 31*E is required when M > 0 (the
 *                 bound of the padded total; MXQ_ERR_SHAPE otherwise).
 *   offsets_padded : device int64 [E+1] receiving the padded offsets, or NULL.
 * Requires F % 32 == 0, K % 32 == 0, M_cap % 32 == 0, ldhq and ldhqT multiples
 * of 16 with 16-byte aligned hq, hqT; ldgu % 8 == 0 and 16-byte aligned gu; the
 * operand requirements of mx_grouped_gemm; an expert's 2F weight rows within
 * 2^30 bytes.  F == 0 is a no-op; with M == 0 only offsets_padded is written.
 */
MXQ_API int mx_grouped_gemm_swiglu(const uint8_t* a, const uint8_t* a_scale, int64_t lda,
                           int64_t ldsa, const uint8_t* b, const uint8_t* b_scale,
                           int64_t ldb, int64_t ldsb, int64_t b_estride, int64_t bs_estride,
                           const int64_t* offsets, int32_t E,
                           int64_t M, int64_t F, int64_t K,
                           void* gu, int64_t ldgu,
                           uint8_t* hq, int64_t ldhq, uint8_t* hs, int64_t ldhs,
                           uint8_t* hqT, int64_t ldhqT, uint8_t* hsT, int64_t ldhsT,
                           int64_t M_cap, int64_t* offsets_padded,
                           hipStream_t stream);

/*
 * Grouped MX GEMM with variable K (MoE weight gradient, contraction over the
 * tokens of each expert; [HP329] §8 wgrad row, [TTNPU] grouped MX quant for
 * wgrad).  Operands come from mx_quantize_colwise with the same offsets:
 *   at, at_scale : device, [N, ld] codes / scales: the column-quantized
 *                  transpose of the output gradient (N = its feature dim).
 *   bt, bt_scale : device, [K, ld] codes / scales: the column-quantized
 *                  transpose of the layer input (K = its feature dim).
 *   offsets_padded : device int64 [E+1], multiples of 32 (poff).
 *   For each group e: dW_e[N, K] = Σ_{t in [poff[e], poff[e+1])} at[:, t] · bt[:, t]ᵀ
 *   c : device [E, N, K] with row stride ldc and expert stride N*ldc; an empty
 *       group writes zeros.
 * Requires lda_t, ldb_t % 16 == 0 and 16-byte aligned code pointers.  As for
 * mx_gemm, scale row strides that are multiples of 16 take the faster path.
 */
MXQ_API int mx_grouped_gemm_wgrad(const uint8_t* at, const uint8_t* at_scale, int64_t lda_t, int64_t ldsa_t,
                          const uint8_t* bt, const uint8_t* bt_scale, int64_t ldb_t, int64_t ldsb_t,
                          const int64_t* offsets_padded, int32_t E,
                          int64_t N, int64_t K,
                          void* c, int64_t ldc, int out_dtype, int accum,
                          hipStream_t stream);

/*
 * Grouped FP8 GEMM with per-group FP32 scales, variable M (the grouped
 * matmul of [HP329] §13.4 on operands from fp8_quantize_per_group, [HP329] §3
 * per-expert current scaling):  for each group e with rows
 * [offsets[e], offsets[e+1]):
 *   C[rows, :] = a_scales[e] * b_scales[e] * (Q_a[rows, :] · Q_b,eᵀ)
 * summed in FP32 on the FP8 matrix unit (unit block scales), the two scales
 * multiplied into the sum before the single rounding to the output type.
 *   a           : device, [M, K] codes, row stride lda.
 *   b           : device, per expert e an [N, K] code matrix at b + e*b_estride
 *                 (row stride ldb).
 *   a_scales, b_scales : device float[E].
 *   offsets, c  : as mx_grouped_gemm.
 * Same requirements as mx_grouped_gemm (K % 32 == 0, 16-byte alignment).
 */
MXQ_API int fp8_grouped_gemm_per_group(const uint8_t* a, const float* a_scales, int64_t lda,
                               const uint8_t* b, const float* b_scales, int64_t ldb,
                               int64_t b_estride, const int64_t* offsets, int32_t E,
                               int64_t M, int64_t N, int64_t K,
                               void* c, int64_t ldc, int out_dtype, int accum,
                               hipStream_t stream);

/*
 * Per-group-scaled gate/up product with SwiGLU in the epilogue, for the
 * per-expert current-scaling format ([HP329] §5.2 gate_up [E, 2F, H] and
 * grouped SwiGLU, §3 per-group scales; [FPBLOG] §七.2 amax taken in the
 * producing matmul's epilogue):  for each group e with rows
 * [offsets[e], offsets[e+1]):
 *   GU = a_scales[e] * b_scales[e] * (Q_a[rows] · Q_b,eᵀ) (FP32),
 *   h  = BF16(silu(GU[:, :F]) * GU[:, F:])  (silu in FP32, one rounding),
 *   h_amax[e] = max |h| over the group's rows (0 for an empty group; NaN if
 *               any h is NaN),
 * so that fp8_quantize_per_group_amax / _colwise_amax quantize h without an
 * amax pass.
 *   a, b        : codes as fp8_grouped_gemm_per_group (b: [2F, K] per expert,
 *                 gate rows [0, F), up rows [F, 2F)); a_scales, b_scales float[E].
 *   gu          : device BF16 [M, 2F] (stride ldgu) or NULL.
 *   h           : device BF16 [M, F], row stride ldh.
 *   h_amax      : device float[E]; cleared and filled by this call.
 * Requires F % 32 == 0, K % 32 == 0, ldh % 8 == 0 and 16-byte aligned h; gu
 * as for mx_grouped_gemm_swiglu; an expert's 2F weight rows within 2^30 bytes.
 */
MXQ_API int fp8_grouped_gemm_per_group_swiglu(const uint8_t* a, const float* a_scales,
                                      int64_t lda, const uint8_t* b, const float* b_scales,
                                      int64_t ldb, int64_t b_estride,
                                      const int64_t* offsets, int32_t E,
                                      int64_t M, int64_t F, int64_t K,
                                      void* gu, int64_t ldgu, uint16_t* h, int64_t ldh,
                                      float* h_amax, hipStream_t stream);

/*
 * Weight gradient with per-group FP32 scales (variable K, the per-expert
 * current-scaling counterpart of mx_grouped_gemm_wgrad): for each group e,
 *   dW_e[N, K] = a_scales[e] * b_scales[e] * Σ_{t in [poff[e], poff[e+1])} at[:, t] · bt[:, t]ᵀ
 * with at [N, ld], bt [K, ld] from fp8_quantize_per_group_colwise (same
 * offsets) and a_scales, b_scales device float[E].  Output, strides and
 * requirements as mx_grouped_gemm_wgrad without the block scales.
 */
MXQ_API int fp8_grouped_gemm_wgrad_per_group(const uint8_t* at, const float* a_scales, int64_t lda_t,
                                     const uint8_t* bt, const float* b_scales, int64_t ldb_t,
                                     const int64_t* offsets_padded, int32_t E,
                                     int64_t N, int64_t K,
                                     void* c, int64_t ldc, int out_dtype, int accum,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Helpers                                                                   *
 * ------------------------------------------------------------------------ */

/* Workspace kinds: per-tensor quantization (n = elements), per-group
 * quantization (n = rows, a1 = groups). */
enum { MXQ_WS_PER_TENSOR = 0, MXQ_WS_PER_GROUP = 1 };

/* Workspace bytes an operation needs (0 if none). */
MXQ_API size_t mxq_workspace_size(int op, int64_t n, int64_t a1, int64_t a2, int64_t a3);

/*
 * Debug check of device-side group offsets: copies them to the host (this
 * call synchronizes the stream) and verifies offsets[0] == 0, non-decreasing,
 * offsets[E] == M.  Returns MXQ_OK or MXQ_ERR_OFFSETS.
 */
MXQ_API int mxq_validate_offsets(const int64_t* offsets, int32_t E, int64_t M, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MXQ_H */
