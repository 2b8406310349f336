/*
 * qgemm.h -- C ABI of the quantized linear layer for AMD MI355X (gfx950).
 *
 * The layer computes Y[M,N] = X[M,K] . W[K,N] from quantized operands:
 *   - per-token dynamic symmetric int8 activations,
 *   - per-output-channel symmetric int8 weights (W8A8), or
 *   - group-wise (128 along K) asymmetric uint4 weights dequantized inside the
 *     GEMM, with int8 activations (W4A8) or 16-bit float activations (W4A16).
 *
 * Sources, cited by page title and section:
 *   「第4章：量化」: §1.1 x_int = round(x/s) + z and x_hat = (x_int - z) s;
 *     §1.2 symmetric s = max|x|/127 and asymmetric scale from max - min;
 *     §1.3 per-channel, per-group (g = 32/64/128) and per-token (dynamic)
 *     granularity; §2.2 the SmoothQuant fold; §2.3 W8A8 runs the GEMM on int8
 *     units; §3.1 weight-only 4-bit keeps activations in 16-bit floats;
 *     §3.2-3.3 bits = 4, group size 128, zero point on, contiguous groups;
 *     §3.5 dequantize inside the GEMM instead of a separate pass.
 *   「Quantization & Flash Attention」 §2.2-2.3: the AWQ per-channel fold.
 *   「LLM推理降本五要素」 §2.1 (W8A8 decode is weight-bandwidth bound), §2.2
 *     (W4A8 with per-group scale and zero; the quantized_matmul(x, weight,
 *     scale, zero) argument order; the INT8 outlier side path), §5.2 (round,
 *     then clamp to int8; KV-cache segments).
 *
 * Conventions for every function below.
 *   Pointers: DEVICE pointers, allocated and freed by the caller, contiguous
 *     row-major, 16-byte aligned.  The library allocates nothing, keeps no
 *     state between calls and may be called from several host threads.
 *   stream: a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; results are ready once the stream is
 *     synchronised.
 *   Sizes: int64_t counts of elements.  M == 0 or N == 0 is a valid empty
 *     problem: nothing is launched and QG_OK is returned.
 *   Errors: arguments are checked on the host before anything is enqueued; a
 *     bad argument returns QG_ERR_NULL / QG_ERR_SHAPE / QG_ERR_ALIGN /
 *     QG_ERR_DTYPE / QG_ERR_ARG and enqueues nothing.  A failed launch returns QG_ERR_HIP.
 *     A device fault surfaces at the caller's next synchronisation.  Inputs
 *     holding NaN or Inf give undefined codes and outputs.
 *   Rounding: quantization decisions use IEEE binary32 with correctly rounded
 *     division and round-half-to-even; outputs are rounded to nearest even.
 *   Packed uint4 format: a weight column n (output channel) stores K codes as
 *     K/8 int32 words, K-contiguous; word i holds k = 8i .. 8i+7, the code of
 *     k = 8i + j in bits 4j .. 4j+3.  Group g covers k in [128g, 128g+128);
 *     its scale and zero point are fp16 values (raw uint16 bits) at [n][g].
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qg_status {
  QG_OK = 0,
  QG_ERR_NULL = 1,   /* a required pointer is NULL                              */
  QG_ERR_SHAPE = 2,  /* a size is negative, zero where not allowed, or breaks a
                        divisibility rule stated below                         */
  QG_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned                        */
  QG_ERR_DTYPE = 4,  /* a dtype argument is not one the function accepts       */
  QG_ERR_HIP = 5,    /* the HIP runtime refused the launch                      */
  QG_ERR_ARG = 6     /* a mode argument is not one the function accepts        */
} qg_status_t;

typedef enum qg_dtype {
  QG_F32 = 0,   /* IEEE binary32                                  */
  QG_F16 = 1,   /* IEEE binary16                                  */
  QG_BF16 = 2,  /* bfloat16 (upper half of a binary32)            */
  QG_I32 = 3    /* int32: raw integer accumulators (test output) */
} qg_dtype_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* qg_status_string(int status);

/* ABI version of this header: 1. */
int qg_abi_version(void);

/*
 * Per-token dynamic symmetric int8 quantization of activations.
 * 「第4章：量化」 §1.3 (per-token, dynamic), §1.2 (symmetric), §1.1;
 * 「LLM推理降本五要素」 §5.2 (round then clamp).
 *   For each row m:  a = max_k |x[m,k]|;  s = a / 127;
 *                    xq[m,k] = clamp(rne(x[m,k] / s), -127, 127);
 *   a row with a == 0 gets s = 0 and all-zero codes.
 * x:        [M][K] of x_dtype (QG_F32, QG_F16 or QG_BF16), read only.
 * xq:       [M][K] int8 codes, written.
 * x_scale:  [M] float scales, written.
 * K must be a positive multiple of 16.
 */
qg_status_t quantize_per_token_i8(const void* x, int x_dtype, int64_t M, int64_t K,
                                  int8_t* xq, float* x_scale, void* stream);

/*
 * Per-output-channel symmetric int8 quantization of a weight matrix (offline).
 * 「第4章：量化」 §1.3 (per-channel), §1.2 (symmetric), §1.1.
 *   For each output channel n:  s = max_k |w[k,n]| / 127;
 *                               wq[n,k] = clamp(rne(w[k,n] / s), -127, 127).
 * w:        [K][N] float (logical W of Y = X W), read only.
 * wq:       [N][K] int8 codes (K-contiguous per output channel), written.
 * w_scale:  [N] float scales, written.
 * K must be a positive multiple of 16.
 */
qg_status_t quantize_weight_i8_per_channel(const float* w, int64_t K, int64_t N,
                                           int8_t* wq, float* w_scale, void* stream);

/*
 * Group-wise asymmetric uint4 quantization of a weight matrix (offline), with
 * groups of 128 consecutive input channels.
 * 「第4章：量化」 §1.1 (round(x/s) + z, rounded before z is added), §1.2
 * (asymmetric, 2^4 - 1 = 15 steps), §1.3 (per-group), §3.2-3.3 (4 bits,
 * group 128, zero point); 「LLM推理降本五要素」 §2.2.
 *   For each output channel n and group g, over its 128 weights:
 *     t = (max - min) / 15 (binary32);  s = the smallest fp16 value >= t;
 *     z = clamp(rne(-min / s), 0, 15);
 *     q = clamp(rne(w / s) + z, 0, 15);
 *   a constant group gets s = 0, z = 0 and q = 0.
 * w:           [K][N] float, read only; (max - min)/15 must fit fp16.
 * wq:          [N][K/8] int32 packed codes (format above), written.
 * w_scale_f16: [N][K/128] fp16 bits of s, written.
 * w_zero_f16:  [N][K/128] fp16 bits of z (an integer 0..15), written.
 * K must be a positive multiple of 128 with K / 128 <= 65535.
 */
qg_status_t quantize_weight_u4_g128(const float* w, int64_t K, int64_t N, int32_t* wq,
                                    uint16_t* w_scale_f16, uint16_t* w_zero_f16,
                                    void* stream);

/*
 * W8A8 GEMM: int8 x int8 -> exact int32 accumulation, then the per-token x
 * per-output-channel scale epilogue.
 * 「第4章：量化」 §2.3 (the GEMM on int8 units), §1.1 (x_hat = x_int s);
 * 「LLM推理降本五要素」 §2.1.
 *   acc[m,n] = sum_k xq[m,k] wq[n,k];   y[m,n] = (acc * x_scale[m]) * w_scale[n]
 * xq [M][K] int8, x_scale [M] float, wq [N][K] int8, w_scale [N] float: read.
 * y: [M][N] of y_dtype, written: QG_F32, QG_BF16 or QG_F16 (the scaled
 *    result), or QG_I32 (acc itself, scales ignored and may be NULL).
 * K must be a positive multiple of 16 (|acc| <= K 127^2 must fit int32, so
 * K <= 133144).  M <= 64 runs a weight-streaming decode kernel, larger M the
 * LDS-tiled matrix-core kernel.
 */
qg_status_t gemm_w8a8(const int8_t* xq, const float* x_scale, const int8_t* wq,
                      const float* w_scale, int64_t M, int64_t N, int64_t K, void* y,
                      int y_dtype, void* stream);

/*
 * Per-token int8 quantization of the activations and the W8A8 GEMM in one
 * call: the results of quantize_per_token_i8 followed by gemm_w8a8, bit for
 * bit (same codes, scales, accumulators and epilogue roundings).
 * 「第4章：量化」 §1.3, §1.2, §1.1, §2.3; 「LLM推理降本五要素」 §2.1, §5.2.
 * x:        [M][K] of x_dtype (QG_F32, QG_F16 or QG_BF16), read only.
 * wq [N][K] int8, w_scale [N] float: read (w_scale unused for QG_I32).
 * y:        [M][N] of y_dtype (QG_F32, QG_BF16, QG_F16 or QG_I32), written.
 * xq [M][K] int8 and x_scale [M] float: written (the activation codes and
 *           scales, as quantize_per_token_i8 writes them).
 * fuse:     QG_FUSE_AUTO, QG_FUSE_NEVER or QG_FUSE_FIT (below).
 * K must be a positive multiple of 16 (K <= 133144).  The fused kernel
 * quantizes the token rows into on-chip memory and runs the product in one
 * launch (no separate quantization pass); it covers M <= 16 and m K <= 32768,
 * m being M rounded up to 1, 2, 4, 8 or 16.  QG_FUSE_FIT runs it on every
 * shape it covers, QG_FUSE_NEVER never, QG_FUSE_AUTO only where it is the
 * faster choice (M <= 4 and N K >= 2^25: a long weight stream, few token
 * rows; or 9 <= M <= 16 with K <= 768); every other case runs the two steps
 * in sequence.  The results do not depend on the choice.  N == 0 computes
 * xq and x_scale only.  quantize_gemm_w8a8_plan tells which form a call
 * takes.
 */
typedef enum qg_fuse {
  QG_FUSE_AUTO = 0,
  QG_FUSE_NEVER = 1,
  QG_FUSE_FIT = 2
} qg_fuse_t;

qg_status_t quantize_gemm_w8a8(const void* x, int x_dtype, const int8_t* wq, const float* w_scale,
                               int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int8_t* xq,
                               float* x_scale, int fuse, void* stream);

/*
 * Which form quantize_gemm_w8a8 takes for these arguments: *fused = 1 for
 * the one-kernel form, 0 for the two kernels in sequence (and for M == 0 or
 * N == 0).  Host only: launches nothing and needs no device.  Returns the
 * status quantize_gemm_w8a8 would return for a bad size, dtype or fuse
 * argument; QG_ERR_NULL when fused is NULL.
 */
qg_status_t quantize_gemm_w8a8_plan(int x_dtype, int64_t M, int64_t N, int64_t K, int fuse,
                                    int* fused);

/*
 * W4A8 GEMM with g=128 uint4 weights unpacked and zero-point corrected inside
 * the kernel (no separate dequantization pass).
 * 「LLM推理降本五要素」 §2.2 (W4A8, group 128, per-group scale and zero);
 * 「第4章：量化」 §1.1, §3.5 (fused dequantization).
 *   acc[m,g,n] = sum_{k in g} xq[m,k] (q[n,k] - z[n,g])   (exact int32)
 *   y[m,n]     = x_scale[m] * sum_g s[n,g] acc[m,g,n]     (binary32)
 * xq [M][K] int8, x_scale [M] float, wq [N][K/8] packed, w_scale_f16 and
 * w_zero_f16 [N][K/128]: read.
 * y: [M][N] of QG_F32, QG_BF16 or QG_F16; or QG_I32, in which case y is
 *    [M][K/128][N] int32 holding acc[m,g,n] (x_scale and w_scale_f16 unused).
 * K must be a positive multiple of 128 with K / 128 <= 65535 (as for
 * quantize_weight_u4_g128).  The int8 matrix cores take the products; one
 * token row with K <= 16384, or two with K <= 4096, take int8 dot products
 * on the vector ALU (the same int32 acc bit for bit).
 */
qg_status_t gemm_w4a8_g128(const int8_t* xq, const float* x_scale, const int32_t* wq,
                           const uint16_t* w_scale_f16, const uint16_t* w_zero_f16,
                           int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                           void* stream);

/*
 * Per-token int8 quantization that also writes a token panel: the codes laid
 * out as the W4A8 kernel's matrix-core operands, and their per-group sums.
 * 「第4章：量化」 §1.1-1.3 (per-token symmetric codes); 「LLM推理降本五要素」
 * §2.2 (W4A8, group 128, zero point: acc = sum xq q - z sum xq needs the
 * token sums per group).
 *   xq, x_scale: as quantize_per_token_i8(x), bit for bit (xq may be NULL:
 *     then only the panel and x_scale are written).
 *   panel: device memory of panel_bytes bytes, 16-byte aligned, owned by the
 *     caller, written (contents on entry ignored).  Layout, for G = K / 128
 *     and m = M rounded up to 1, 2, 4, 8 or 16: bytes [0, 128 m G) hold
 *     16-byte entries [g][h][r][j] (g < G, h < 2, r < m, j < 4), entry =
 *     codes of row r at k = 128 g + 32 j + 16 h + i in the order
 *     i = 0 2 4 6 1 3 5 7 8 10 12 14 9 11 13 15 (the order in which a packed
 *     word's eight codes unpack; rows M..m-1: zeros); bytes
 *     [128 m G, 2048 G) are not used; bytes [2048 G, 2112 G) hold int32
 *     sums [g][16] (row r of group g: sum of its 128 codes; rows >= M: 0).
 * 1 <= M <= 16; K a multiple of 128 with K <= 16384 (else QG_ERR_SHAPE);
 * panel_bytes >= quantize_per_token_i8_panel_bytes(M, K) (else QG_ERR_SHAPE).
 * M == 0: nothing is done.
 */
qg_status_t quantize_per_token_i8_panel(const void* x, int x_dtype, int64_t M, int64_t K,
                                        int8_t* xq, float* x_scale, void* panel,
                                        int64_t panel_bytes, void* stream);

/* Bytes of the token panel for M rows of K: (K / 128) * 2112 for the sizes
 * quantize_per_token_i8_panel takes, else 0.  Host only. */
int64_t quantize_per_token_i8_panel_bytes(int64_t M, int64_t K);

/*
 * W4A8 g=128 GEMM reading the token panel instead of xq.
 * 「LLM推理降本五要素」 §2.2; 「第4章：量化」 §1.1, §3.5.
 *   acc and y exactly as gemm_w4a8_g128(xq, x_scale, ...) for the xq the
 *   panel was written from: acc bit for bit, y within the same rounding
 *   bound (the groups' scaled terms may be summed in another order).
 * panel: written by quantize_per_token_i8_panel with the same M and K, read.
 * x_scale [M], wq, w_scale_f16, w_zero_f16, y, y_dtype: as gemm_w4a8_g128.
 * Sizes as quantize_per_token_i8_panel; N >= 0.
 * The weight rows of each 16-channel block are streamed into on-chip memory
 * by direct buffer-to-LDS loads, every load of a wave issued before the
 * first is used.
 */
qg_status_t gemm_w4a8_g128_panel(const void* panel, int64_t panel_bytes, const float* x_scale,
                                 const int32_t* wq, const uint16_t* w_scale_f16,
                                 const uint16_t* w_zero_f16, int64_t M, int64_t N, int64_t K,
                                 void* y, int y_dtype, void* stream);

/*
 * Per-token int8 quantization of X and the W4A8 g=128 GEMM in one call.
 * 「第4章：量化」 §1.1-1.3 (per-token symmetric codes), §3.5 (dequantize
 * inside the GEMM); 「LLM推理降本五要素」 §2.2 (W4A8, group 128, per-group
 * scale and zero).
 *   xq, x_scale as quantize_per_token_i8(x), bit for bit; y as
 *   gemm_w4a8_g128(xq, x_scale, wq, w_scale_f16, w_zero_f16): the int32
 *   accumulators bit for bit, the scaled outputs within the same rounding
 *   bound (the groups' scaled terms may be summed in another order).
 * x [M][K] of x_dtype (QG_F32, QG_F16 or QG_BF16), wq, w_scale_f16,
 *   w_zero_f16 as gemm_w4a8_g128: read.
 * y: [M][N] of QG_F32, QG_BF16 or QG_F16, or QG_I32 ([M][K/128][N] int32
 *    acc[m,g,n]; w_scale_f16 then unused and may be NULL), written.
 * xq [M][K] int8, x_scale [M] float: written.
 * workspace: device memory of workspace_bytes bytes (16-byte aligned), owned
 *   by the caller; contents on entry ignored, on return unspecified.  Calls
 *   that share a workspace must not overlap.  Its required size is
 *   quantize_gemm_w4a8_g128_workspace_bytes(M, N, K): where that is > 0 the
 *   call runs quantize_per_token_i8_panel then gemm_w4a8_g128_panel with the
 *   workspace as the panel, where it is 0 quantize_per_token_i8 then
 *   gemm_w4a8_g128, and workspace may be NULL.  Smaller than required:
 *   QG_ERR_SHAPE; NULL while required: QG_ERR_NULL.
 * The panel pair runs for 1 <= M <= 16 and K <= 16384 on 4096 < N < 6129
 * (257-383 blocks of 16 output channels); elsewhere the plain kernels
 * measured faster per call (on 384 blocks or more the plain GEMM is the wide
 * kernel, which stages the token rows once per workgroup of several weight
 * blocks).
 * K must be a positive multiple of 128 with K / 128 <= 65535.  N == 0
 * computes xq and x_scale only.
 */
qg_status_t quantize_gemm_w4a8_g128(const void* x, int x_dtype, const int32_t* wq,
                                    const uint16_t* w_scale_f16, const uint16_t* w_zero_f16,
                                    int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                                    int8_t* xq, float* x_scale, void* workspace,
                                    int64_t workspace_bytes, void* stream);

/*
 * Workspace bytes quantize_gemm_w4a8_g128 needs for these sizes: 0 when it
 * runs the two plain kernels (and for sizes it rejects), else
 * quantize_per_token_i8_panel_bytes(M, K).  Host only.
 */
int64_t quantize_gemm_w4a8_g128_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * quantize_gemm_w4a8_g128 for callers that cannot allocate device memory or
 * hand over a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and checks
 * without workspace / workspace_bytes: where the panel pair runs, the panel
 * lives in a fixed array inside the library, 270336 bytes per GPU (the
 * panel of K = 16384), held by each GPU the library runs on until the
 * process ends.  A panel larger than that array is rejected with
 * QG_ERR_SHAPE (no size the panel pair takes needs more).  The call
 * allocates nothing; on its first call on a device it looks up that
 * device's copy of the array (a failure there returns QG_ERR_HIP).  All
 * calls on one GPU share the array: calls that overlap on one GPU (several
 * streams, several host threads) race and must be serialised by the caller.
 */
qg_status_t quantize_gemm_w4a8_g128_noalloc(const void* x, int x_dtype, const int32_t* wq,
                                            const uint16_t* w_scale_f16,
                                            const uint16_t* w_zero_f16, int64_t M, int64_t N,
                                            int64_t K, void* y, int y_dtype, int8_t* xq,
                                            float* x_scale, void* stream);

/*
 * Group-wise (g = 128) uint4 weights with the largest weights of every group
 * kept in an INT8 side store (offline).
 * 「LLM推理降本五要素」 §2.2 (the top 2% of each group by magnitude stored at
 * INT8 precision and computed on a side path); 「第4章：量化」 §1.1-1.3.
 *   For each output channel n and group g: the 3 weights of largest |w|
 *   (2% of 128 rounded up; equal magnitudes go to the lower index) are the
 *   outliers.  Scale, zero point and codes of the other 125 weights follow
 *   quantize_weight_u4_g128; an outlier position gets the code z (it adds
 *   nothing to the 4-bit product).
 *   Per output channel: s8 = max |outlier| / 127 (binary32; 0 if every
 *   outlier is 0) and code = rne(w / s8) in [-127, 127].
 * w:           [K][N] float, read only.
 * wq, w_scale_f16, w_zero_f16: as quantize_weight_u4_g128, written.
 * w_out_rec:   [N][K/128] uint64 records, written: bits 16i..16i+15 hold slot
 *              i = (index in the group << 8) | code byte (two's complement)
 *              for the outliers by ascending index (i = 0, 1, 2); slot 3 is
 *              0xFFFF.
 * w_out_scale: [N] float s8, written.
 * K must be a positive multiple of 128 with K / 128 <= 1279.
 */
qg_status_t quantize_weight_u4_g128_outliers(const float* w, int64_t K, int64_t N, int32_t* wq,
                                             uint16_t* w_scale_f16, uint16_t* w_zero_f16,
                                             uint64_t* w_out_rec, float* w_out_scale,
                                             void* stream);

/*
 * W4A8 GEMM with the INT8 outlier side path fused into the same kernel.
 * 「LLM推理降本五要素」 §2.2; 「第4章：量化」 §1.1, §3.5.
 *   acc[m,g,n] as gemm_w4a8_g128 (outlier positions hold q = z: no term);
 *   acc_o[m,n] = sum over the channel's records of xq[m, 128 g + index] * code
 *                (exact int32);
 *   y[m,n]     = x_scale[m] * (sum_g s[n,g] acc[m,g,n] + s8[n] acc_o[m,n])
 *                (binary32).
 * Arguments as gemm_w4a8_g128 plus w_out_rec [N][K/128] and w_out_scale [N]
 * from quantize_weight_u4_g128_outliers (only slots 0-2 of a record are read).
 * y: [M][N] of QG_F32, QG_BF16 or QG_F16; or QG_I32, in which case y is
 *    [M][K/128 + 1][N] int32: slices 0 .. K/128 - 1 hold acc[m,g,n], the last
 *    holds acc_o[m,n] (x_scale, w_scale_f16 and w_out_scale unused, may be
 *    NULL).
 * K must be a positive multiple of 128 with K / 128 <= 1279.  The kernel
 * streams the weights once per 16 token rows.
 */
qg_status_t gemm_w4a8_g128_outliers(const int8_t* xq, const float* x_scale, const int32_t* wq,
                                    const uint16_t* w_scale_f16, const uint16_t* w_zero_f16,
                                    const uint64_t* w_out_rec, const float* w_out_scale,
                                    int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                                    void* stream);

/*
 * gemm_w4a8_g128_outliers reading the token panel of
 * quantize_per_token_i8_panel instead of xq.
 * 「LLM推理降本五要素」 §2.2 (INT8 outlier side path); 「第4章：量化」 §1.1, §3.5.
 *   acc, acc_o and y exactly as gemm_w4a8_g128_outliers(xq, x_scale, ...)
 *   for the xq the panel was written from: acc and acc_o bit for bit, y
 *   within the same rounding bound.
 * panel: written by quantize_per_token_i8_panel with the same M and K, read;
 *   panel_bytes its size.
 * Other arguments as gemm_w4a8_g128_outliers; sizes as
 * quantize_per_token_i8_panel (1 <= M <= 16, K <= 16384; else QG_ERR_SHAPE);
 * N >= 0.  Measured on MI355X against gemm_w4a8_g128_outliers: 20-27%
 * faster at 1-8 token rows; at 16 rows of K = 11008 slower (14.6 against
 * 12.8 us), where building the outlier operands bounds it.
 */
qg_status_t gemm_w4a8_g128_outliers_panel(const void* panel, int64_t panel_bytes,
                                          const float* x_scale, const int32_t* wq,
                                          const uint16_t* w_scale_f16,
                                          const uint16_t* w_zero_f16, const uint64_t* w_out_rec,
                                          const float* w_out_scale, int64_t M, int64_t N,
                                          int64_t K, void* y, int y_dtype, void* stream);

/*
 * 2:4 structured-sparse uint4 weights (offline): of every 4 consecutive input
 * channels of an output channel the 2 of largest |w| are kept (equal
 * magnitudes to the lower index), and the 64 kept weights of each group of 128
 * inputs are quantized as quantize_weight_u4_g128 does (pruned weights have
 * no code).  「LLM推理降本五要素」 §3.2; 「现代AI加速技术全景解析」 §3.1.
 * w:           [K][N] float, read only.
 * wsp:         [ceil(N/16)][K/128][16][12] int32, written: channels in tiles
 *              of 16 (the last tile's channels past N zero); per (channel,
 *              group) four blocks of 32 inputs, each three words: code words 0
 *              and 1, then a position word.  The block's 16 kept weights in
 *              ascending k are values j = 0..15; value j's code sits in word
 *              j / 8 at bits 8 i .. 8 i + 3 (i = j % 8 < 4) or
 *              8 (i - 4) + 4 .. 8 (i - 4) + 7 (i >= 4); its place within its 4
 *              inputs (0..3) at bits 2 j, 2 j + 1 of the position word.
 * w_scale_f16, w_zero_f16: [N][K/128] fp16 bits, written.
 * K must be a positive multiple of 128.
 */
qg_status_t quantize_weight_u4_g128_sparse24(const float* w, int64_t K, int64_t N, int32_t* wsp,
                                             uint16_t* w_scale_f16, uint16_t* w_zero_f16,
                                             void* stream);

/*
 * W4A8 GEMM on 2:4 sparse uint4 weights, on the sparse int8 matrix cores.
 * 「LLM推理降本五要素」 §3.2; 「第4章：量化」 §1.1.
 *   acc[m,g,n] = sum over the kept k of group g of xq[m,k] (q[n,k] - z[n,g])
 *                (exact int32);
 *   y[m,n]     = x_scale[m] * sum_g s[n,g] acc[m,g,n]   (binary32).
 * xq [M][K] int8, x_scale [M], wsp / w_scale_f16 / w_zero_f16 from
 * quantize_weight_u4_g128_sparse24: read.
 * y: [M][N] of QG_F32, QG_BF16 or QG_F16; or QG_I32: [M][K/128][N] int32
 *    holding acc[m,g,n] (x_scale and w_scale_f16 unused, may be NULL).
 * K must be a positive multiple of 128 with K / 128 <= 1279; M <= 1048560.
 */
qg_status_t gemm_w4a8_g128_sparse24(const int8_t* xq, const float* x_scale, const int32_t* wsp,
                                    const uint16_t* w_scale_f16, const uint16_t* w_zero_f16,
                                    int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                                    void* stream);

/*
 * W4A16 weight-only GEMM: 16-bit float activations, g=128 uint4 weights
 * unpacked to exact (q - z) values in registers and fed to the fp16 (or bf16)
 * matrix cores (one fp16 token row with K <= 4096: to fp16 dot products on
 * the vector ALU instead); each group's binary32 partial sum is then scaled
 * by s.
 * 「第4章：量化」 §3.1 (weight-only 4-bit), §3.5 (fused dequantization);
 * 「Quantization & Flash Attention」 §2.2 (the AWQ-folded weights it serves).
 *   p[m,g,n] = sum_{k in g} x[m,k] (q[n,k] - z[n,g]);  y[m,n] = sum_g s[n,g] p[m,g,n]
 * x: [M][K] of x_dtype, QG_F16 (fp16 matrix cores) or QG_BF16 (bf16).
 * y: [M][N] of y_dtype: QG_F16, QG_BF16 or QG_F32.
 * K must be a positive multiple of 128 with K / 128 <= 65535 (as for
 * quantize_weight_u4_g128).
 */
qg_status_t gemm_w4a16_g128(const void* x, int x_dtype, const int32_t* wq,
                            const uint16_t* w_scale_f16, const uint16_t* w_zero_f16,
                            int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                            void* stream);

/*
 * Offline SmoothQuant fold with alpha = 0.5 (「第4章：量化」 §2.2):
 *   s[j] = sqrt(max_t |x_cal[t,j]|) / sqrt(max_n |w[j,n]|)  (binary32, each
 *          root and the quotient correctly rounded; s = 1 if either max is 0)
 *   w_out[j,n] = s[j] * w[j,n]
 * x_cal [T][K] float (calibration activations), w [K][N] float: read.
 * s [K] float and w_out [K][N] float: written (w_out may equal w).
 * Activations are then divided by s (apply_smoothing).  K % 4 == 0.
 */
qg_status_t smoothquant_fold(const float* x_cal, int64_t T, const float* w, int64_t K,
                             int64_t N, float* s, float* w_out, void* stream);

/*
 * Offline AWQ fold with alpha = 0.5 (「Quantization & Flash Attention」 §2.3):
 *   s[c] = sqrt(mean_t |x_cal[t,c]|), the mean a binary64 sum in token order
 *          divided by T and rounded to binary32, then a binary32 root
 *          (s = 1 if the mean is 0);
 *   w_out[c,n] = s[c] * w[c,n]
 * Arguments as for smoothquant_fold.
 */
qg_status_t awq_fold(const float* x_cal, int64_t T, const float* w, int64_t K, int64_t N,
                     float* s, float* w_out, void* stream);

/*
 * Divide activation columns by a fold's scales: x_out[m,j] = x[m,j] / s[j]
 * (binary32, correctly rounded), stored as out_dtype (QG_F32, QG_F16 or
 * QG_BF16, round to nearest even).  x [M][K] float, s [K]: read.  K % 4 == 0.
 * (「第4章：量化」 §2.2: X diag(s)^-1.)
 */
qg_status_t apply_smoothing(const float* x, int64_t M, int64_t K, const float* s,
                            void* x_out, int out_dtype, void* stream);

/*
 * KV-cache INT8 quantization in position segments of 128 with one scale per
 * (kv head, segment, head-dim channel).
 * 「LLM推理降本五要素」 §5.2 (segments of 128 positions, per-channel scales,
 * round then clamp to int8); 「第4章：量化」 §1.2 (symmetric s = max|x|/127),
 * §1.1; 「现代AI加速技术全景解析」 §5.2 (the cache grouped in blocks of 128
 * positions, [L/G][G][H][D]).
 *   For each head h, segment g (positions [128g, min(T, 128g + 128))) and
 *   channel d:  a = max_t |kv[t,h,d]|;  s = a / 127;
 *               kv_q[t,h,d] = clamp(rne(kv[t,h,d] / s), -127, 127);
 *   a channel with a == 0 in a segment gets s = 0 and zero codes.  A last,
 *   partial segment is quantized over the positions it has.
 * kv:       [T][H][D] of kv_dtype (QG_F32, QG_F16 or QG_BF16), read only;
 *           position-major, the layout in which a cache grows.
 * kv_q:     [T][H][D] int8 codes, written.
 * kv_scale: [H][ceil(T/128)][D] float scales, written.
 * T >= 0 (T == 0: nothing is launched); H >= 1; D a multiple of 16 in
 * [16, 256]; H * D <= 2^22.  One layer of one sequence per call.
 * The per-token variant (one scale per position and head) is
 * quantize_per_token_i8 on kv viewed as [T*H][D].
 */
qg_status_t quantize_kv_i8_segments(const void* kv, int kv_dtype, int64_t T, int64_t H,
                                    int64_t D, int8_t* kv_q, float* kv_scale, void* stream);

/*
 * Dequantization of a segment-quantized KV cache (「第4章：量化」 §1.1,
 * x_hat = x_int * s):  out[t,h,d] = kv_q[t,h,d] * kv_scale[h, t/128, d],
 * the product rounded to binary32, then to out_dtype (QG_F32, QG_F16 or
 * QG_BF16, round to nearest even).  Shapes and rules as for
 * quantize_kv_i8_segments; out is [T][H][D], written.
 */
qg_status_t dequantize_kv_i8_segments(const int8_t* kv_q, const float* kv_scale, int64_t T,
                                      int64_t H, int64_t D, void* out, int out_dtype,
                                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
