// C ABI of the library (declared in include/qgemm.h): host-side argument
// checks, then one launcher per entry point.  Nothing here allocates device
// memory or synchronises the stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qgemm.h"
#include "qg_launch.hpp"

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline qg_status_t hip_status(hipError_t e) { return e == hipSuccess ? QG_OK : QG_ERR_HIP; }

inline bool is_float_dtype(int d) { return d == QG_F32 || d == QG_F16 || d == QG_BF16; }

// Largest K for which K * 127 * 127 still fits int32.
constexpr int64_t kMaxK8 = 2147483647LL / (127 * 127);
constexpr int64_t kMaxDim = 2147483647LL;
// Groups per row of the g=128 uint4 paths (what the weight quantizer
// produces); the kernels' 32-bit buffer offsets are sized for this.
constexpr int64_t kMaxGroups = 65535;
// Groups per row of the outlier-retention and 2:4 sparse paths: their kernels
// stage a 16-row block's scales and zero points in 80 KB of LDS
// (16 x (G + 1) words).
constexpr int64_t kMaxOutlierGroups = 1279;

qg_status_t check_dims(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return QG_ERR_SHAPE;
  return QG_OK;
}

// KV cache [T][H][D]: T >= 0 positions, H >= 1 heads, D a multiple of 16 in
// [16, 256], H * D <= 2^22 (a 128-position segment then spans less than
// 2^31 bytes, the reach of the kernels' 32-bit buffer offsets).
qg_status_t check_kv_dims(int64_t T, int64_t H, int64_t D) {
  if (T < 0 || T > kMaxDim || H < 1 || D < 16 || D > 256 || D % 16) return QG_ERR_SHAPE;
  if (H * D > ((int64_t)1 << 22)) return QG_ERR_SHAPE;
  return QG_OK;
}

}  // namespace

extern "C" {

const char* qg_status_string(int status) {
  switch (status) {
    case QG_OK: return "QG_OK";
    case QG_ERR_NULL: return "QG_ERR_NULL: a required pointer is NULL";
    case QG_ERR_SHAPE: return "QG_ERR_SHAPE: a size is out of range or breaks a divisibility rule";
    case QG_ERR_ALIGN: return "QG_ERR_ALIGN: a pointer is not 16-byte aligned";
    case QG_ERR_DTYPE: return "QG_ERR_DTYPE: unsupported dtype for this function";
    case QG_ERR_HIP: return "QG_ERR_HIP: the HIP runtime refused the launch";
    case QG_ERR_ARG: return "QG_ERR_ARG: unsupported mode argument for this function";
    default: return "unknown qg status";
  }
}

int qg_abi_version(void) { return 1; }

qg_status_t quantize_per_token_i8(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* xq,
                                  float* x_scale, void* stream) {
  if (qg_status_t s = check_dims(M, 1, K)) return s;
  if (K % 16) return QG_ERR_SHAPE;
  if (!is_float_dtype(x_dtype)) return QG_ERR_DTYPE;
  if (M == 0) return QG_OK;
  if (!x || !xq || !x_scale) return QG_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_quant_per_token(x, x_dtype, M, K, xq, x_scale,
                                               static_cast<hipStream_t>(stream)));
}

qg_status_t quantize_weight_i8_per_channel(const float* w, int64_t K, int64_t N, int8_t* wq,
                                           float* w_scale, void* stream) {
  if (qg_status_t s = check_dims(1, N, K)) return s;
  if (K % 16) return QG_ERR_SHAPE;
  if (N == 0) return QG_OK;
  if (!w || !wq || !w_scale) return QG_ERR_NULL;
  if (!aligned16(w) || !aligned16(wq)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_quant_weight_i8(w, K, N, wq, w_scale, static_cast<hipStream_t>(stream)));
}

qg_status_t quantize_weight_u4_g128(const float* w, int64_t K, int64_t N, int32_t* wq,
                                    uint16_t* w_scale_f16, uint16_t* w_zero_f16, void* stream) {
  if (qg_status_t s = check_dims(1, N, K)) return s;
  if (K % 128 || K / 128 > kMaxGroups) return QG_ERR_SHAPE;
  if (N == 0) return QG_OK;
  if (!w || !wq || !w_scale_f16 || !w_zero_f16) return QG_ERR_NULL;
  if (!aligned16(w) || !aligned16(wq)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_quant_weight_u4(w, K, N, wq, w_scale_f16, w_zero_f16,
                                               static_cast<hipStream_t>(stream)));
}

qg_status_t gemm_w8a8(const int8_t* xq, const float* x_scale, const int8_t* wq,
                      const float* w_scale, int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                      void* stream) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (K % 16 || K > kMaxK8) return QG_ERR_SHAPE;
  if (!is_float_dtype(y_dtype) && y_dtype != QG_I32) return QG_ERR_DTYPE;
  if (M == 0 || N == 0) return QG_OK;
  if (!xq || !wq || !y) return QG_ERR_NULL;
  if (y_dtype != QG_I32 && (!x_scale || !w_scale)) return QG_ERR_NULL;
  if (!aligned16(xq) || !aligned16(wq)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_gemm_w8a8(xq, x_scale, wq, w_scale, M, N, K, y, y_dtype,
                                         static_cast<hipStream_t>(stream)));
}

qg_status_t quantize_gemm_w8a8(const void* x, int x_dtype, const int8_t* wq, const float* w_scale,
                               int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int8_t* xq,
                               float* x_scale, int fuse, void* stream) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (K % 16 || K > kMaxK8) return QG_ERR_SHAPE;
  if (fuse != QG_FUSE_AUTO && fuse != QG_FUSE_NEVER && fuse != QG_FUSE_FIT) return QG_ERR_ARG;
  if (!is_float_dtype(x_dtype)) return QG_ERR_DTYPE;
  if (!is_float_dtype(y_dtype) && y_dtype != QG_I32) return QG_ERR_DTYPE;
  if (M == 0) return QG_OK;
  if (!x || !xq || !x_scale) return QG_ERR_NULL;
  if (N > 0 && (!wq || !y || (y_dtype != QG_I32 && !w_scale))) return QG_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq) || (N > 0 && !aligned16(wq))) return QG_ERR_ALIGN;
  if (N == 0)   // nothing to multiply: the codes and scales alone
    return hip_status(qg::launch_quant_per_token(x, x_dtype, M, K, xq, x_scale,
                                                 static_cast<hipStream_t>(stream)));
  return hip_status(qg::launch_quantize_gemm_w8a8(x, x_dtype, wq, w_scale, M, N, K, y, y_dtype,
                                                  xq, x_scale, fuse,
                                                  static_cast<hipStream_t>(stream)));
}

qg_status_t quantize_gemm_w8a8_plan(int x_dtype, int64_t M, int64_t N, int64_t K, int fuse,
                                    int* fused) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (K % 16 || K > kMaxK8) return QG_ERR_SHAPE;
  if (fuse != QG_FUSE_AUTO && fuse != QG_FUSE_NEVER && fuse != QG_FUSE_FIT) return QG_ERR_ARG;
  if (!is_float_dtype(x_dtype)) return QG_ERR_DTYPE;
  if (!fused) return QG_ERR_NULL;
  *fused = qg::quantize_gemm_w8a8_fused(x_dtype, M, N, K, fuse) ? 1 : 0;
  return QG_OK;
}

qg_status_t gemm_w4a8_g128(const int8_t* xq, const float* x_scale, const int32_t* wq,
                           const uint16_t* w_scale_f16, const uint16_t* w_zero_f16, int64_t M,
                           int64_t N, int64_t K, void* y, int y_dtype, void* stream) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (K % 128 || K / 128 > kMaxGroups) return QG_ERR_SHAPE;
  if (y_dtype == QG_I32 && M * (K / 128) * N > kMaxDim) return QG_ERR_SHAPE;
  if (!is_float_dtype(y_dtype) && y_dtype != QG_I32) return QG_ERR_DTYPE;
  if (M == 0 || N == 0) return QG_OK;
  if (!xq || !wq || !w_zero_f16 || !y) return QG_ERR_NULL;
  if (y_dtype != QG_I32 && (!x_scale || !w_scale_f16)) return QG_ERR_NULL;
  if (!aligned16(xq) || !aligned16(wq)) return QG_ERR_ALIGN;
  // the kernel reads the scales unconditionally; in I32 mode point them at
  // the zero points (same shape, values unused)
  const uint16_t* ws = w_scale_f16 ? w_scale_f16 : w_zero_f16;
  return hip_status(qg::launch_gemm_w4a8(xq, x_scale, wq, ws, w_zero_f16, M, N, K, y, y_dtype,
                                         static_cast<hipStream_t>(stream)));
}

int64_t quantize_per_token_i8_panel_bytes(int64_t M, int64_t K) {
  if (check_dims(M, 1, K)) return 0;
  return qg::panel_bytes(M, K);
}

qg_status_t quantize_per_token_i8_panel(const void* x, int x_dtype, int64_t M, int64_t K,
                                        int8_t* xq, float* x_scale, void* panel,
                                        int64_t panel_bytes, void* stream) {
  if (qg_status_t s = check_dims(M, 1, K)) return s;
  if (!is_float_dtype(x_dtype)) return QG_ERR_DTYPE;
  if (M == 0) return QG_OK;
  const int64_t need = qg::panel_bytes(M, K);
  if (need == 0 || panel_bytes < need) return QG_ERR_SHAPE;
  if (!x || !x_scale || !panel) return QG_ERR_NULL;
  if (!aligned16(x) || (xq && !aligned16(xq)) || !aligned16(panel)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_quant_panel(x, x_dtype, M, K, xq, x_scale, panel,
                                           static_cast<hipStream_t>(stream)));
}

qg_status_t gemm_w4a8_g128_panel(const void* panel, int64_t panel_bytes, const float* x_scale,
                                 const int32_t* wq, const uint16_t* w_scale_f16,
                                 const uint16_t* w_zero_f16, int64_t M, int64_t N, int64_t K,
                                 void* y, int y_dtype, void* stream) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (!is_float_dtype(y_dtype) && y_dtype != QG_I32) return QG_ERR_DTYPE;
  if (M == 0 || N == 0) return QG_OK;
  const int64_t need = qg::panel_bytes(M, K);
  if (need == 0 || panel_bytes < need || !qg::gemm_w4a8_panel_ok(M, N, K)) return QG_ERR_SHAPE;
  if (y_dtype == QG_I32 && M * (K / 128) * N > kMaxDim) return QG_ERR_SHAPE;
  if (!panel || !wq || !w_zero_f16 || !y) return QG_ERR_NULL;
  if (y_dtype != QG_I32 && (!x_scale || !w_scale_f16)) return QG_ERR_NULL;
  if (!aligned16(panel) || !aligned16(wq)) return QG_ERR_ALIGN;
  const uint16_t* ws = w_scale_f16 ? w_scale_f16 : w_zero_f16;   // I32: values unused
  return hip_status(qg::launch_gemm_w4a8_panel(panel, x_scale, wq, ws, w_zero_f16, M, N, K, y,
                                               y_dtype, static_cast<hipStream_t>(stream)));
}

int64_t quantize_gemm_w4a8_g128_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_dims(M, N, K) || K % 128 || K / 128 > kMaxGroups) return 0;
  return qg::quantize_gemm_w4a8_workspace(M, N, K);
}

qg_status_t quantize_gemm_w4a8_g128(const void* x, int x_dtype, const int32_t* wq,
                                    const uint16_t* w_scale_f16, const uint16_t* w_zero_f16,
                                    int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                                    int8_t* xq, float* x_scale, void* workspace,
                                    int64_t workspace_bytes, void* stream) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (K % 128 || K / 128 > kMaxGroups) return QG_ERR_SHAPE;
  if (y_dtype == QG_I32 && M * (K / 128) * N > kMaxDim) return QG_ERR_SHAPE;
  if (!is_float_dtype(x_dtype)) return QG_ERR_DTYPE;
  if (!is_float_dtype(y_dtype) && y_dtype != QG_I32) return QG_ERR_DTYPE;
  if (workspace_bytes < 0) return QG_ERR_SHAPE;
  if (M == 0) return QG_OK;
  const int64_t need = N > 0 ? qg::quantize_gemm_w4a8_workspace(M, N, K) : 0;
  if (workspace_bytes < need) return QG_ERR_SHAPE;
  if (!x || !xq || !x_scale) return QG_ERR_NULL;
  if (N > 0 && (!wq || !w_zero_f16 || !y || (y_dtype != QG_I32 && !w_scale_f16)))
    return QG_ERR_NULL;
  if (need > 0 && !workspace) return QG_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq) || (N > 0 && !aligned16(wq)) ||
      (need > 0 && !aligned16(workspace)))
    return QG_ERR_ALIGN;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (N == 0) return hip_status(qg::launch_quant_per_token(x, x_dtype, M, K, xq, x_scale, st));
  const uint16_t* ws = w_scale_f16 ? w_scale_f16 : w_zero_f16;   // I32: values unused
  return hip_status(qg::launch_quantize_gemm_w4a8(x, x_dtype, wq, ws, w_zero_f16, M, N, K, y,
                                                  y_dtype, xq, x_scale, workspace, st));
}

qg_status_t quantize_gemm_w4a8_g128_noalloc(const void* x, int x_dtype, const int32_t* wq,
                                            const uint16_t* w_scale_f16,
                                            const uint16_t* w_zero_f16, int64_t M, int64_t N,
                                            int64_t K, void* y, int y_dtype, int8_t* xq,
                                            float* x_scale, void* stream) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (K % 128 || K / 128 > kMaxGroups) return QG_ERR_SHAPE;
  if (y_dtype == QG_I32 && M * (K / 128) * N > kMaxDim) return QG_ERR_SHAPE;
  if (!is_float_dtype(x_dtype)) return QG_ERR_DTYPE;
  if (!is_float_dtype(y_dtype) && y_dtype != QG_I32) return QG_ERR_DTYPE;
  if (M == 0) return QG_OK;
  // the panel the call needs must fit the library's array
  if (N > 0 && qg::quantize_gemm_w4a8_workspace(M, N, K) > qg::noalloc_scratch_bytes())
    return QG_ERR_SHAPE;
  if (!x || !xq || !x_scale) return QG_ERR_NULL;
  if (N > 0 && (!wq || !w_zero_f16 || !y || (y_dtype != QG_I32 && !w_scale_f16)))
    return QG_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq) || (N > 0 && !aligned16(wq))) return QG_ERR_ALIGN;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (N == 0) return hip_status(qg::launch_quant_per_token(x, x_dtype, M, K, xq, x_scale, st));
  const uint16_t* ws = w_scale_f16 ? w_scale_f16 : w_zero_f16;   // I32: values unused
  return hip_status(qg::launch_quantize_gemm_w4a8_noalloc(x, x_dtype, wq, ws, w_zero_f16, M, N,
                                                          K, y, y_dtype, xq, x_scale, st));
}

qg_status_t quantize_weight_u4_g128_outliers(const float* w, int64_t K, int64_t N, int32_t* wq,
                                             uint16_t* w_scale_f16, uint16_t* w_zero_f16,
                                             uint64_t* w_out_rec, float* w_out_scale,
                                             void* stream) {
  if (qg_status_t s = check_dims(1, N, K)) return s;
  if (K % 128 || K / 128 > kMaxOutlierGroups) return QG_ERR_SHAPE;
  if (N == 0) return QG_OK;
  if (!w || !wq || !w_scale_f16 || !w_zero_f16 || !w_out_rec || !w_out_scale) return QG_ERR_NULL;
  if (!aligned16(w) || !aligned16(wq) || !aligned16(w_out_rec)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_quant_weight_u4_outl(w, K, N, wq, w_scale_f16, w_zero_f16,
                                                    w_out_rec, w_out_scale,
                                                    static_cast<hipStream_t>(stream)));
}

qg_status_t gemm_w4a8_g128_outliers(const int8_t* xq, const float* x_scale, const int32_t* wq,
                                    const uint16_t* w_scale_f16, const uint16_t* w_zero_f16,
                                    const uint64_t* w_out_rec, const float* w_out_scale,
                                    int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                                    void* stream) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (K % 128 || K / 128 > kMaxOutlierGroups) return QG_ERR_SHAPE;
  if (y_dtype == QG_I32 && M * (K / 128 + 1) * N > kMaxDim) return QG_ERR_SHAPE;
  if (!is_float_dtype(y_dtype) && y_dtype != QG_I32) return QG_ERR_DTYPE;
  if (M == 0 || N == 0) return QG_OK;
  if (!xq || !wq || !w_zero_f16 || !w_out_rec || !y) return QG_ERR_NULL;
  if (y_dtype != QG_I32 && (!x_scale || !w_scale_f16 || !w_out_scale)) return QG_ERR_NULL;
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(w_out_rec)) return QG_ERR_ALIGN;
  const uint16_t* ws = w_scale_f16 ? w_scale_f16 : w_zero_f16;   // read, unused in I32 mode
  return hip_status(qg::launch_gemm_w4a8_outl(xq, x_scale, wq, ws, w_zero_f16, w_out_rec,
                                              w_out_scale, M, N, K, y, y_dtype,
                                              static_cast<hipStream_t>(stream)));
}

qg_status_t gemm_w4a8_g128_outliers_panel(const void* panel, int64_t panel_bytes,
                                          const float* x_scale, const int32_t* wq,
                                          const uint16_t* w_scale_f16,
                                          const uint16_t* w_zero_f16, const uint64_t* w_out_rec,
                                          const float* w_out_scale, int64_t M, int64_t N,
                                          int64_t K, void* y, int y_dtype, void* stream) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (!is_float_dtype(y_dtype) && y_dtype != QG_I32) return QG_ERR_DTYPE;
  if (M == 0 || N == 0) return QG_OK;
  const int64_t need = qg::panel_bytes(M, K);
  if (need == 0 || panel_bytes < need || !qg::gemm_w4a8_panel_ok(M, N, K)) return QG_ERR_SHAPE;
  if (y_dtype == QG_I32 && M * (K / 128 + 1) * N > kMaxDim) return QG_ERR_SHAPE;
  if (!panel || !wq || !w_zero_f16 || !w_out_rec || !y) return QG_ERR_NULL;
  if (y_dtype != QG_I32 && (!x_scale || !w_scale_f16 || !w_out_scale)) return QG_ERR_NULL;
  if (!aligned16(panel) || !aligned16(wq) || !aligned16(w_out_rec)) return QG_ERR_ALIGN;
  const uint16_t* ws = w_scale_f16 ? w_scale_f16 : w_zero_f16;   // I32: values unused
  return hip_status(qg::launch_gemm_w4a8_outl_panel(panel, x_scale, wq, ws, w_zero_f16, w_out_rec,
                                                    w_out_scale, M, N, K, y, y_dtype,
                                                    static_cast<hipStream_t>(stream)));
}

qg_status_t quantize_weight_u4_g128_sparse24(const float* w, int64_t K, int64_t N, int32_t* wsp,
                                             uint16_t* w_scale_f16, uint16_t* w_zero_f16,
                                             void* stream) {
  if (qg_status_t s = check_dims(1, N, K)) return s;
  if (K % 128 || K / 128 > kMaxGroups) return QG_ERR_SHAPE;
  if (N == 0) return QG_OK;
  if (!w || !wsp || !w_scale_f16 || !w_zero_f16) return QG_ERR_NULL;
  if (!aligned16(w) || !aligned16(wsp)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_quant_weight_u4_sp24(w, K, N, wsp, w_scale_f16, w_zero_f16,
                                                    static_cast<hipStream_t>(stream)));
}

qg_status_t gemm_w4a8_g128_sparse24(const int8_t* xq, const float* x_scale, const int32_t* wsp,
                                    const uint16_t* w_scale_f16, const uint16_t* w_zero_f16,
                                    int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                                    void* stream) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (K % 128 || K / 128 > kMaxOutlierGroups) return QG_ERR_SHAPE;
  if (M > 16 * 65535) return QG_ERR_SHAPE;
  if (y_dtype == QG_I32 && M * (K / 128) * N > kMaxDim) return QG_ERR_SHAPE;
  if (!is_float_dtype(y_dtype) && y_dtype != QG_I32) return QG_ERR_DTYPE;
  if (M == 0 || N == 0) return QG_OK;
  if (!xq || !wsp || !w_zero_f16 || !y) return QG_ERR_NULL;
  if (y_dtype != QG_I32 && (!x_scale || !w_scale_f16)) return QG_ERR_NULL;
  if (!aligned16(xq) || !aligned16(wsp)) return QG_ERR_ALIGN;
  const uint16_t* ws = w_scale_f16 ? w_scale_f16 : w_zero_f16;   // read, unused in I32 mode
  return hip_status(qg::launch_gemm_w4a8_sp24(xq, x_scale, wsp, ws, w_zero_f16, M, N, K, y,
                                              y_dtype, static_cast<hipStream_t>(stream)));
}

qg_status_t gemm_w4a16_g128(const void* x, int x_dtype, const int32_t* wq,
                            const uint16_t* w_scale_f16, const uint16_t* w_zero_f16, int64_t M,
                            int64_t N, int64_t K, void* y, int y_dtype, void* stream) {
  if (qg_status_t s = check_dims(M, N, K)) return s;
  if (K % 128 || K / 128 > kMaxGroups) return QG_ERR_SHAPE;
  if (x_dtype != QG_F16 && x_dtype != QG_BF16) return QG_ERR_DTYPE;
  if (!is_float_dtype(y_dtype)) return QG_ERR_DTYPE;
  if (M == 0 || N == 0) return QG_OK;
  if (!x || !wq || !w_scale_f16 || !w_zero_f16 || !y) return QG_ERR_NULL;
  if (!aligned16(x) || !aligned16(wq)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_gemm_w4a16(x, x_dtype, wq, w_scale_f16, w_zero_f16, M, N, K, y,
                                          y_dtype, static_cast<hipStream_t>(stream)));
}

qg_status_t smoothquant_fold(const float* x_cal, int64_t T, const float* w, int64_t K, int64_t N,
                             float* s, float* w_out, void* stream) {
  if (T <= 0 || N < 0 || K <= 0 || T > kMaxDim || K > kMaxDim || N > kMaxDim) return QG_ERR_SHAPE;
  if (K % 4) return QG_ERR_SHAPE;
  if (!x_cal || !w || !s || !w_out) return QG_ERR_NULL;
  return hip_status(qg::launch_smoothquant_fold(x_cal, T, w, K, N, s, w_out,
                                                static_cast<hipStream_t>(stream)));
}

qg_status_t awq_fold(const float* x_cal, int64_t T, const float* w, int64_t K, int64_t N, float* s,
                     float* w_out, void* stream) {
  if (T <= 0 || N < 0 || K <= 0 || T > kMaxDim || K > kMaxDim || N > kMaxDim) return QG_ERR_SHAPE;
  if (K % 4) return QG_ERR_SHAPE;
  if (!x_cal || !w || !s || !w_out) return QG_ERR_NULL;
  return hip_status(qg::launch_awq_fold(x_cal, T, w, K, N, s, w_out, static_cast<hipStream_t>(stream)));
}

qg_status_t apply_smoothing(const float* x, int64_t M, int64_t K, const float* s, void* x_out,
                            int out_dtype, void* stream) {
  if (M < 0 || K <= 0 || M > kMaxDim || K > kMaxDim) return QG_ERR_SHAPE;
  if (K % 4) return QG_ERR_SHAPE;
  if (!is_float_dtype(out_dtype)) return QG_ERR_DTYPE;
  if (M == 0) return QG_OK;
  if (!x || !s || !x_out) return QG_ERR_NULL;
  return hip_status(qg::launch_apply_smoothing(x, M, K, s, x_out, out_dtype,
                                               static_cast<hipStream_t>(stream)));
}

qg_status_t quantize_kv_i8_segments(const void* kv, int kv_dtype, int64_t T, int64_t H, int64_t D,
                                    int8_t* kv_q, float* kv_scale, void* stream) {
  if (qg_status_t s = check_kv_dims(T, H, D)) return s;
  if (!is_float_dtype(kv_dtype)) return QG_ERR_DTYPE;
  if (T == 0) return QG_OK;
  if (!kv || !kv_q || !kv_scale) return QG_ERR_NULL;
  if (!aligned16(kv) || !aligned16(kv_q) || !aligned16(kv_scale)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_kv_quant_seg(kv, kv_dtype, T, H, D, kv_q, kv_scale,
                                            static_cast<hipStream_t>(stream)));
}

qg_status_t dequantize_kv_i8_segments(const int8_t* kv_q, const float* kv_scale, int64_t T,
                                      int64_t H, int64_t D, void* out, int out_dtype,
                                      void* stream) {
  if (qg_status_t s = check_kv_dims(T, H, D)) return s;
  if (!is_float_dtype(out_dtype)) return QG_ERR_DTYPE;
  if (T == 0) return QG_OK;
  if (!kv_q || !kv_scale || !out) return QG_ERR_NULL;
  if (!aligned16(kv_q) || !aligned16(kv_scale) || !aligned16(out)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_kv_dequant_seg(kv_q, kv_scale, T, H, D, out, out_dtype,
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"
