// Internal launchers: one per C-ABI entry point.  Arguments are already
// validated by api.hip; each launcher only picks a kernel variant and
// enqueues it on the stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

enum DType { F32 = 0, F16 = 1, BF16 = 2, I32 = 3 };
// fused quantize + W8A8 policy (values of the C interface's qg_fuse)
enum Fuse { kFuseAuto = 0, kFuseNever = 1, kFuseFit = 2 };

hipError_t launch_quant_per_token(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* xq,
                                  float* x_scale, hipStream_t st);
hipError_t launch_quant_weight_i8(const float* w, int64_t K, int64_t N, int8_t* wq, float* ws,
                                  hipStream_t st);
hipError_t launch_quant_weight_u4(const float* w, int64_t K, int64_t N, int32_t* wq,
                                  uint16_t* ws, uint16_t* wz, hipStream_t st);
hipError_t launch_gemm_w8a8(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws,
                            int64_t M, int64_t N, int64_t K, void* y, int y_dtype, hipStream_t st);
hipError_t launch_quantize_gemm_w8a8(const void* x, int x_dtype, const int8_t* wq,
                                     const float* ws, int64_t M, int64_t N, int64_t K, void* y,
                                     int y_dtype, int8_t* xq, float* xs, int fuse,
                                     hipStream_t st);
// Whether launch_quantize_gemm_w8a8 with these arguments runs the one-kernel
// form (host only).
bool quantize_gemm_w8a8_fused(int x_dtype, int64_t M, int64_t N, int64_t K, int fuse);
hipError_t launch_gemm_w4a8(const int8_t* xq, const float* xs, const int32_t* wq,
                            const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                            int64_t K, void* y, int y_dtype, hipStream_t st);
// Token panel of per-token int8 codes (operand order + per-group sums) for
// the W4A8 panel GEMM: its bytes for M rows of K (0 where unsupported), the
// quantizer writing it (xq may be NULL), the GEMM reading it.
int64_t panel_bytes(int64_t M, int64_t K);
bool gemm_w4a8_panel_ok(int64_t M, int64_t N, int64_t K);
hipError_t launch_quant_panel(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* xq,
                              float* xs, void* panel, hipStream_t st);
hipError_t launch_gemm_w4a8_panel(const void* panel, const float* xs, const int32_t* wq,
                                  const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                                  int64_t K, void* y, int y_dtype, hipStream_t st);
hipError_t launch_gemm_w4a8_outl_panel(const void* panel, const float* xs, const int32_t* wq,
                                       const uint16_t* ws, const uint16_t* wz,
                                       const uint64_t* orec, const float* os8, int64_t M,
                                       int64_t N, int64_t K, void* y, int y_dtype,
                                       hipStream_t st);
// Quantize + W4A8: the panel pair where quantize_gemm_w4a8_workspace > 0
// (workspace of that size), else the two plain kernels in sequence.
hipError_t launch_quantize_gemm_w4a8(const void* x, int x_dtype, const int32_t* wq,
                                     const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                                     int64_t K, void* y, int y_dtype, int8_t* xq, float* xs,
                                     void* workspace, hipStream_t st);
int64_t quantize_gemm_w4a8_workspace(int64_t M, int64_t N, int64_t K);
// The same with the library's own per-device panel array (no allocation,
// no workspace argument), and that array's size.
hipError_t launch_quantize_gemm_w4a8_noalloc(const void* x, int x_dtype, const int32_t* wq,
                                             const uint16_t* ws, const uint16_t* wz, int64_t M,
                                             int64_t N, int64_t K, void* y, int y_dtype,
                                             int8_t* xq, float* xs, hipStream_t st);
int64_t noalloc_scratch_bytes();
hipError_t launch_quant_weight_u4_outl(const float* w, int64_t K, int64_t N, int32_t* wq,
                                       uint16_t* ws, uint16_t* wz, uint64_t* rec, float* s8,
                                       hipStream_t st);
hipError_t launch_gemm_w4a8_outl(const int8_t* xq, const float* xs, const int32_t* wq,
                                 const uint16_t* ws, const uint16_t* wz, const uint64_t* orec,
                                 const float* os8, int64_t M, int64_t N, int64_t K, void* y,
                                 int y_dtype, hipStream_t st);
hipError_t launch_quant_weight_u4_sp24(const float* w, int64_t K, int64_t N, int32_t* wsp,
                                       uint16_t* ws, uint16_t* wz, hipStream_t st);
hipError_t launch_gemm_w4a8_sp24(const int8_t* xq, const float* xs, const int32_t* wsp,
                                 const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                                 int64_t K, void* y, int y_dtype, hipStream_t st);
hipError_t launch_gemm_w4a16(const void* x, int x_dtype, const int32_t* wq, const uint16_t* ws,
                             const uint16_t* wz, int64_t M, int64_t N, int64_t K, void* y,
                             int y_dtype, hipStream_t st);
hipError_t launch_smoothquant_fold(const float* x_cal, int64_t T, const float* w, int64_t K,
                                   int64_t N, float* s, float* w_out, hipStream_t st);
hipError_t launch_awq_fold(const float* x_cal, int64_t T, const float* w, int64_t K, int64_t N,
                           float* s, float* w_out, hipStream_t st);
hipError_t launch_apply_smoothing(const float* x, int64_t M, int64_t K, const float* s,
                                  void* x_out, int out_dtype, hipStream_t st);
hipError_t launch_kv_quant_seg(const void* kv, int kv_dtype, int64_t T, int64_t H, int64_t D,
                               int8_t* kv_q, float* kv_scale, hipStream_t st);
hipError_t launch_kv_dequant_seg(const int8_t* kv_q, const float* kv_scale, int64_t T, int64_t H,
                                 int64_t D, void* out, int out_dtype, hipStream_t st);

}  // namespace qg
