// Offline smoothing folds, alpha = 0.5: Y = X W = (X diag(s)^-1)(diag(s) W).
// 「第4章：量化」 §2.2 (SmoothQuant: s_j = max|X_j|^a / max|W_j|^(1-a));
// 「Quantization & Flash Attention」 §2.2-2.3 (AWQ: s_c = mean|X_c|^a).
#include "qg_device.hpp"
#include "qg_launch.hpp"

namespace qg {

// a_j = max_t |x_cal[t, j]|: one thread per column, coalesced along K.
__global__ __launch_bounds__(256) void k_col_absmax(const float* __restrict__ x, int64_t T,
                                                    int64_t K, float* __restrict__ out) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= K) return;
  float a = 0.f;
  for (int64_t t = 0; t < T; ++t) a = fmaxf(a, fabsf(x[t * K + j]));
  out[j] = a;
}

// One workgroup per weight row j: b_j = max_n |w[j, n]|, then
// s_j = sqrt(a_j) / sqrt(b_j) (s holds a_j on entry), then w_out[j, :] = s_j w[j, :].
__global__ __launch_bounds__(256) void k_smoothquant_rows(const float* __restrict__ w, int64_t N,
                                                          float* __restrict__ s,
                                                          float* __restrict__ w_out) {
  __shared__ float red[4];
  const int64_t j = blockIdx.x;
  const float* wr = w + j * N;
  const float a = s[j];
  float b = 0.f;
  for (int64_t n = threadIdx.x; n < N; n += 256) b = fmaxf(b, fabsf(wr[n]));
  b = block_max<256>(b, red);
  const float sj = (a > 0.f && b > 0.f) ? __builtin_sqrtf(a) / __builtin_sqrtf(b) : 1.f;
  __syncthreads();  // every thread has read s[j]
  if (threadIdx.x == 0) s[j] = sj;
  float* orow = w_out + j * N;
  for (int64_t n = threadIdx.x; n < N; n += 256) orow[n] = sj * wr[n];
}

// AWQ scale per column: binary64 sum of |x| in token order, / T, to binary32,
// binary32 square root.
__global__ __launch_bounds__(256) void k_awq_scales(const float* __restrict__ x, int64_t T,
                                                    int64_t K, float* __restrict__ s) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= K) return;
  double acc = 0.0;
  for (int64_t t = 0; t < T; ++t) acc += (double)fabsf(x[t * K + j]);
  const float m = (float)(acc / (double)T);
  s[j] = m > 0.f ? __builtin_sqrtf(m) : 1.f;
}

// One workgroup per weight row j: w_out[j, :] = s_j w[j, :].
__global__ __launch_bounds__(256) void k_scale_rows(const float* __restrict__ w,
                                                    const float* __restrict__ s, int64_t N,
                                                    float* __restrict__ w_out) {
  const int64_t j = blockIdx.x;
  const float sj = s[j];
  for (int64_t n = threadIdx.x; n < N; n += 256) w_out[j * N + n] = sj * w[j * N + n];
}

template <int DT>
__global__ __launch_bounds__(256) void k_apply_smoothing(const float* __restrict__ x,
                                                         const float* __restrict__ s, int64_t M,
                                                         int64_t K, void* __restrict__ out) {
  const int64_t total = M * K;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const float v = x[i] / s[i % K];
    if constexpr (DT == F32) reinterpret_cast<float*>(out)[i] = v;
    else if constexpr (DT == BF16) reinterpret_cast<uint16_t*>(out)[i] = f32_to_bf16_bits(v);
    else reinterpret_cast<uint16_t*>(out)[i] = f32_to_f16_bits(v);
  }
}

hipError_t launch_smoothquant_fold(const float* x_cal, int64_t T, const float* w, int64_t K,
                                   int64_t N, float* s, float* w_out, hipStream_t st) {
  k_col_absmax<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(x_cal, T, K, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_smoothquant_rows<<<dim3((unsigned)K), dim3(256), 0, st>>>(w, N, s, w_out);
  return hipGetLastError();
}

hipError_t launch_awq_fold(const float* x_cal, int64_t T, const float* w, int64_t K, int64_t N,
                           float* s, float* w_out, hipStream_t st) {
  k_awq_scales<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(x_cal, T, K, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_scale_rows<<<dim3((unsigned)K), dim3(256), 0, st>>>(w, s, N, w_out);
  return hipGetLastError();
}

hipError_t launch_apply_smoothing(const float* x, int64_t M, int64_t K, const float* s,
                                  void* x_out, int out_dtype, hipStream_t st) {
  const int64_t total = M * K;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  dim3 grid((unsigned)blocks), block(256);
  switch (out_dtype) {
    case F32: k_apply_smoothing<F32><<<grid, block, 0, st>>>(x, s, M, K, x_out); break;
    case F16: k_apply_smoothing<F16><<<grid, block, 0, st>>>(x, s, M, K, x_out); break;
    default: k_apply_smoothing<BF16><<<grid, block, 0, st>>>(x, s, M, K, x_out); break;
  }
  return hipGetLastError();
}

}  // namespace qg
