// W4A8 GEMM on 2:4 structured-sparse uint4 weights (「LLM推理降本五要素」 §3.2:
// keep the 2 largest of every 4 weights, then 4-bit g=128 with zero point;
// the sparse matrix cores skip the pruned half).
//
//   acc[m,g,n] = sum over the kept k of group g of xq[m,k] (q[n,k] - z[n,g])   (exact int32)
//   y[m,n]     = x_scale[m] * sum_g s[n,g] acc[m,g,n]                           (binary32)
//
// Weight storage (include/qgemm.h): per (output channel n, group g) four
// 12-byte blocks, block b covering inputs 32 b .. 32 b + 31 of the group: two
// code words (kept value j, j = 0..15 in ascending k, at bits 8 i + 4 [i >= 4]
// of word j / 8, i = j % 8) and a position word (2 bits per kept value: its
// place within its 4 inputs).  Channels are stored in tiles of 16, so one
// group of a workgroup's 16 channels is 768 contiguous bytes: a wave reads it
// with one 12-byte load per lane, six whole cache lines.
//
// One v_smfmac_i32_16x16x128_i8 covers a whole group: the sparse operand is
// 16 weight rows x 128 inputs held as 64 kept bytes per row, lane l carrying
// row l % 16, block l / 16 (its 16 kept values and its position word as the
// instruction's index operand); the dense operand is 16 token rows, lane l
// carrying token l % 16, inputs 16 (l / 16) + [0, 16) and 64 + 16 (l / 16) +
// [0, 16) (two plain 16-byte loads).  Result lane l: rows n = 4 (l / 16) + i,
// token l % 16 (this operand arrangement was measured on MI355X with random
// operands against the dense product).
//
// Code bytes become (q - z) in place: w & 0x0F0F0F0F gives values 0..3 (the
// high nibbles, shifted, 4..7) as bytes 0..15; (b + 128 - z) never borrows
// across bytes, and xor 0x80 turns it into the two's complement byte of q - z.
#include "qg_device.hpp"
#include "qg_decode.hpp"
#include "qg_launch.hpp"

namespace qg {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kSp24Waves = 8;
constexpr int kSp24Batch = 2;   // groups per load batch

// 16 operand bytes (q - z) from a block's two code words, z replicated in zr
__device__ __forceinline__ v4i sp24_operand(u32 w0, u32 w1, u32 zr) {
  const u32 m = 0x0F0F0F0Fu, h = 0x80808080u;
  return v4i{(int)((((w0 & m) | h) - zr) ^ h), (int)(((((w0 >> 4) & m) | h) - zr) ^ h),
             (int)((((w1 & m) | h) - zr) ^ h), (int)(((((w1 >> 4) & m) | h) - zr) ^ h)};
}

// A workgroup owns 16 weight rows (output channels) x 16 token rows; its
// kSp24Waves waves split the groups into contiguous runs and reduce their
// binary32 partial sums through LDS.  Scales and zero points of the 16 weight
// rows are staged in LDS (s | z << 16 per (row, group)).
template <typename OutT>
__global__ __launch_bounds__(64 * kSp24Waves) void k_w4a8_sp24(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, const int32_t* __restrict__ wsp,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero, int M, int N, int K,
    OutT* __restrict__ y) {
  constexpr bool kI32 = __is_same(OutT, int32_t);
  constexpr int kThreads = 64 * kSp24Waves;
  extern __shared__ __attribute__((aligned(16))) u32 szl[];   // 16 x sz_pitch(G) words
  __shared__ v4f red[kI32 ? 1 : kSp24Waves][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int n_base = blockIdx.x * 16, m_base = blockIdx.y * 16;
  const int G = K >> 7;
  const int gb = (int)((int64_t)G * wave / kSp24Waves), ge = (int)((int64_t)G * (wave + 1) / kSp24Waves);

  const int rows_n = min(16, N - n_base), rows_m = min(16, M - m_base);
  // tile blockIdx.x: group g's 16 rows are 768 contiguous bytes; row r's
  // block j at 48 r + 12 j (rows past N are stored as zeros)
  const rsrc_t wr = make_rsrc_uniform(wsp + (int64_t)blockIdx.x * G * 192, (u32)(G * 768));
  const u32 woff = (u32)(48 * r + 12 * j);
  // token row r: inputs 16 j and 64 + 16 j of the group
  const rsrc_t xr = make_rsrc_uniform(xq + (int64_t)m_base * K, (u32)(rows_m * K));
  const u32 xoff = (u32)(r * K + 16 * j);

  ScaleZeroStage<kThreads, 2> sz;
  const rsrc_t sr = make_rsrc_uniform(wscale + (int64_t)n_base * G, (u32)(rows_n * G * 2));
  const rsrc_t zr = make_rsrc_uniform(wzero + (int64_t)n_base * G, (u32)(rows_n * G * 2));
  sz.load(sr, zr, 16 * G, 0);
  sz.finish(sr, zr, szl, G, 16 * G);
  lds_barrier();

  v4f yacc = {0.f, 0.f, 0.f, 0.f};
  // a batch: kSp24Batch consecutive groups; two batches in flight
  struct Batch {
    v4i w[kSp24Batch], x[kSp24Batch][2];
  };
  auto load = [&](Batch& bt, int g0) {
#pragma unroll
    for (int u = 0; u < kSp24Batch; ++u) {
      const int g = g0 + u;
      const bool in = g < ge;
      const auto t = __builtin_amdgcn_raw_buffer_load_b96(wr, in ? woff + 768 * g : kOOB, 0, 0);
      bt.w[u] = v4i{(int)t[0], (int)t[1], (int)t[2], 0};
      bt.x[u][0] = bld16(xr, in ? xoff + 128 * g : kOOB);
      bt.x[u][1] = bld16(xr, in ? xoff + 128 * g + 64 : kOOB);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mma = [&](const Batch& bt, int g0) {
#pragma unroll
    for (int u = 0; u < kSp24Batch; ++u) {
      const int g = g0 + u;
      const v4i& wv = bt.w[u];
      const u32 szw = g < ge ? szl[r * sz_pitch(G) + g] : 0u;      // row r: z of the operand
      const u32 z = (u32)(int)f16_bits_to_f32((uint16_t)(szw >> 16));
      const v4i a = sp24_operand((u32)wv[0], (u32)wv[1], z * 0x01010101u);
      const v8i b = {bt.x[u][0][0], bt.x[u][0][1], bt.x[u][0][2], bt.x[u][0][3],
                     bt.x[u][1][0], bt.x[u][1][1], bt.x[u][1][2], bt.x[u][1][3]};
      const v4i acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, v4i{0, 0, 0, 0}, wv[2], 0, 0);
      if (g >= ge) continue;
      if constexpr (kI32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = n_base + 4 * j + i, m = m_base + r;
          if (n < N && m < M) y[((int64_t)m * G + g) * N + n] = acc[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sc = f16_bits_to_f32((uint16_t)(szl[(4 * j + i) * sz_pitch(G) + g] & 0xFFFFu));
          yacc[i] = __builtin_fmaf(sc, (float)acc[i], yacc[i]);
        }
      }
    }
  };
  Batch b0, b1;
  load(b0, gb);
  for (int g = gb; g < ge; g += 2 * kSp24Batch) {
    load(b1, g + kSp24Batch);
    mma(b0, g);
    load(b0, g + 2 * kSp24Batch);
    mma(b1, g + kSp24Batch);
  }

  if constexpr (!kI32) {
    red[wave][lane] = yacc;
    __syncthreads();
    if (tid < 64) {
      v4f sum = red[0][lane];
#pragma unroll
      for (int w = 1; w < kSp24Waves; ++w) sum += red[w][lane];
      const int m = m_base + r;
      if (m < M) {
        const float sx = xs[m];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = n_base + 4 * j + i;
          if (n < N) y[(int64_t)m * N + n] = Out<OutT>::cvt(sum[i] * sx);
        }
      }
    }
  }
}

template <typename OutT>
static hipError_t gemm_w4a8_sp24_t(const int8_t* xq, const float* xs, const int32_t* wsp,
                                   const uint16_t* ws, const uint16_t* wz, int M, int N, int K,
                                   OutT* y, hipStream_t st) {
  const int G = K / 128;
  const size_t lds = (size_t)16 * sz_pitch(G) * 4;
  if (lds > kDecLdsMaxBytes) return hipErrorInvalidValue;   // excluded by the API checks
  const dim3 grid((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16)), block(64 * kSp24Waves);
  k_w4a8_sp24<OutT><<<grid, block, lds, st>>>(xq, xs, wsp, ws, wz, M, N, K, y);
  return hipGetLastError();
}

hipError_t launch_gemm_w4a8_sp24(const int8_t* xq, const float* xs, const int32_t* wsp,
                                 const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                                 int64_t K, void* y, int y_dtype, hipStream_t st) {
  const int m = (int)M, n = (int)N, k = (int)K;
  switch (y_dtype) {
    case F32: return gemm_w4a8_sp24_t<float>(xq, xs, wsp, ws, wz, m, n, k, (float*)y, st);
    case F16: return gemm_w4a8_sp24_t<_Float16>(xq, xs, wsp, ws, wz, m, n, k, (_Float16*)y, st);
    case BF16: return gemm_w4a8_sp24_t<uint16_t>(xq, xs, wsp, ws, wz, m, n, k, (uint16_t*)y, st);
    default: return gemm_w4a8_sp24_t<int32_t>(xq, xs, wsp, ws, wz, m, n, k, (int32_t*)y, st);
  }
}

}  // namespace qg
