// Building blocks of the per-token int8 quantizers: 16-value chunks of a
// token row (fp32, fp16 or bf16) loaded, widened exactly to binary32 and
// turned into symmetric int8 codes (sym_code_t).  Shared by every kernel
// that quantizes activation rows, so all of them produce the same codes.
#pragma once

#include "qg_device.hpp"
#include "qg_launch.hpp"

namespace qg {

// Chunk c of a row through a buffer resource over the row: a chunk past the
// row's end reads zeros, so a thread's loads need no branch and all of them
// are in flight together.
template <int DT>
__device__ __forceinline__ void load_chunk16_rs(rsrc_t row, bool valid, int c, v4i (&raw)[4]) {
  constexpr int kBytes = DT == F32 ? 64 : 32;
#pragma unroll
  for (int i = 0; i < kBytes / 16; ++i)
    raw[i] = bld16(row, valid ? (u32)(c * kBytes + 16 * i) : kOOB);
}

template <int DT>
__device__ __forceinline__ void widen16(const v4i (&raw)[4], float (&v)[16]) {
  if constexpr (DT == F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = __int_as_float(raw[i][e]);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32 u = (u32)raw[i][e];
        if constexpr (DT == BF16) {
          v[8 * i + 2 * e] = bf16_bits_to_f32(u & 0xFFFFu);
          v[8 * i + 2 * e + 1] = bf16_bits_to_f32(u >> 16);
        } else {
          v[8 * i + 2 * e] = f16_bits_to_f32((uint16_t)(u & 0xFFFFu));
          v[8 * i + 2 * e + 1] = f16_bits_to_f32((uint16_t)(u >> 16));
        }
      }
  }
}

template <int DT>
__device__ __forceinline__ void load_chunk16(const void* row, int c, float (&v)[16]) {
  if constexpr (DT == F32) {
    const float* p = reinterpret_cast<const float*>(row) + c * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v4i t = ld16(p + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = __int_as_float(t[e]);
    }
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row) + c * 16;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v4i t = ld16(p + 8 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32 u = (u32)t[e];
        if constexpr (DT == BF16) {
          v[8 * i + 2 * e] = bf16_bits_to_f32(u & 0xFFFFu);
          v[8 * i + 2 * e + 1] = bf16_bits_to_f32(u >> 16);
        } else {
          v[8 * i + 2 * e] = f16_bits_to_f32((uint16_t)(u & 0xFFFFu));
          v[8 * i + 2 * e + 1] = f16_bits_to_f32((uint16_t)(u >> 16));
        }
      }
    }
  }
}

// codes of 16 values of one slice with scale s and reciprocal r (sym_code_r)
__device__ __forceinline__ v4i codes16(const float (&v)[16], float s, float r) {
  v4i out;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    out[w] = (int)pack_code_bytes(sym_code_t(v[4 * w], s, r), sym_code_t(v[4 * w + 1], s, r),
                                  sym_code_t(v[4 * w + 2], s, r), sym_code_t(v[4 * w + 3], s, r));
  return out;
}

template <int DT>
constexpr int esize() { return DT == F32 ? 4 : 2; }

}  // namespace qg
