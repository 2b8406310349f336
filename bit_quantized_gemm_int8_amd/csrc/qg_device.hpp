// Device-side helpers shared by the gfx950 kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32;

constexpr int kWave = 64;

// ---- 16-byte global accesses ------------------------------------------------

__device__ __forceinline__ v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }

// Streaming load: weights are read once per call, so keep them out of the way
// of the activations in the caches.
__device__ __forceinline__ v4i ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

__device__ __forceinline__ void st16(void* p, v4i v) { *reinterpret_cast<v4i*>(p) = v; }

// ---- raw buffer loads --------------------------------------------------------
// A buffer resource covers [base, base + bytes); a load whose offset lies past
// the end returns zeros instead of touching memory, so edge tiles and masked
// lanes need no branch: they pass kOOB (or any offset >= bytes).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr u32 kOOB = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ v4i bld16(rsrc_t r, u32 off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Streaming variant (non-temporal cache policy) for data read exactly once per
// call, i.e. the weight stream; measured ~6% faster than the default policy
// for a 45 MB stream on MI355X.
constexpr int kAuxNonTemporal = 2;
__device__ __forceinline__ v4i bld16_nt(rsrc_t r, u32 off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNonTemporal));
}
__device__ __forceinline__ uint16_t bld2(rsrc_t r, u32 off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// ---- number formats ----------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(u32 h) { return __uint_as_float(h << 16); }

// binary32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  u32 u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

template <typename OutT> struct Out;
template <> struct Out<float> {
  static __device__ __forceinline__ float cvt(float v) { return v; }
};
template <> struct Out<uint16_t> {  // bfloat16 stored as bits
  static __device__ __forceinline__ uint16_t cvt(float v) { return f32_to_bf16_bits(v); }
};
template <> struct Out<_Float16> {
  static __device__ __forceinline__ _Float16 cvt(float v) { return (_Float16)v; }
};

// ---- reductions --------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Max over a whole workgroup of NT threads; every thread gets the result.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red /* LDS, NT/64 floats */) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// ---- symmetric int8 code of x given the scale s > 0 ------------------------
// x / s is the correctly rounded binary32 quotient (hipcc's default fp32
// division); rintf rounds half to even.
__device__ __forceinline__ int sym_code_i8(float x, float s) {
  float q = __builtin_rintf(x / s);
  q = fminf(fmaxf(q, -127.f), 127.f);
  return (int)q;
}

}  // namespace qg
