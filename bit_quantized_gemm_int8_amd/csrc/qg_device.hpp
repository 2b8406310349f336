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

// Sum over each aligned group of 8 lanes, every lane of the group receiving
// it: DPP swaps of neighbours and of pairs (quad permutations), then the
// mirror within each half row pairs the two quads.
__device__ __forceinline__ int sum_lanes8(int t) {
  t += __builtin_amdgcn_mov_dpp(t, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  t += __builtin_amdgcn_mov_dpp(t, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  t += __builtin_amdgcn_mov_dpp(t, 0x141, 0xF, 0xF, false);   // row_half_mirror
  return t;
}

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
// The same from values every lane holds alike, pinned to scalar registers: a
// resource the compiler keeps in vector registers costs a waterfall loop
// around every load that uses it.
__device__ __forceinline__ rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return make_rsrc((const void*)(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(bytes));
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

// Max of non-negative values over a wave through DPP: rotations within each
// row of 16 lanes (every lane then holds its row's max), then the four rows'
// values read into scalars.  No LDS round trips.  The result is uniform.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  int x = __float_as_int(v);   // non-negative floats order as their bit patterns
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x121, 0xF, 0xF, false));   // row_ror:1
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x122, 0xF, 0xF, false));   // row_ror:2
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, false));   // row_ror:4
  x = max(x, __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));   // row_ror:8
  const int a = max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16));
  const int b = max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48));
  return __int_as_float(max(a, b));
}

// Max of non-negative values over a workgroup of NT threads, for a kernel
// that reduces once: one barrier (red is not reused afterwards).
template <int NT>
__device__ __forceinline__ float block_max_nonneg_once(float v, float* red /* LDS, NT/64 */) {
  v = wave_max_nonneg(v);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, red[i]);
  return r;
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

// ---- symmetric int8 codes ---------------------------------------------------
// The code of x under the scale s = fl32(max|x| / 127) > 0 of its slice (row,
// column, channel) is clamp(rint(fl32(x / s)), -127, 127), with x / s the
// correctly rounded binary32 quotient and rint half to even.  While s is a
// normal number |x / s| stays within one rounding of 127, but a subnormal s
// carries fewer significant bits and can come out well below max|x| / 127
// (max|x| = 316 * 2^-149 gives s = 2 * 2^-149 and max|x| / s = 158): the
// clamp then binds.
//
// sym_code_t forms the code from the reciprocal r = fl32(1 / s), computed once
// per slice.  A finite r means s >= 2^-128, where s has at least 21
// significant bits: with q = x / s exact, |q| <= 127 (1 + 2^-21), fl32(q) lies
// within 2^-24 |q| of q and x * r, rounded once or not at all, within
// (2^-23 + 2^-48) |q|: the two differ by less than 2.3e-5 < 2^-15, and
// neither leaves [-127.5, 127.5].  When x * r is at least 2^-15 away from
// every half-integer, both round to the same integer; otherwise (and for any
// x when r is infinite, i.e. s < 2^-128) the correctly rounded division
// decides, clamped to [-127, 127] before rounding (the bounds are integers,
// so clamping first is the same as clamping the rounded code).  Adding
// 1.5 * 2^23 rounds to an integer (half to even) and leaves it, two's
// complement, in the low bits: the returned float's low byte is the code.
// r = 0 (an all-zero slice) gives code 0.
constexpr float kCodeTie = 0.5f - 1.f / 32768.f;
constexpr float kRoundMagic = 12582912.f;   // 1.5 * 2^23

__device__ __forceinline__ float sym_code_t(float x, float s, float r) {
  const float a = x * r;
  float t = a + kRoundMagic;
  // near a tie (or NaN: r infinite): the correctly rounded quotient, clamped
  if (!(fabsf(a - (t - kRoundMagic)) <= kCodeTie))
    t = (s > 0.f ? __builtin_amdgcn_fmed3f(x / s, -127.f, 127.f) : 0.f) + kRoundMagic;
  return t;
}

// Reciprocal of a slice's scale for sym_code_t: 0 for an all-zero slice.
__device__ __forceinline__ float sym_code_r(float amax, float s) {
  return amax > 0.f ? 1.f / s : 0.f;
}

// The low bytes of four sym_code_t results as one word (byte j from t_j).
__device__ __forceinline__ u32 pack_code_bytes(float t0, float t1, float t2, float t3) {
  // v_perm selector 0x0c yields a zero byte
  return __builtin_amdgcn_perm(__float_as_uint(t1), __float_as_uint(t0), 0x0c0c0400u) |
         __builtin_amdgcn_perm(__float_as_uint(t3), __float_as_uint(t2), 0x04000c0cu);
}

}  // namespace qg
