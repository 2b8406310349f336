// Measurement probes: what the chip delivers on the layer's two bounds, so
// that the kernels can be compared with measured ceilings as well as with the
// published peaks (「LLM推理降本五要素」 §2.1 quotes the W8A8 layer's weight
// bandwidth against its part's own peak in the same way).
//
//   * a streaming read of a buffer of the decode layers' size, shaped like
//     the best plain read measured on MI355X: one workgroup of 8 waves per
//     CU at most, each workgroup a contiguous stretch, each wave a contiguous
//     part of it, every 16-byte load of a wave issued before any is used;
//   * loops of int8 and fp16 matrix-core instructions on random register
//     operands, with the per-wave shader-clock and real-time counters, so the
//     clock the chip runs at under that load is known;
//   * an empty kernel: the fixed cost of one launch.
// Nothing here is on the method's path.
#include "qg_device.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemm.h"
#include "qgemm_peaks.h"

namespace qg {

constexpr int kReadWaves = 8;

// Workgroup b reads KB [b W CH, (b + 1) W CH) of the buffer; wave w the CH KB
// starting at (b W + w) CH; load c of a lane covers bytes 16 l of KB c.
template <int CH>
__global__ __launch_bounds__(64 * kReadWaves) void k_peak_read(const int8_t* __restrict__ p,
                                                               int64_t bytes,
                                                               int32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kReadWaves + (threadIdx.x >> 6);
  const int64_t base = wave * CH * 1024;
  const int64_t left = bytes - base;
  const rsrc_t r = make_rsrc(p + (left > 0 ? base : 0),
                             (u32)(left <= 0 ? 0 : left < CH * 1024 ? left : CH * 1024));
  v4i v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = bld16_nt(r, (u32)(c * 1024 + 16 * lane));
  int x = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) x ^= v[c][0] ^ v[c][1] ^ v[c][2] ^ v[c][3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, kWave);
  if (lane == 0) sink[wave] = x;
}

constexpr int kReadCh[] = {4, 8, 12, 16, 24, 32};

static int read_ch(int64_t bytes) {
  const int64_t kb = (bytes + 1023) / 1024;
  for (int ch : kReadCh)
    if (kb <= (int64_t)256 * kReadWaves * ch) return ch;
  return 32;
}

static int64_t read_waves(int64_t bytes) {
  const int64_t per = (int64_t)read_ch(bytes) * 1024 * kReadWaves;
  return (bytes + per - 1) / per * kReadWaves;
}

// Matrix-core loop: each wave keeps four independent accumulators and feeds
// them four operand pairs drawn from a per-lane hash (full-range values), for
// `iters` rounds.  Kind 0: v_mfma_i32_32x32x32_i8; 1: v_mfma_i32_16x16x64_i8;
// 2: v_mfma_f32_32x32x16_f16; 3: v_mfma_f32_32x32x16_bf16.
__device__ __forceinline__ u32 hash32(u32 x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <int KIND>
__global__ __launch_bounds__(256) void k_peak_mfma(int64_t iters, uint64_t* __restrict__ clocks,
                                                   int32_t* __restrict__ sink) {
  const u32 gid = blockIdx.x * 256 + threadIdx.x;
  v4i a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32 ha = hash32(gid * 131u + 8u * i + e), hb = hash32(gid * 977u + 8u * i + e + 4u);
      if constexpr (KIND >= 2) {   // finite 16-bit values: clear the top exponent bit of each half
        ha &= 0xBFFFBFFFu;
        hb &= 0xBFFFBFFFu;
      }
      a[i][e] = (int)ha;
      b[i][e] = (int)hb;
    }
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  int32_t out = 0;
  if constexpr (KIND == 0) {
    v16i acc[4] = {};
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[i], acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) out ^= acc[i][0] ^ acc[i][15];
  } else if constexpr (KIND == 1) {
    v4i acc[4] = {};
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[i], acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) out ^= acc[i][0] ^ acc[i][3];
  } else {
    typedef float v16f __attribute__((ext_vector_type(16)));
    v16f acc[4] = {};
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (KIND == 2)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a[i]),
                                                          __builtin_bit_cast(v8h, b[i]), acc[i], 0, 0, 0);
        else
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[i]),
                                                           __builtin_bit_cast(v8bf, b[i]), acc[i], 0, 0, 0);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) out ^= __float_as_int(acc[i][0]) ^ __float_as_int(acc[i][15]);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  const u32 wave = gid >> 6;
  if ((threadIdx.x & 63) == 0) {
    clocks[2 * wave] = t1 - t0;
    clocks[2 * wave + 1] = r1 - r0;
  }
  sink[gid] = out;
}

constexpr int64_t kPeakOpsPerMfma[] = {2LL * 32 * 32 * 32, 2LL * 16 * 16 * 64, 2LL * 32 * 32 * 16,
                                       2LL * 32 * 32 * 16};

__global__ void k_peak_empty() {}

}  // namespace qg

using namespace qg;

extern "C" {

int64_t qg_peak_stream_read_sink(int64_t bytes) { return bytes <= 0 ? 0 : read_waves(bytes); }

qg_status_t qg_peak_stream_read(const void* src, int64_t bytes, int32_t* sink, void* stream) {
  if (!src || !sink) return QG_ERR_NULL;
  if (bytes <= 0 || bytes > ((int64_t)1 << 31)) return QG_ERR_SHAPE;
  if (((uintptr_t)src & 15) != 0) return QG_ERR_ALIGN;
  const hipStream_t st = (hipStream_t)stream;
  const int ch = read_ch(bytes);
  const unsigned grid = (unsigned)(read_waves(bytes) / kReadWaves);
  const int8_t* p = (const int8_t*)src;
  switch (ch) {
    case 4: k_peak_read<4><<<grid, 64 * kReadWaves, 0, st>>>(p, bytes, sink); break;
    case 8: k_peak_read<8><<<grid, 64 * kReadWaves, 0, st>>>(p, bytes, sink); break;
    case 12: k_peak_read<12><<<grid, 64 * kReadWaves, 0, st>>>(p, bytes, sink); break;
    case 16: k_peak_read<16><<<grid, 64 * kReadWaves, 0, st>>>(p, bytes, sink); break;
    case 24: k_peak_read<24><<<grid, 64 * kReadWaves, 0, st>>>(p, bytes, sink); break;
    default: k_peak_read<32><<<grid, 64 * kReadWaves, 0, st>>>(p, bytes, sink); break;
  }
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}

int64_t qg_peak_mfma_ops(int kind, int64_t iters, int64_t workgroups) {
  if (kind < 0 || kind > 3 || iters < 0 || workgroups < 0) return -1;
  return kPeakOpsPerMfma[kind] * 4 * iters * workgroups * 4;   // 4 waves x 4 MFMAs per round
}

qg_status_t qg_peak_mfma(int kind, int64_t iters, int64_t workgroups, uint64_t* clocks,
                         int32_t* sink, void* stream) {
  if (!clocks || !sink) return QG_ERR_NULL;
  if (kind < 0 || kind > 3) return QG_ERR_ARG;
  if (iters < 1 || workgroups < 1 || workgroups > 65535) return QG_ERR_SHAPE;
  const hipStream_t st = (hipStream_t)stream;
  const unsigned g = (unsigned)workgroups;
  switch (kind) {
    case 0: k_peak_mfma<0><<<g, 256, 0, st>>>(iters, clocks, sink); break;
    case 1: k_peak_mfma<1><<<g, 256, 0, st>>>(iters, clocks, sink); break;
    case 2: k_peak_mfma<2><<<g, 256, 0, st>>>(iters, clocks, sink); break;
    default: k_peak_mfma<3><<<g, 256, 0, st>>>(iters, clocks, sink); break;
  }
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}

qg_status_t qg_peak_empty(void* stream) {
  k_peak_empty<<<1, 64, 0, (hipStream_t)stream>>>();
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}

}  // extern "C"
