// Quantizers: per-token int8 activations (hot path), per-channel int8 and
// g=128 uint4 weights (offline).
//
// 「第4章：量化」 §1.1 x_int = round(x/s) + z; §1.2 symmetric s = max|x|/127,
// asymmetric scale from (max - min) over 2^bits - 1 steps; §1.3 per-token,
// per-channel and per-group granularity.  「LLM推理降本五要素」 §5.2: round,
// then clamp to the int8 range.
#include "qg_device.hpp"
#include "qg_launch.hpp"
#include "qg_quant.hpp"

namespace qg {

// ---------------------------------------------------------------------------
// Per-token activation quantization.  One 256-thread workgroup per token
// (row).  Each thread owns up to CH chunks of 16 consecutive elements, held in
// registers between the absmax pass and the quantize pass, so the row is read
// from HBM once; codes leave as one 16-byte store per chunk.
// ---------------------------------------------------------------------------

// NT threads per row (256 to 1024: more for long rows, so that few rows
// still keep many lanes busy).  CH > 0: row cached in registers.  CH == 0:
// rows too long for that; the second pass re-reads the row (it is then L2
// resident).
template <int DT, int CH, int NT>
__global__ __launch_bounds__(NT) void k_quant_per_token(const void* __restrict__ x, int64_t K,
                                                        int8_t* __restrict__ xq,
                                                        float* __restrict__ xs) {
  __shared__ float red[NT / kWave];
  const int64_t row = blockIdx.x;
  const char* xr = reinterpret_cast<const char*>(x) + row * K * esize<DT>();
  int8_t* qr = xq + row * K;
  const int nch = (int)(K >> 4);
  float amax = 0.f;
  if constexpr (CH > 0) {
    // K <= 4 * 1024 * 16 here, so the row's bytes fit a buffer resource
    const rsrc_t rr = make_rsrc(xr, (uint32_t)(K * esize<DT>()));
    v4i raw[CH][4];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = threadIdx.x + c * NT;
      load_chunk16_rs<DT>(rr, idx < nch, idx, raw[c]);
    }
    float v[CH][16];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      widen16<DT>(raw[c], v[c]);
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[c][e]));   // zeros past the end
    }
    amax = block_max_nonneg_once<NT>(amax, red);
    const float s = amax / 127.f, r = sym_code_r(amax, s);
    if (threadIdx.x == 0) xs[row] = amax > 0.f ? s : 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = threadIdx.x + c * NT;
      if (idx < nch) st16(qr + (int64_t)idx * 16, codes16(v[c], s, r));
    }
  } else {
    for (int idx = threadIdx.x; idx < nch; idx += NT) {
      float v[16];
      load_chunk16<DT>(xr, idx, v);
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = block_max_nonneg_once<NT>(amax, red);
    const float s = amax / 127.f, r = sym_code_r(amax, s);
    if (threadIdx.x == 0) xs[row] = amax > 0.f ? s : 0.f;
    for (int idx = threadIdx.x; idx < nch; idx += NT) {
      float v[16];
      load_chunk16<DT>(xr, idx, v);
      st16(qr + (int64_t)idx * 16, codes16(v, s, r));
    }
  }
}

// Many rows (prefill): one wave per row, four rows per workgroup.  Lane l
// holds bytes 1024 c + 16 l of its row for c < NC -- every load of the row
// in flight at once, each instruction a whole kilobyte -- then the row's
// maximum is a DPP reduction inside the wave (no LDS, no barrier), and the
// codes of each 16-byte chunk leave as one 8-byte (16-bit input) or 4-byte
// (fp32) store, a whole 512 or 256 bytes per instruction.  Chunks past the
// row read zeros through the buffer resource and their stores fall outside
// the codes' resource.  The codes are those of k_quant_per_token: the same
// scale, reciprocal and sym_code_t.
typedef int v2i_ __attribute__((ext_vector_type(2)));

template <int DT, int NC>
__global__ __launch_bounds__(256) void k_quant_rows_wave(const void* __restrict__ x, int64_t M,
                                                         int64_t K, int8_t* __restrict__ xq,
                                                         float* __restrict__ xs) {
  constexpr int E = esize<DT>(), VPC = 16 / E;   // input bytes per element, values per chunk
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;   // wave-uniform
  const rsrc_t xr = make_rsrc_uniform(reinterpret_cast<const char*>(x) + row * K * E, (u32)(K * E));
  const rsrc_t qr = make_rsrc_uniform(xq + row * K, (u32)K);
  v4i raw[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) raw[c] = bld16(xr, (u32)(1024 * c + 16 * lane));
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const u32 u = (u32)raw[c][e];
      if constexpr (DT == F32) {
        amax = fmaxf(amax, fabsf(__uint_as_float(u)));
      } else if constexpr (DT == BF16) {
        amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(u & 0xFFFFu)), fabsf(bf16_bits_to_f32(u >> 16))));
      } else {
        amax = fmaxf(amax, fmaxf(fabsf(f16_bits_to_f32((uint16_t)(u & 0xFFFFu))),
                                 fabsf(f16_bits_to_f32((uint16_t)(u >> 16)))));
      }
    }
  amax = wave_max_nonneg(amax);
  const float s = amax / 127.f, r = sym_code_r(amax, s);
  if (lane == 0) xs[row] = amax > 0.f ? s : 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const u32 u = (u32)raw[c][e];
      if constexpr (DT == F32) {
        v[e] = __uint_as_float(u);
      } else if constexpr (DT == BF16) {
        v[2 * e] = bf16_bits_to_f32(u & 0xFFFFu);
        v[2 * e + 1] = bf16_bits_to_f32(u >> 16);
      } else {
        v[2 * e] = f16_bits_to_f32((uint16_t)(u & 0xFFFFu));
        v[2 * e + 1] = f16_bits_to_f32((uint16_t)(u >> 16));
      }
    }
    const u32 off = (u32)((1024 * c + 16 * lane) / E);   // first code of the chunk
    if constexpr (VPC == 8) {
      const u32 w0 = pack_code_bytes(sym_code_t(v[0], s, r), sym_code_t(v[1], s, r),
                                     sym_code_t(v[2], s, r), sym_code_t(v[3], s, r));
      const u32 w1 = pack_code_bytes(sym_code_t(v[4], s, r), sym_code_t(v[5], s, r),
                                     sym_code_t(v[6], s, r), sym_code_t(v[7], s, r));
      __builtin_amdgcn_raw_buffer_store_b64(v2i_{(int)w0, (int)w1}, qr, off, 0, 0);
    } else {
      const u32 w0 = pack_code_bytes(sym_code_t(v[0], s, r), sym_code_t(v[1], s, r),
                                     sym_code_t(v[2], s, r), sym_code_t(v[3], s, r));
      __builtin_amdgcn_raw_buffer_store_b32((int)w0, qr, off, 0, 0);
    }
  }
}

// rows at or above which the one-wave-per-row form runs (enough rows for
// every CU to hold several waves of it)
constexpr int64_t kRowsWaveMinM = 1024;

template <int DT>
static hipError_t quant_rows_wave(const void* x, int64_t M, int64_t K, int8_t* xq, float* xs,
                                  hipStream_t st) {
  const int64_t nc = (K * esize<DT>() + 1023) / 1024;
  const dim3 grid((unsigned)((M + 3) / 4)), block(256);
  if (nc <= 4) k_quant_rows_wave<DT, 4><<<grid, block, 0, st>>>(x, M, K, xq, xs);
  else if (nc <= 8) k_quant_rows_wave<DT, 8><<<grid, block, 0, st>>>(x, M, K, xq, xs);
  else if (nc <= 12) k_quant_rows_wave<DT, 12><<<grid, block, 0, st>>>(x, M, K, xq, xs);
  else k_quant_rows_wave<DT, 16><<<grid, block, 0, st>>>(x, M, K, xq, xs);   // rows <= 16 KB
  return hipGetLastError();
}

template <int DT>
static hipError_t quant_per_token_dt(const void* x, int64_t M, int64_t K, int8_t* xq, float* xs,
                                     hipStream_t st) {
  const int64_t nch = K / 16;
  const dim3 grid((unsigned)M);
  if (M >= kRowsWaveMinM && K * esize<DT>() <= 16 * 1024)
    return quant_rows_wave<DT>(x, M, K, xq, xs, st);
  if (nch <= 256)
    k_quant_per_token<DT, 1, 256><<<grid, 256, 0, st>>>(x, K, xq, xs);
  else if (nch <= 512)
    k_quant_per_token<DT, 1, 512><<<grid, 512, 0, st>>>(x, K, xq, xs);
  else if (nch <= 1024)   // 512 threads x 2 chunks: measured faster than 1024 x 1 on MI355X
    k_quant_per_token<DT, 2, 512><<<grid, 512, 0, st>>>(x, K, xq, xs);
  else if (nch <= 2048)
    k_quant_per_token<DT, 2, 1024><<<grid, 1024, 0, st>>>(x, K, xq, xs);
  else if (nch <= 4096)
    k_quant_per_token<DT, 4, 1024><<<grid, 1024, 0, st>>>(x, K, xq, xs);
  else
    k_quant_per_token<DT, 0, 1024><<<grid, 1024, 0, st>>>(x, K, xq, xs);
  return hipGetLastError();
}

hipError_t launch_quant_per_token(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* xq,
                                  float* x_scale, hipStream_t st) {
  switch (x_dtype) {
    case F32: return quant_per_token_dt<F32>(x, M, K, xq, x_scale, st);
    case F16: return quant_per_token_dt<F16>(x, M, K, xq, x_scale, st);
    default: return quant_per_token_dt<BF16>(x, M, K, xq, x_scale, st);
  }
}

// ---------------------------------------------------------------------------
// Per-output-channel int8 weights.  A workgroup owns 64 output channels:
// pass 1 reduces max|w| down each column (coalesced along N), pass 2 walks K
// in 64-row tiles, transposes through LDS and writes K-contiguous codes.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_quant_weight_i8(const float* __restrict__ w, int64_t K,
                                                         int64_t N, int8_t* __restrict__ wq,
                                                         float* __restrict__ ws) {
  __shared__ float red[4][64];
  __shared__ float colmax[64];
  __shared__ float tile[64][65];
  const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t n = n0 + c;
  float amax = 0.f;
  if (n < N)
    for (int64_t k = r; k < K; k += 4) amax = fmaxf(amax, fabsf(w[k * N + n]));
  red[r][c] = amax;
  __syncthreads();
  if (r == 0) {
    const float a = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
    colmax[c] = a;
    if (n < N) ws[n] = a > 0.f ? a / 127.f : 0.f;
  }
  __syncthreads();
  const int cc = threadIdx.x >> 2, seg = threadIdx.x & 3;
  const int64_t ncol = n0 + cc;
  const float a = colmax[cc];
  const float s = a / 127.f, rs = sym_code_r(a, s);
  for (int64_t k0 = 0; k0 < K; k0 += 64) {
    for (int kk = r; kk < 64; kk += 4)
      tile[kk][c] = (k0 + kk < K && n < N) ? w[(k0 + kk) * N + n] : 0.f;
    __syncthreads();
    if (ncol < N && k0 + seg * 16 < K) {
      float v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = tile[seg * 16 + e][cc];
      st16(wq + ncol * K + k0 + seg * 16, codes16(v, s, rs));
    }
    __syncthreads();
  }
}

hipError_t launch_quant_weight_i8(const float* w, int64_t K, int64_t N, int8_t* wq, float* ws,
                                  hipStream_t st) {
  dim3 grid((unsigned)((N + 63) / 64)), block(256);
  k_quant_weight_i8<<<grid, block, 0, st>>>(w, K, N, wq, ws);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// g=128 asymmetric uint4 weights.  A workgroup owns 64 output channels x one
// group; each thread holds 32 of a column's 128 weights, the four quarters
// meet in LDS for min/max, then every thread derives the same (s, z) and packs
// its 32 codes into 4 words (one 16-byte store).
// ---------------------------------------------------------------------------

// Smallest fp16 value >= t (t >= 0, finite): the stored scale never falls
// below (max - min)/15, so codes stay within [0, 15].
__device__ __forceinline__ _Float16 f16_round_up(float t) {
  _Float16 h = (_Float16)t;  // round to nearest even
  if ((float)h < t) h = __builtin_bit_cast(_Float16, (uint16_t)(__builtin_bit_cast(uint16_t, h) + 1));
  return h;
}

__global__ __launch_bounds__(256) void k_quant_weight_u4(const float* __restrict__ w, int64_t K,
                                                         int64_t N, int32_t* __restrict__ wq,
                                                         uint16_t* __restrict__ wscale,
                                                         uint16_t* __restrict__ wzero) {
  __shared__ float rlo[4][64], rhi[4][64];
  const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 64 + c;
  const int64_t g = blockIdx.y;
  const int64_t G = K >> 7;
  float v[32];
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
  if (n < N) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = w[(g * 128 + r * 32 + i) * N + n];
      lo = fminf(lo, v[i]);
      hi = fmaxf(hi, v[i]);
    }
  }
  rlo[r][c] = lo;
  rhi[r][c] = hi;
  __syncthreads();
  if (n >= N) return;
  lo = fminf(fminf(rlo[0][c], rlo[1][c]), fminf(rlo[2][c], rlo[3][c]));
  hi = fmaxf(fmaxf(rhi[0][c], rhi[1][c]), fmaxf(rhi[2][c], rhi[3][c]));
  const float t = (hi - lo) / 15.f;
  const _Float16 h = f16_round_up(t);
  const float s = (float)h;
  float z = 0.f;
  if (s > 0.f) z = fminf(fmaxf(__builtin_rintf(-lo / s), 0.f), 15.f);
  v4i words;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32 word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float q = 0.f;
      if (s > 0.f) q = fminf(fmaxf(__builtin_rintf(v[8 * i + e] / s) + z, 0.f), 15.f);
      word |= ((u32)q) << (4 * e);
    }
    words[i] = (int)word;
  }
  st16(wq + n * (K >> 3) + g * 16 + r * 4, words);
  if (r == 0) {
    wscale[n * G + g] = __builtin_bit_cast(uint16_t, h);
    wzero[n * G + g] = __builtin_bit_cast(uint16_t, (_Float16)z);
  }
}

hipError_t launch_quant_weight_u4(const float* w, int64_t K, int64_t N, int32_t* wq,
                                  uint16_t* ws, uint16_t* wz, hipStream_t st) {
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)(K / 128)), block(256);
  k_quant_weight_u4<<<grid, block, 0, st>>>(w, K, N, wq, ws, wz);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// g=128 uint4 weights with the top 3 of each group (by |w|, ties to the lower
// index) kept in an INT8 side store (「LLM推理降本五要素」 §2.2).  Same
// workgroup shape as k_quant_weight_u4.  Each thread picks the top 3 of its 32
// weights; the four quarters' candidates meet in LDS and every thread merges
// them in ascending index order, a candidate entering only if strictly
// larger, so equal magnitudes keep the lower index.  The group's scale and
// zero point come from the other 125 weights; outlier positions get code z.
// The record gets the outliers' indices (ascending) with code bytes 0 and
// slot 3 = 0xFFFF; k_outlier_codes fills in the codes once every group of
// the column is known.
// ---------------------------------------------------------------------------

struct Top3 {
  float m[3];   // magnitudes, descending
  int k[3];     // indices
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      m[i] = -1.f;
      k[i] = 1 << 20;
    }
  }
  // offer in ascending index order: a candidate enters only if strictly larger
  __device__ __forceinline__ void offer(float a, int idx) {
    if (a > m[2]) {
      if (a > m[1]) {
        m[2] = m[1];
        k[2] = k[1];
        if (a > m[0]) {
          m[1] = m[0];
          k[1] = k[0];
          m[0] = a;
          k[0] = idx;
        } else {
          m[1] = a;
          k[1] = idx;
        }
      } else {
        m[2] = a;
        k[2] = idx;
      }
    }
  }
};

__global__ __launch_bounds__(256) void k_quant_weight_u4_outl(const float* __restrict__ w,
                                                              int64_t K, int64_t N,
                                                              int32_t* __restrict__ wq,
                                                              uint16_t* __restrict__ wscale,
                                                              uint16_t* __restrict__ wzero,
                                                              uint64_t* __restrict__ rec) {
  __shared__ float rlo[4][64], rhi[4][64];
  __shared__ int cand[4][64][3];
  const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 64 + c;
  const int64_t g = blockIdx.y;
  const int64_t G = K >> 7;
  float v[32];
  Top3 t3;
  t3.init();
  if (n < N) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = w[(g * 128 + r * 32 + i) * N + n];
      t3.offer(fabsf(v[i]), r * 32 + i);
    }
  }
  // the quarter's candidates by ascending index
  int ks[3] = {t3.k[0], t3.k[1], t3.k[2]};
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2 - a; ++b)
      if (ks[b] > ks[b + 1]) {
        const int tmp = ks[b];
        ks[b] = ks[b + 1];
        ks[b + 1] = tmp;
      }
#pragma unroll
  for (int i = 0; i < 3; ++i) cand[r][c][i] = ks[i];
  __syncthreads();
  const bool valid = n < N;   // no early return: a second barrier follows
  // merge (every thread of the column, redundantly): magnitudes re-read from
  // global memory, in ascending index order
  Top3 all;
  all.init();
  if (valid)
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int kk = cand[q][c][i];
        all.offer(fabsf(w[(g * 128 + kk) * N + n]), kk);
      }
  int o[3] = {all.k[0], all.k[1], all.k[2]};
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2 - a; ++b)
      if (o[b] > o[b + 1]) {
        const int tmp = o[b];
        o[b] = o[b + 1];
        o[b + 1] = tmp;
      }
  bool out[32];
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int kk = r * 32 + i;
    out[i] = kk == o[0] || kk == o[1] || kk == o[2];
    if (valid && !out[i]) {
      lo = fminf(lo, v[i]);
      hi = fmaxf(hi, v[i]);
    }
  }
  rlo[r][c] = lo;
  rhi[r][c] = hi;
  __syncthreads();
  if (!valid) return;
  lo = fminf(fminf(rlo[0][c], rlo[1][c]), fminf(rlo[2][c], rlo[3][c]));
  hi = fmaxf(fmaxf(rhi[0][c], rhi[1][c]), fmaxf(rhi[2][c], rhi[3][c]));
  const float t = (hi - lo) / 15.f;
  const _Float16 h = f16_round_up(t);
  const float s = (float)h;
  float z = 0.f;
  if (s > 0.f) z = fminf(fmaxf(__builtin_rintf(-lo / s), 0.f), 15.f);
  v4i words;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32 word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float q = 0.f;
      if (s > 0.f) q = fminf(fmaxf(__builtin_rintf(v[8 * i + e] / s) + z, 0.f), 15.f);
      if (out[8 * i + e]) q = z;
      word |= ((u32)q) << (4 * e);
    }
    words[i] = (int)word;
  }
  st16(wq + n * (K >> 3) + g * 16 + r * 4, words);
  if (r == 0) {
    wscale[n * G + g] = __builtin_bit_cast(uint16_t, h);
    wzero[n * G + g] = __builtin_bit_cast(uint16_t, (_Float16)z);
    uint64_t rc = (uint64_t)0xFFFF << 48;
#pragma unroll
    for (int i = 0; i < 3; ++i) rc |= (uint64_t)(o[i] << 8) << (16 * i);
    rec[n * G + g] = rc;
  }
}

// ---------------------------------------------------------------------------
// 2:4 structured-sparse g=128 uint4 weights (「LLM推理降本五要素」 §3.2).
// Same workgroup shape as k_quant_weight_u4: thread (column, quarter r) owns
// block r of the group (32 inputs).  In each 4 it keeps the 2 largest |w|
// (strictly larger wins, so ties keep the lower index); the kept weights'
// min / max meet in LDS; each thread then writes its block: two code words
// (value j at bits 8 i + 4 [i >= 4], i = j % 8) and the position word (2 bits
// per kept value), in the 16-channel tile layout.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_weight_u4_sp24(const float* __restrict__ w,
                                                              int64_t K, int64_t N,
                                                              int32_t* __restrict__ wsp,
                                                              uint16_t* __restrict__ wscale,
                                                              uint16_t* __restrict__ wzero) {
  __shared__ float rlo[4][64], rhi[4][64];
  const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 64 + c;
  const int64_t g = blockIdx.y;
  const int64_t G = K >> 7;
  const bool valid = n < N;
  float kv[16];
  u32 posw = 0;
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
  if (valid) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = w[(g * 128 + r * 32 + 4 * t + i) * N + n];
      // top 2 of 4 by |w|, in index order with strict comparisons
      int i0 = 0, i1 = -1;
      float m0 = fabsf(v[0]), m1 = -1.f;
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        const float a = fabsf(v[i]);
        if (a > m0) {
          m1 = m0;
          i1 = i0;
          m0 = a;
          i0 = i;
        } else if (a > m1) {
          m1 = a;
          i1 = i;
        }
      }
      const int pa = i0 < i1 ? i0 : i1, pb = i0 < i1 ? i1 : i0;
      kv[2 * t] = v[pa];
      kv[2 * t + 1] = v[pb];
      posw |= ((u32)pa << (4 * t)) | ((u32)pb << (4 * t + 2));
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        lo = fminf(lo, kv[2 * t + e]);
        hi = fmaxf(hi, kv[2 * t + e]);
      }
    }
  }
  rlo[r][c] = lo;
  rhi[r][c] = hi;
  __syncthreads();
  // channels are stored in tiles of 16: [N/16][G][16][12] words
  int32_t* dst = wsp + (((n >> 4) * G + g) * 16 + (n & 15)) * 12 + 3 * r;
  if (!valid) {
    if (n < ((N + 15) & ~(int64_t)15)) {   // the last tile's rows past N are zero
      dst[0] = 0;
      dst[1] = 0;
      dst[2] = 0;
    }
    return;
  }
  lo = fminf(fminf(rlo[0][c], rlo[1][c]), fminf(rlo[2][c], rlo[3][c]));
  hi = fmaxf(fmaxf(rhi[0][c], rhi[1][c]), fmaxf(rhi[2][c], rhi[3][c]));
  const float t = (hi - lo) / 15.f;
  const _Float16 h = f16_round_up(t);
  const float s = (float)h;
  float z = 0.f;
  if (s > 0.f) z = fminf(fmaxf(__builtin_rintf(-lo / s), 0.f), 15.f);
  u32 cw[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float q = 0.f;
    if (s > 0.f) q = fminf(fmaxf(__builtin_rintf(kv[j] / s) + z, 0.f), 15.f);
    const int i = j & 7;
    cw[j >> 3] |= (u32)q << (i < 4 ? 8 * i : 8 * (i - 4) + 4);
  }
  dst[0] = (int32_t)cw[0];
  dst[1] = (int32_t)cw[1];
  dst[2] = (int32_t)posw;
  if (r == 0) {
    wscale[n * G + g] = __builtin_bit_cast(uint16_t, h);
    wzero[n * G + g] = __builtin_bit_cast(uint16_t, (_Float16)z);
  }
}

hipError_t launch_quant_weight_u4_sp24(const float* w, int64_t K, int64_t N, int32_t* wsp,
                                       uint16_t* ws, uint16_t* wz, hipStream_t st) {
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)(K / 128)), block(256);
  k_quant_weight_u4_sp24<<<grid, block, 0, st>>>(w, K, N, wsp, ws, wz);
  return hipGetLastError();
}

// Per output channel: s8 = max |outlier| / 127 over the channel's records,
// then the outliers' INT8 codes into the records' code bytes.
__global__ __launch_bounds__(256) void k_outlier_codes(const float* __restrict__ w, int64_t K,
                                                       int64_t N, uint64_t* __restrict__ rec,
                                                       float* __restrict__ s8) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int64_t G = K >> 7;
  float amax = 0.f;
  for (int64_t g = 0; g < G; ++g) {
    const uint64_t rc = rec[n * G + g];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int kk = (int)((rc >> (16 * i + 8)) & 0xFF);
      amax = fmaxf(amax, fabsf(w[(g * 128 + kk) * N + n]));
    }
  }
  const float sc = amax / 127.f, rs = sym_code_r(amax, sc);
  s8[n] = amax > 0.f ? sc : 0.f;
  for (int64_t g = 0; g < G; ++g) {
    uint64_t rc = rec[n * G + g];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int kk = (int)((rc >> (16 * i + 8)) & 0xFF);
      const u32 byte = __float_as_uint(sym_code_t(w[(g * 128 + kk) * N + n], sc, rs)) & 0xFFu;
      rc = (rc & ~((uint64_t)0xFF << (16 * i))) | ((uint64_t)byte << (16 * i));
    }
    rec[n * G + g] = rc;
  }
}

hipError_t launch_quant_weight_u4_outl(const float* w, int64_t K, int64_t N, int32_t* wq,
                                       uint16_t* ws, uint16_t* wz, uint64_t* rec, float* s8,
                                       hipStream_t st) {
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)(K / 128)), block(256);
  k_quant_weight_u4_outl<<<grid, block, 0, st>>>(w, K, N, wq, ws, wz, rec);
  if (hipError_t e = hipGetLastError()) return e;
  k_outlier_codes<<<(unsigned)((N + 255) / 256), 256, 0, st>>>(w, K, N, rec, s8);
  return hipGetLastError();
}

}  // namespace qg
