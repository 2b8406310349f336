// Decode W8A8 with the per-token activation quantization fused in: one kernel
// takes the 16-bit (or fp32) token rows, quantizes them into LDS and runs
// the int8 product and its epilogue.
//
// 「第4章：量化」 §1.3 (per-token dynamic quantization), §1.2, §1.1, §2.3 (the
// product on int8 units); 「LLM推理降本五要素」 §2.1 (decode is bound by the
// weight stream), §5.2.
//   s[m] = max_k |x[m,k]| / 127;  xq[m,k] = rint(x[m,k] / s[m]) (codes of
//   sym_code_t, identical to quantize_per_token_i8);
//   acc[m,n] = sum_k xq[m,k] wq[n,k];  y[m,n] = (acc * s[m]) * w_scale[n].
//
// Shape of the kernel.  A workgroup of 16 waves owns BL (1, 2 or 4) blocks of
// 16 weight rows; each block's K is split over 16 / BL waves (wave = split *
// BL + block), and a wave streams its run of whole-line units (two loads of
// 8 rows x 128 bytes, turned into MFMA fragments through a 2 KB wave-private
// LDS tile) with D units in flight in a register ring.  The splits' int32
// partials meet in LDS.  Every workgroup quantizes the MR token rows itself
// -- so the separate quantization launch and its dependency disappear -- but
// only N / (16 BL) workgroups do; each wave works on a single token row (its
// row index, maximum, scale and reciprocal are wave-uniform scalars), each
// thread handles at most 4 chunks of 8 values (16 or 32 bytes each), and
// each wave's first D weight units are already in flight while it does.
// Codes go straight into LDS (row pitch an odd number of 16-byte chunks);
// workgroup 0 also writes the codes and scales out.
//
// The separate quantization pass costs a launch and a dependency; the fused
// prologue costs MR K / 8 chunks of work per workgroup.  With 8 token rows
// of K = 4096 the second is the larger (measured), so the library picks
// this kernel for few rows and a long weight stream, and for 9-16 short
// rows, where the two-kernel path would take the wide GEMM.
#include "qg_decode.hpp"
#include "qg_device.hpp"
#include "qg_launch.hpp"

namespace qg {

constexpr int kFqWaves = 16;    // waves per workgroup: BL blocks x (16 / BL) K splits
constexpr int kFqDepth = 4;     // weight units in flight per wave (8 measured slower)

// Bytes of one activation element, and 16-byte loads per 8-value chunk.
template <int DT>
constexpr int fq_esize() { return DT == F32 ? 4 : 2; }
template <int DT>
constexpr int fq_loads() { return DT == F32 ? 2 : 1; }

template <int DT>
__device__ __forceinline__ void fq_widen8(const v4i (&raw)[fq_loads<DT>()], float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (DT == F32) {
      v[e] = __int_as_float(raw[0][e]);
      v[4 + e] = __int_as_float(raw[fq_loads<DT>() - 1][e]);
    } else {
      const u32 u = (u32)raw[0][e];
      if constexpr (DT == BF16) {
        v[2 * e] = bf16_bits_to_f32(u & 0xFFFFu);
        v[2 * e + 1] = bf16_bits_to_f32(u >> 16);
      } else {
        v[2 * e] = f16_bits_to_f32((uint16_t)(u & 0xFFFFu));
        v[2 * e + 1] = f16_bits_to_f32((uint16_t)(u >> 16));
      }
    }
  }
}

// MR token rows of K values of type DT (F32, F16 or BF16); CPT 8-value
// chunks per thread (K / 8 <= 64 (kFqWaves / MR) CPT).
template <int MR, int CPT, int BL, int DT, typename OutT>
__global__ __launch_bounds__(64 * kFqWaves) void k_w8a8_fq(
    const void* __restrict__ x, const int8_t* __restrict__ wq, const float* __restrict__ ws,
    int M, int N, int K, OutT* __restrict__ y, int8_t* __restrict__ xq_out,
    float* __restrict__ xs_out) {
  constexpr int kFqSplit = kFqWaves / BL;
  extern __shared__ __attribute__((aligned(16))) int8_t xl[];   // MR code rows, pitch stage_pitch(K)
  __shared__ __attribute__((aligned(16))) int8_t tiles[kFqWaves][kTileBytes];
  __shared__ v4i red[kFqWaves][64];
  __shared__ float rmax[kFqWaves][1];
  __shared__ float srow[16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blk = wave % BL, split = wave / BL;
  const int r = lane & 15, j = lane >> 4;
  const int n_base = (blockIdx.x * BL + blk) * 16;
  const int units = (K + kUnitBytes - 1) / kUnitBytes;
  const int ub = units * split / kFqSplit, ue = units * (split + 1) / kFqSplit;
  const int pitch = stage_pitch(K);
  const int cpr = K >> 3;                        // 8-value chunks per token row

  // 1. token rows first (vmcnt retires in issue order: loads issued after
  //    them stay in flight while they are used).  Row m belongs to waves
  //    m * WPR .. m * WPR + WPR - 1 (WPR = kFqWaves / MR), so a wave's row is
  //    a scalar; lane l of the row's wave part p takes chunks
  //    p * 64 * CPT + l + 64 i (i < CPT) of the row's cpr chunks.
  constexpr int WPR = kFqWaves / MR;
  const int m_w = wave / WPR, part = wave % WPR;        // wave-uniform
  constexpr int kL = fq_loads<DT>();
  const rsrc_t xr = make_rsrc(x, (u32)(M * K * fq_esize<DT>()));
  v4i raw[CPT][kL];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ch = part * 64 * CPT + lane + 64 * i;
    const u32 off = m_w < M && ch < cpr ? (u32)(16 * kL * (m_w * cpr + ch)) : kOOB;
#pragma unroll
    for (int l = 0; l < kL; ++l) raw[i][l] = bld16(xr, off + 16 * l);   // kOOB + 16: still out
  }
  // 2. this wave's first kFqDepth weight units, in flight during the
  //    quantization below
  const int rows_n = max(0, min(16, N - n_base));
  const rsrc_t wr = make_rsrc_uniform(wq + (int64_t)min(n_base, N) * K, (u32)(rows_n * K));
  const UnitLanes ul = unit_lanes(lane, K);
  v4i b[kFqDepth][2];
#pragma unroll
  for (int d = 0; d < kFqDepth; ++d) unit_load(b[d], wr, ul, ub + d, ub + d < ue, K);
  __builtin_amdgcn_sched_barrier(0);

  float v[CPT][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    fq_widen8<DT>(raw[i], v[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));   // zeros past the row
  }
  amax = wave_max_nonneg(amax);
  if (lane == 0) rmax[wave][0] = amax;
  __syncthreads();
  // row m_w's max over its WPR waves; scale and reciprocal (uniform)
  float a = rmax[m_w * WPR][0];
#pragma unroll
  for (int p = 1; p < WPR; ++p) a = fmaxf(a, rmax[m_w * WPR + p][0]);
  const float s = a > 0.f ? a / 127.f : 0.f, rr = sym_code_r(a, a / 127.f);
  if (part == 0 && lane == 0) {
    srow[m_w] = s;
    if (blockIdx.x == 0 && m_w < M) xs_out[m_w] = s;
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ch = part * 64 * CPT + lane + 64 * i;
    if (ch < cpr) {
      const u32 w0 = pack_code_bytes(sym_code_t(v[i][0], s, rr), sym_code_t(v[i][1], s, rr),
                                     sym_code_t(v[i][2], s, rr), sym_code_t(v[i][3], s, rr));
      const u32 w1 = pack_code_bytes(sym_code_t(v[i][4], s, rr), sym_code_t(v[i][5], s, rr),
                                     sym_code_t(v[i][6], s, rr), sym_code_t(v[i][7], s, rr));
      *reinterpret_cast<uint2*>(xl + m_w * pitch + 8 * ch) = uint2{w0, w1};
      if (blockIdx.x == 0 && m_w < M)
        *reinterpret_cast<uint2*>(xq_out + (int64_t)m_w * K + 8 * ch) = uint2{w0, w1};
    }
  }
  __syncthreads();

  // 3. the weight stream: unit q's fragments against token chunk q of the
  //    staged rows; rows r >= MR read row 0 (their outputs are never stored)
  const int8_t* xrow = xl + (r < MR ? r : 0) * pitch;
  int8_t* tile = tiles[wave];
  v4i acc = {0, 0, 0, 0};
  for (int q0 = ub; q0 < ue; q0 += kFqDepth) {
#pragma unroll
    for (int d = 0; d < kFqDepth; ++d) {
      const int q = q0 + d;
      v4i f[2];
      unit_transpose(tile, b[d], ul, f);
      unit_load(b[d], wr, ul, q + kFqDepth, q + kFqDepth < ue, K);   // refill the slot
      const bool qin = q < ue;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int ka = kUnitBytes * q + 64 * s + 16 * j;
        const v4i a = ld16(xrow + (qin && ka < K ? ka : 0));
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, f[s], acc, 0, 0, 0);
      }
    }
  }

  // 4. the splits' partials meet in LDS; the split-0 wave of each block
  //    writes its 16 x 16 outputs (lane (r, j): tokens 4 j + i of row n_base + r)
  red[wave][lane] = acc;
  __syncthreads();
  if (split != 0) return;
  v4i sum = red[blk][lane];
#pragma unroll
  for (int sp = 1; sp < kFqSplit; ++sp) sum += red[sp * BL + blk][lane];
  const int n = n_base + r;
  if (n < N) {
    if constexpr (__is_same(OutT, int32_t)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * j + i;
        if (m < M) y[(int64_t)m * N + n] = sum[i];
      }
    } else {
      const float sw = ws[n];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * j + i;
        if (m < M) y[(int64_t)m * N + n] = Out<OutT>::cvt(((float)sum[i] * srow[m]) * sw);
      }
    }
  }
}

template <int MR, int BL, int DT, typename OutT>
static hipError_t fq_bl(const void* x, const int8_t* wq, const float* ws, int M, int N, int K,
                        OutT* y, int8_t* xq, float* xs, hipStream_t st) {
  const size_t lds = (size_t)MR * stage_pitch(K);
  // a row's K / 8 chunks over kFqWaves / MR waves: cpt per lane
  const int chunks = MR * (K / 8), cpt = (chunks + 64 * kFqWaves - 1) / (64 * kFqWaves);
  const dim3 grid((unsigned)((N + 16 * BL - 1) / (16 * BL))), block(64 * kFqWaves);
  if (cpt <= 1) k_w8a8_fq<MR, 1, BL, DT, OutT><<<grid, block, lds, st>>>(x, wq, ws, M, N, K, y, xq, xs);
  else if (cpt <= 2) k_w8a8_fq<MR, 2, BL, DT, OutT><<<grid, block, lds, st>>>(x, wq, ws, M, N, K, y, xq, xs);
  else k_w8a8_fq<MR, 4, BL, DT, OutT><<<grid, block, lds, st>>>(x, wq, ws, M, N, K, y, xq, xs);
  return hipGetLastError();
}

// Blocks per workgroup: every workgroup repeats the quantization, so fewer,
// larger workgroups cost less, but a grid under about kFqMinGroups (of 256
// compute units) streams the weights more slowly (measured on MI355X): the
// most blocks that still leave that many workgroups.
constexpr int kFqMinGroups = 160;

template <int MR, int DT, typename OutT>
static hipError_t fq_mr(const void* x, const int8_t* wq, const float* ws, int M, int N, int K,
                        OutT* y, int8_t* xq, float* xs, hipStream_t st) {
  const int blocks = (N + 15) / 16;
  if (blocks >= 4 * kFqMinGroups) return fq_bl<MR, 4, DT, OutT>(x, wq, ws, M, N, K, y, xq, xs, st);
  if (blocks >= 2 * kFqMinGroups) return fq_bl<MR, 2, DT, OutT>(x, wq, ws, M, N, K, y, xq, xs, st);
  return fq_bl<MR, 1, DT, OutT>(x, wq, ws, M, N, K, y, xq, xs, st);
}

template <int DT, typename OutT>
static hipError_t fq_dt(const void* x, const int8_t* wq, const float* ws, int M, int N, int K,
                        OutT* y, int8_t* xq, float* xs, hipStream_t st) {
  if (M <= 1) return fq_mr<1, DT, OutT>(x, wq, ws, M, N, K, y, xq, xs, st);
  if (M <= 2) return fq_mr<2, DT, OutT>(x, wq, ws, M, N, K, y, xq, xs, st);
  if (M <= 4) return fq_mr<4, DT, OutT>(x, wq, ws, M, N, K, y, xq, xs, st);
  if (M <= 8) return fq_mr<8, DT, OutT>(x, wq, ws, M, N, K, y, xq, xs, st);
  return fq_mr<16, DT, OutT>(x, wq, ws, M, N, K, y, xq, xs, st);
}

// Token rows handled by one launch: M rounded up to 1, 2, 4, 8 or 16.
static int64_t fq_rows(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

// The fused kernel covers M <= 16 token rows whose codes fit the LDS budget
// and a thread's registers (rows x K / 8 <= 4 chunks x 1024 threads).
bool fq_fused_fits(int x_dtype, int64_t M, int64_t K) {
  const int64_t mr = fq_rows(M);
  return (x_dtype == F32 || x_dtype == BF16 || x_dtype == F16) && M >= 1 && M <= 16 &&
         (size_t)mr * stage_pitch((int)K) <= kDecLdsMaxBytes && mr * (K / 8) <= 4 * 64 * kFqWaves;
}

// Where it pays (measured on MI355X against the two kernels in sequence):
// with few token rows and a long weight stream the repeated quantization is
// hidden behind the first weight loads, and one launch and its dependency
// are saved; with 9-16 short rows (K <= 768) the two-kernel path would take
// the wide GEMM, and the single launch is the shorter chain.  Elsewhere the
// repeated quantization costs more than the separate pass.
static bool fq_fused_pays(int64_t M, int64_t N, int64_t K) {
  return (M <= 4 && N * K >= (int64_t(1) << 25)) || (M > 8 && K <= 768);
}

bool quantize_gemm_w8a8_fused(int x_dtype, int64_t M, int64_t N, int64_t K, int fuse) {
  return M > 0 && N > 0 && fuse != kFuseNever && fq_fused_fits(x_dtype, M, K) &&
         (fuse == kFuseFit || fq_fused_pays(M, N, K));
}

template <int DT>
static hipError_t fq_xt(const void* x, const int8_t* wq, const float* ws, int m, int n, int k,
                        void* y, int y_dtype, int8_t* xq, float* xs, hipStream_t st) {
  switch (y_dtype) {
    case F32: return fq_dt<DT, float>(x, wq, ws, m, n, k, (float*)y, xq, xs, st);
    case F16: return fq_dt<DT, _Float16>(x, wq, ws, m, n, k, (_Float16*)y, xq, xs, st);
    case BF16: return fq_dt<DT, uint16_t>(x, wq, ws, m, n, k, (uint16_t*)y, xq, xs, st);
    default: return fq_dt<DT, int32_t>(x, wq, ws, m, n, k, (int32_t*)y, xq, xs, st);
  }
}

hipError_t launch_quantize_gemm_w8a8(const void* x, int x_dtype, const int8_t* wq,
                                     const float* ws, int64_t M, int64_t N, int64_t K, void* y,
                                     int y_dtype, int8_t* xq, float* xs, int fuse, hipStream_t st) {
  if (!quantize_gemm_w8a8_fused(x_dtype, M, N, K, fuse)) {
    if (hipError_t e = launch_quant_per_token(x, x_dtype, M, K, xq, xs, st)) return e;
    return launch_gemm_w8a8(xq, xs, wq, ws, M, N, K, y, y_dtype, st);
  }
  const int m = (int)M, n = (int)N, k = (int)K;
  switch (x_dtype) {
    case F32: return fq_xt<F32>(x, wq, ws, m, n, k, y, y_dtype, xq, xs, st);
    case F16: return fq_xt<F16>(x, wq, ws, m, n, k, y, y_dtype, xq, xs, st);
    default: return fq_xt<BF16>(x, wq, ws, m, n, k, y, y_dtype, xq, xs, st);
  }
}

}  // namespace qg
