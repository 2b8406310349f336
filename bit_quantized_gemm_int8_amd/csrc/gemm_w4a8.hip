// W4A8 GEMM with g=128 asymmetric uint4 weights dequantized inside the kernel.
// 「LLM推理降本五要素」 §2.2 (W4A8, group size 128, per-group scale and zero
// point); 「第4章：量化」 §1.1 (x_hat = (x_int - z) s) and §3.5 (fuse the
// dequantization into the GEMM rather than running a separate pass).
//
// Per group g of 128 input channels (exact int32):
//   acc[m,g,n] = sum_{k in g} xq[m,k] q[n,k]  -  z[n,g] * sum_{k in g} xq[m,k]
// then y[m,n] = s_x[m] * sum_g s[n,g] * acc[m,g,n] in binary32.
//
// Unpack in registers: a packed word holds 8 codes (nibble j = k 8i+j);
// w & 0x0F0F0F0F gives the even-k codes as bytes and (w >> 4) & 0x0F0F0F0F the
// odd-k codes -- each already a valid int8 operand (0..15).  The activation
// bytes are shuffled into the same [0,2,4,6,1,3,5,7] order, so the matrix core
// pairs every code with its own activation.  The zero point enters once per
// group through the token sums sum_k xq[m,k], which one extra MFMA against an
// all-ones operand produces in the accumulator layout.
#include "qg_decode.hpp"
#include "qg_device.hpp"
#include "qg_launch.hpp"

#include <algorithm>

namespace qg {

// bytes [b0..b7] of (lo, hi) -> [b0 b2 b4 b6 | b1 b3 b5 b7]
__device__ __forceinline__ void even_odd_bytes(u32 lo, u32 hi, u32& e, u32& o) {
  e = __builtin_amdgcn_perm(hi, lo, 0x06040200u);
  o = __builtin_amdgcn_perm(hi, lo, 0x07050301u);
}

__device__ __forceinline__ v4i shuffle_act16(v4i x) {
  v4i r;
  u32 e, o;
  even_odd_bytes((u32)x[0], (u32)x[1], e, o);
  r[0] = (int)e;
  r[1] = (int)o;
  even_odd_bytes((u32)x[2], (u32)x[3], e, o);
  r[2] = (int)e;
  r[3] = (int)o;
  return r;
}

__device__ __forceinline__ v4i unpack_u4_pair(u32 w0, u32 w1) {
  return v4i{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu), (int)(w1 & 0x0F0F0F0Fu),
             (int)((w1 >> 4) & 0x0F0F0F0Fu)};
}

template <typename OutT>
__device__ __forceinline__ void store_out(OutT* y, int64_t idx, float v) {
  y[idx] = Out<OutT>::cvt(v);
}

template <int MT, int NT, int U>
struct W4A8Batch {
  v4i wv[U][NT], xa[U][MT][2];
  uint16_t sbits[U][NT], zbits[U][NT];
};

// Issue the loads of groups [g0, g0 + U) (those below ge; the rest read zeros).
template <int MT, int NT, int U>
__device__ __forceinline__ void w4a8_load(W4A8Batch<MT, NT, U>& bt, int g0, int ge, rsrc_t wr,
                                          const u32 (&woff)[NT], rsrc_t sr, rsrc_t zr,
                                          const u32 (&soff)[NT], rsrc_t xr,
                                          const u32 (&xoff)[MT]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = g0 + u;
    const bool gin = g < ge;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bt.wv[u][t] = bld16_nt(wr, gin ? woff[t] + 64 * g : kOOB);
      bt.sbits[u][t] = bld2(sr, gin ? soff[t] + 2 * g : kOOB);
      bt.zbits[u][t] = bld2(zr, gin ? soff[t] + 2 * g : kOOB);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      bt.xa[u][mt][0] = bld16(xr, gin ? xoff[mt] + 128 * g : kOOB);
      bt.xa[u][mt][1] = bld16(xr, gin ? xoff[mt] + 128 * g + 16 : kOOB);
    }
  }
  // keep the whole batch of loads ahead of the multiplies that follow
  __builtin_amdgcn_sched_barrier(0);
}

// Multiply the groups of a batch; float mode accumulates s * acc into yacc,
// int32 mode writes the per-group accumulators.
template <int MT, int NT, int U, typename OutT>
__device__ __forceinline__ void w4a8_mma(const W4A8Batch<MT, NT, U>& bt, int g0, int ge, int G,
                                         int N, int M, int m_base, int j, const int (&ncol)[NT],
                                         const bool (&nok)[NT], v4f (&yacc)[MT][NT],
                                         OutT* __restrict__ y) {
  constexpr bool kI32 = __is_same(OutT, int32_t);
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = g0 + u;          // g >= ge: zero operands, zero contribution
    v4i a[MT][2], rs[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      a[mt][0] = shuffle_act16(bt.xa[u][mt][0]);
      a[mt][1] = shuffle_act16(bt.xa[u][mt][1]);
      rs[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt][0], ones, v4i{0, 0, 0, 0}, 0, 0, 0);
      rs[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt][1], ones, rs[mt], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const v4i b0 = unpack_u4_pair((u32)bt.wv[u][t][0], (u32)bt.wv[u][t][1]);
      const v4i b1 = unpack_u4_pair((u32)bt.wv[u][t][2], (u32)bt.wv[u][t][3]);
      const int z = (int)f16_bits_to_f32(bt.zbits[u][t]);
      const float s = f16_bits_to_f32(bt.sbits[u][t]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v4i acc;   // |z| <= 15, |token sum| <= 128 * 127: 24-bit multiplies are exact
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __mul24(-z, rs[mt][i]);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt][0], b0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt][1], b1, acc, 0, 0, 0);
        if constexpr (kI32) {
          if (nok[t] && g < ge) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = m_base + 16 * mt + 4 * j + i;
              if (m < M) y[((int64_t)m * G + g) * N + ncol[t]] = acc[i];
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) yacc[mt][t][i] = __builtin_fmaf(s, (float)acc[i], yacc[mt][t][i]);
        }
      }
    }
  }
}

// Workgroup = WAVES waves owning 16*NT output columns and 16*MT rows; the
// groups of K are split across the waves (contiguous runs), walked in batches
// of U groups with the next batch's loads issued before the current batch is
// multiplied.  Lane l: MFMA row/column (l & 15); within a group, words
// 4j..4j+3 of its column with j = l >> 4 (one 16-byte load), of which MFMA h
// takes words 4j+2h and 4j+2h+1 (k = 32j + 16h + 0..15).
template <int MT, int NT, int WAVES, int U, typename OutT>
__global__ __launch_bounds__(64 * WAVES) void k_w4a8(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, const int32_t* __restrict__ wq,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero, int M, int N, int K,
    OutT* __restrict__ y) {
  constexpr bool kI32 = __is_same(OutT, int32_t);
  __shared__ v4f red[kI32 ? 1 : WAVES][MT][NT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int n_base = blockIdx.x * 16 * NT;
  const int m_base = blockIdx.y * 16 * MT;
  const int G = K >> 7, Kw = K >> 3;
  const int gb = (int)((int64_t)G * wave / WAVES), ge = (int)((int64_t)G * (wave + 1) / WAVES);

  bool nok[NT];
  int ncol[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    ncol[t] = n_base + 16 * t + r;
    nok[t] = ncol[t] < N;
  }
  // buffer resources cover this workgroup's weight columns and token rows;
  // columns past N and rows past M read as zeros
  const int rows_n = min(16 * NT, N - n_base), rows_m = min(16 * MT, M - m_base);
  const rsrc_t wr = make_rsrc(wq + (int64_t)n_base * Kw, (u32)(rows_n * Kw * 4));
  const rsrc_t sr = make_rsrc(wscale + (int64_t)n_base * G, (u32)(rows_n * G * 2));
  const rsrc_t zr = make_rsrc(wzero + (int64_t)n_base * G, (u32)(rows_n * G * 2));
  const rsrc_t xr = make_rsrc(xq + (int64_t)m_base * K, (u32)(rows_m * K));
  u32 woff[NT], soff[NT], xoff[MT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    woff[t] = (u32)(((16 * t + r) * Kw + 4 * j) * 4);
    soff[t] = (u32)((16 * t + r) * G * 2);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xoff[mt] = (u32)((16 * mt + r) * K + 32 * j);

  v4f yacc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) yacc[mt][t] = v4f{0.f, 0.f, 0.f, 0.f};

  W4A8Batch<MT, NT, U> p0, p1;
  w4a8_load(p0, gb, ge, wr, woff, sr, zr, soff, xr, xoff);
  // Branch-free software pipeline: groups past this wave's range read zeros
  // (and add zero), so each batch waits only for its own loads.
  for (int g0 = gb; g0 < ge; g0 += 2 * U) {
    w4a8_load(p1, g0 + U, ge, wr, woff, sr, zr, soff, xr, xoff);
    w4a8_mma(p0, g0, ge, G, N, M, m_base, j, ncol, nok, yacc, y);
    w4a8_load(p0, g0 + 2 * U, ge, wr, woff, sr, zr, soff, xr, xoff);
    w4a8_mma(p1, g0 + U, ge, G, N, M, m_base, j, ncol, nok, yacc, y);
  }

  if constexpr (!kI32) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) red[wave][mt][t][lane] = yacc[mt][t];
    __syncthreads();
    for (int it = threadIdx.x; it < MT * NT * 64; it += 64 * WAVES) {
      const int l = it & 63, t = (it >> 6) % NT, mt = (it >> 6) / NT;
      v4f sum = red[0][mt][t][l];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][mt][t][l];
      const int n = n_base + 16 * t + (l & 15);
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m_base + 16 * mt + 4 * (l >> 4) + i;
        if (m < M) store_out<OutT>(y, (int64_t)m * N + n, sum[i] * xs[m]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 16) on whole-line weight units (see qg_decode.hpp): a
// unit is two g=128 groups of 16 weight rows.  Scales and zero points are
// staged in LDS; the token rows (up to 16 x K bytes, too many to stage whole
// for long K) come straight from the L2 into the MFMA operand registers with
// the unit they belong to.  Wave w streams its contiguous run of units in
// batches of UB, two batches in flight.
// ---------------------------------------------------------------------------
template <int UB, bool OUTL>
struct W4A8DecBatch {
  v4i w[UB][2], xa[UB][2][2];   // unit v: weight loads; group s, MFMA h token fragment
  v4i orc[OUTL ? UB : 1];       // unit v: the two groups' outlier records
};

// Outlier-retention side path (「LLM推理降本五要素」 §2.2).  A group's record
// holds three (index << 8 | code byte) slots.  For one MFMA of the group, lane
// (row r, k-block j) covers the 16 inputs k = 32 j + 16 h + [0, 16) of weight
// row r; the slots falling there are placed at their byte positions, giving a
// sparse int8 operand whose product with the raw (unpermuted) token fragment
// accumulates sum_k x_q[m, k] * code exactly in int32.
__device__ __forceinline__ v4i outlier_operand(u32 lo, u32 hi, int kb) {
  uint64_t b0 = 0, b1 = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const u32 slot = (i == 0 ? lo : i == 1 ? lo >> 16 : hi) & 0xFFFFu;
    const int pos = (int)(slot >> 8) - kb;
    const uint64_t v = (uint64_t)(slot & 0xFFu) << (8 * (pos & 7));
    b0 |= (u32)pos < 8u ? v : 0;
    b1 |= (u32)(pos - 8) < 8u ? v : 0;
  }
  return v4i{(int)(u32)b0, (int)(u32)(b0 >> 32), (int)(u32)b1, (int)(u32)(b1 >> 32)};
}

template <int MR, int WAVES, int UB, bool OUTL, typename OutT>
__global__ __launch_bounds__(64 * WAVES) void k_w4a8_dec(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, const int32_t* __restrict__ wq,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero,
    const uint64_t* __restrict__ orec, const float* __restrict__ os8, int M, int N, int K,
    OutT* __restrict__ y) {
  constexpr bool kI32 = __is_same(OutT, int32_t);
  constexpr int kThreads = 64 * WAVES;
  extern __shared__ __attribute__((aligned(16))) u32 szl[];   // 16 x sz_pitch(G) words
  __shared__ __attribute__((aligned(16))) int8_t tiles[WAVES][kTileBytes];
  __shared__ v4f red[kI32 ? 1 : WAVES][64];
  __shared__ v4i redo[OUTL ? WAVES : 1][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int n_base = blockIdx.x * 16;
  const int G = K >> 7, Kw = K >> 3, RB = Kw * 4;
  const int GY = OUTL ? G + 1 : G;   // int32 output slices per token: groups (+ side sum)
  const int units = (RB + kUnitBytes - 1) / kUnitBytes;
  const int ub = (int)((int64_t)units * wave / WAVES), ue = (int)((int64_t)units * (wave + 1) / WAVES);

  const int rows_n = min(16, N - n_base);
  const rsrc_t wr = make_rsrc(wq + (int64_t)n_base * Kw, (u32)(rows_n * RB));
  const UnitLanes ul = unit_lanes(lane, RB);
  // token row r (rows >= M past the resource's end read zeros), k = 32j + 16h
  const rsrc_t xr = make_rsrc(xq, (u32)(M * K));
  const u32 xoff = (u32)((r < MR ? r : MR) * K + 32 * j);
  // outlier records of row r: unit q's two groups are 16 bytes at 16 q
  const rsrc_t orr = OUTL ? make_rsrc(orec + (int64_t)n_base * G, (u32)(rows_n * G * 8)) : wr;
  const u32 ooff = (u32)(r * G * 8);

  using Batch = W4A8DecBatch<UB, OUTL>;
  auto load = [&](Batch& bt, int q0) {
#pragma unroll
    for (int v = 0; v < UB; ++v) {
      const int q = q0 + v;
      unit_load(bt.w[v], wr, ul, q, q < ue, RB);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int g = 2 * q + s;
        const bool gin = q < ue && g < G;
#pragma unroll
        for (int h = 0; h < 2; ++h) bt.xa[v][s][h] = bld16(xr, gin ? xoff + 128 * g + 16 * h : kOOB);
      }
      if constexpr (OUTL) bt.orc[v] = bld16(orr, q < ue ? ooff + 16 * q : kOOB);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  Batch b0, b1;
  ScaleZeroStage<kThreads, 4> sz;
  const rsrc_t sr = make_rsrc(wscale + (int64_t)n_base * G, (u32)(rows_n * G * 2));
  const rsrc_t zr = make_rsrc(wzero + (int64_t)n_base * G, (u32)(rows_n * G * 2));
  sz.load(sr, zr, 16 * G, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(b0, ub);
  float sx[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!kI32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * j + i;
      sx[i] = xs[m < M ? m : M - 1];
    }
  }
  sz.finish(sr, zr, szl, G, 16 * G);
  lds_barrier();

  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const u32* szrow = szl + r * sz_pitch(G);
  int8_t* tile = tiles[wave];
  v4f yacc = {0.f, 0.f, 0.f, 0.f};
  v4i oacc = {0, 0, 0, 0};
  auto mma = [&](const Batch& bt, int q0) {
#pragma unroll
    for (int v = 0; v < UB; ++v) {
      v4i f[2];
      unit_transpose(tile, bt.w[v], ul, f);
      const int q = q0 + v;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // groups past this wave's run or past G: zero codes, zero point and scale
        const int g = 2 * q + s;
        const bool gin = q < ue && g < G;
        const u32 szw = gin ? szrow[g] : 0u;
        const v4i a0 = shuffle_act16(bt.xa[v][s][0]), a1 = shuffle_act16(bt.xa[v][s][1]);
        v4i rs = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, ones, v4i{0, 0, 0, 0}, 0, 0, 0);
        rs = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, ones, rs, 0, 0, 0);
        const int z = (int)f16_bits_to_f32((uint16_t)(szw >> 16));
        // |z| <= 15 and |token sum| <= 128 * 127: the 24-bit multiply is exact
        v4i acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __mul24(-z, rs[i]);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, unpack_u4_pair((u32)f[s][0], (u32)f[s][1]),
                                                    acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, unpack_u4_pair((u32)f[s][2], (u32)f[s][3]),
                                                    acc, 0, 0, 0);
        if constexpr (OUTL) {
          // a group past G (odd G) or past the run has a zero token fragment
          const u32 lo = (u32)bt.orc[v][2 * s], hi = (u32)bt.orc[v][2 * s + 1];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            oacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(bt.xa[v][s][h],
                                                         outlier_operand(lo, hi, 32 * j + 16 * h),
                                                         oacc, 0, 0, 0);
        }
        if constexpr (kI32) {
          const int n = n_base + r;
          if (gin && n < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = 4 * j + i;
              if (m < M) y[((int64_t)m * GY + g) * N + n] = acc[i];
            }
          }
        } else {
          const float sc = f16_bits_to_f32((uint16_t)(szw & 0xFFFFu));
#pragma unroll
          for (int i = 0; i < 4; ++i) yacc[i] = __builtin_fmaf(sc, (float)acc[i], yacc[i]);
        }
      }
    }
  };
  for (int q0 = ub; q0 < ue; q0 += 2 * UB) {
    load(b1, q0 + UB);
    mma(b0, q0);
    load(b0, q0 + 2 * UB);
    mma(b1, q0 + UB);
  }

  if constexpr (!kI32) red[wave][lane] = yacc;
  if constexpr (OUTL) redo[wave][lane] = oacc;
  if constexpr (!kI32 || OUTL) {
    __syncthreads();
    if (tid < 64) {
      const int n = n_base + r;
      v4i osum = {0, 0, 0, 0};
      if constexpr (OUTL) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) osum += redo[w][lane];
      }
      if (n < N) {
        if constexpr (kI32) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 4 * j + i;
            if (m < M) y[((int64_t)m * GY + G) * N + n] = osum[i];
          }
        } else {
          v4f sum = red[0][lane];
#pragma unroll
          for (int w = 1; w < WAVES; ++w) sum += red[w][lane];
          const float s8 = OUTL ? os8[n] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 4 * j + i;
            // y = s_x (sum_g s_g acc_g + s8 acc_o)
            const float t = OUTL ? __builtin_fmaf(s8, (float)osum[i], sum[i]) : sum[i];
            if (m < M) store_out<OutT>(y, (int64_t)m * N + n, t * sx[i]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode kernel for 16 < M <= 16 MT token rows: as k_w4a8_dec (whole-line
// units, scales and zero points staged in LDS, waves splitting K), but each
// group's codes are unpacked once and multiplied against MT tiles of 16
// token rows, so the weights stream once for all of them.  The token
// fragments of every tile come straight from L2 with the unit they belong to.
// ---------------------------------------------------------------------------
template <int MT, int UB>
struct W4A8MtBatch {
  v4i w[UB][2], xa[UB][2][MT][2];   // unit v: weight loads; group s, tile t, MFMA h fragment
};

template <int MT, int WAVES, int UB, typename OutT>
__global__ __launch_bounds__(64 * WAVES) void k_w4a8_dec_mt(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, const int32_t* __restrict__ wq,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero, int M, int N, int K,
    OutT* __restrict__ y) {
  constexpr bool kI32 = __is_same(OutT, int32_t);
  constexpr int kThreads = 64 * WAVES;
  extern __shared__ __attribute__((aligned(16))) u32 szl[];   // 16 x sz_pitch(G) words
  __shared__ __attribute__((aligned(16))) int8_t tiles[WAVES][kTileBytes];
  __shared__ v4f red[kI32 ? 1 : WAVES][MT][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int n_base = blockIdx.x * 16;
  const int G = K >> 7, Kw = K >> 3, RB = Kw * 4;
  const int units = (RB + kUnitBytes - 1) / kUnitBytes;
  const int ub = (int)((int64_t)units * wave / WAVES), ue = (int)((int64_t)units * (wave + 1) / WAVES);

  const int rows_n = min(16, N - n_base);
  const rsrc_t wr = make_rsrc(wq + (int64_t)n_base * Kw, (u32)(rows_n * RB));
  const UnitLanes ul = unit_lanes(lane, RB);
  // token row 16 t + r of tile t (rows past M lie past the resource's end:
  // zeros), k = 32j + 16h of the group
  const rsrc_t xr = make_rsrc(xq, (u32)(M * K));
  u32 xoff[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xoff[t] = (u32)((16 * t + r) * K + 32 * j);

  using Batch = W4A8MtBatch<MT, UB>;
  auto load = [&](Batch& bt, int q0) {
#pragma unroll
    for (int v = 0; v < UB; ++v) {
      const int q = q0 + v;
      unit_load(bt.w[v], wr, ul, q, q < ue, RB);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int g = 2 * q + s;
        const bool gin = q < ue && g < G;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            bt.xa[v][s][t][h] = bld16(xr, gin ? xoff[t] + 128 * g + 16 * h : kOOB);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  Batch b0, b1;
  ScaleZeroStage<kThreads, 4> sz;
  const rsrc_t sr = make_rsrc(wscale + (int64_t)n_base * G, (u32)(rows_n * G * 2));
  const rsrc_t zr = make_rsrc(wzero + (int64_t)n_base * G, (u32)(rows_n * G * 2));
  sz.load(sr, zr, 16 * G, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(b0, ub);
  sz.finish(sr, zr, szl, G, 16 * G);
  lds_barrier();

  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const u32* szrow = szl + r * sz_pitch(G);
  int8_t* tile = tiles[wave];
  v4f yacc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) yacc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const Batch& bt, int q0) {
#pragma unroll
    for (int v = 0; v < UB; ++v) {
      v4i f[2];
      unit_transpose(tile, bt.w[v], ul, f);
      const int q = q0 + v;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // groups past this wave's run or past G: zero codes, zero point and scale
        const int g = 2 * q + s;
        const bool gin = q < ue && g < G;
        const u32 szw = gin ? szrow[g] : 0u;
        const int z = (int)f16_bits_to_f32((uint16_t)(szw >> 16));
        const float sc = f16_bits_to_f32((uint16_t)(szw & 0xFFFFu));
        const v4i w0 = unpack_u4_pair((u32)f[s][0], (u32)f[s][1]);
        const v4i w1 = unpack_u4_pair((u32)f[s][2], (u32)f[s][3]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const v4i a0 = shuffle_act16(bt.xa[v][s][t][0]), a1 = shuffle_act16(bt.xa[v][s][t][1]);
          v4i rs = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, ones, v4i{0, 0, 0, 0}, 0, 0, 0);
          rs = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, ones, rs, 0, 0, 0);
          // |z| <= 15 and |token sum| <= 128 * 127: the 24-bit multiply is exact
          v4i acc;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = __mul24(-z, rs[i]);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, w0, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, w1, acc, 0, 0, 0);
          if constexpr (kI32) {
            const int n = n_base + r;
            if (gin && n < N) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int m = 16 * t + 4 * j + i;
                if (m < M) y[((int64_t)m * G + g) * N + n] = acc[i];
              }
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) yacc[t][i] = __builtin_fmaf(sc, (float)acc[i], yacc[t][i]);
          }
        }
      }
    }
  };
  for (int q0 = ub; q0 < ue; q0 += 2 * UB) {
    load(b1, q0 + UB);
    mma(b0, q0);
    load(b0, q0 + 2 * UB);
    mma(b1, q0 + UB);
  }

  if constexpr (!kI32) {
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][t][lane] = yacc[t];
    __syncthreads();
    for (int it = tid; it < MT * 64; it += kThreads) {
      const int l = it & 63, t = it >> 6;
      v4f sum = red[0][t][l];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][t][l];
      const int n = n_base + (l & 15);
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * t + 4 * (l >> 4) + i;
        if (m < M) store_out<OutT>(y, (int64_t)m * N + n, sum[i] * xs[m]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode kernel for wide layers (M <= 16, N / 32 >= 256): each wave streams
// two 16-row weight blocks over its run of K, so one token fragment -- and
// one token-sum MFMA -- serves both blocks' codes: half the token traffic
// and a third fewer MFMAs per weight byte, at half as many workgroups.
// Otherwise as k_w4a8_dec (scales and zero points of the 32 rows staged in
// LDS, whole-line units transposed through the wave's tile).
// ---------------------------------------------------------------------------
template <int WAVES, typename OutT>
__global__ __launch_bounds__(64 * WAVES) void k_w4a8_dec2(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, const int32_t* __restrict__ wq,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero, int M, int N, int K,
    OutT* __restrict__ y) {
  constexpr bool kI32 = __is_same(OutT, int32_t);
  constexpr int kThreads = 64 * WAVES;
  extern __shared__ __attribute__((aligned(16))) u32 szl[];   // 32 x sz_pitch(G) words
  __shared__ __attribute__((aligned(16))) int8_t tiles[WAVES][kTileBytes];
  __shared__ v4f red[kI32 ? 1 : WAVES][2][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int n0 = blockIdx.x * 32;
  const int G = K >> 7, Kw = K >> 3, RB = Kw * 4;
  const int units = (RB + kUnitBytes - 1) / kUnitBytes;
  const int ub = (int)((int64_t)units * wave / WAVES), ue = (int)((int64_t)units * (wave + 1) / WAVES);
  rsrc_t wr[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int nb = n0 + 16 * b;
    const int rows = max(0, min(16, N - nb));
    wr[b] = make_rsrc_uniform(wq + (int64_t)min(nb, N) * Kw, (u32)(rows * RB));
  }
  const UnitLanes ul = unit_lanes(lane, RB);
  const rsrc_t xr = make_rsrc(xq, (u32)(M * K));
  const u32 xoff = (u32)(r * K + 32 * j);
  struct Batch { v4i w[2][2], xa[2][2]; };
  auto load = [&](Batch& bt, int q) {
#pragma unroll
    for (int b = 0; b < 2; ++b) unit_load(bt.w[b], wr[b], ul, q, q < ue, RB);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int g = 2 * q + s;
      const bool gin = q < ue && g < G;
#pragma unroll
      for (int h = 0; h < 2; ++h) bt.xa[s][h] = bld16(xr, gin ? xoff + 128 * g + 16 * h : kOOB);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  Batch b0, b1;
  ScaleZeroStage<kThreads, 4> sz;
  const int srows = max(0, min(32, N - n0));
  const rsrc_t sr = make_rsrc_uniform(wscale + (int64_t)min(n0, N) * G, (u32)(srows * G * 2));
  const rsrc_t zr = make_rsrc_uniform(wzero + (int64_t)min(n0, N) * G, (u32)(srows * G * 2));
  sz.load(sr, zr, 32 * G, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(b0, ub);
  sz.finish(sr, zr, szl, G, 32 * G);
  lds_barrier();

  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  int8_t* tile = tiles[wave];
  v4f yacc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
  auto mma = [&](const Batch& bt, int q) {
    v4i f[2][2];
    unit_transpose(tile, bt.w[0], ul, f[0]);
    unit_transpose(tile, bt.w[1], ul, f[1]);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int g = 2 * q + s;
      const bool gin = q < ue && g < G;
      const v4i a0 = shuffle_act16(bt.xa[s][0]), a1 = shuffle_act16(bt.xa[s][1]);
      v4i rs = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, ones, v4i{0, 0, 0, 0}, 0, 0, 0);
      rs = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, ones, rs, 0, 0, 0);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const u32 szw = gin ? szl[(16 * b + r) * sz_pitch(G) + g] : 0u;
        const int z = (int)f16_bits_to_f32((uint16_t)(szw >> 16));
        v4i acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __mul24(-z, rs[i]);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, unpack_u4_pair((u32)f[b][s][0], (u32)f[b][s][1]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, unpack_u4_pair((u32)f[b][s][2], (u32)f[b][s][3]), acc, 0, 0, 0);
        if constexpr (kI32) {
          const int n = n0 + 16 * b + r;
          if (gin && n < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = 4 * j + i;
              if (m < M) y[((int64_t)m * G + g) * N + n] = acc[i];
            }
          }
        } else {
          const float sc = f16_bits_to_f32((uint16_t)(szw & 0xFFFFu));
#pragma unroll
          for (int i = 0; i < 4; ++i) yacc[b][i] = __builtin_fmaf(sc, (float)acc[i], yacc[b][i]);
        }
      }
    }
  };
  for (int q = ub; q < ue; q += 2) {
    load(b1, q + 1);
    mma(b0, q);
    load(b0, q + 2);
    mma(b1, q + 1);
  }
  if constexpr (!kI32) {
    red[wave][0][lane] = yacc[0];
    red[wave][1][lane] = yacc[1];
    __syncthreads();
    if (wave < 2) {
      const int b = wave;
      v4f sum = red[0][b][lane];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][b][lane];
      const int n = n0 + 16 * b + r;
      if (n < N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * j + i;
          if (m < M) store_out<OutT>(y, (int64_t)m * N + n, sum[i] * xs[m]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wide kernel (up to 64 token rows on layers of at least 384 weight blocks): as
// k_w8a8_wide / k_w4a16_wide, a workgroup owns NB 16-row weight blocks and
// moves through K in phases of PU units (2 PU groups).  Each block has KS
// waves that split a phase's units between them, so a SIMD holds more than
// one wave to hide the per-group LDS and MFMA latencies; their partial sums
// meet in LDS at the end.  A phase's token rows (16 MT rows x 256 PU bytes)
// are staged once in LDS for all waves, each 16-byte chunk already permuted
// to the unpack order, and the per-(group, row) token sums that carry the
// zero point are formed while staging (byte sums reduced over the 8 lanes
// that hold a group's chunks); two-deep LDS ring, one barrier per phase.  The
// weight stream runs WR phases ahead and the token rows XR phases ahead, in
// register rings.  Each unpacked weight fragment feeds the MFMAs of all MT
// m-tiles.
// ---------------------------------------------------------------------------
// Static LDS of k_w4a8_wide (token ring, token sums, weight tiles, partial
// sums), checked against the kernel's arrays.
template <int MT, int NB, int KS, int MS, int PU, bool I32>
__host__ __device__ constexpr size_t w4a8_wide_static_lds() {
  return (size_t)2 * 16 * MT * (2 * kUnitBytes * PU + 16) + (size_t)2 * 2 * PU * 16 * MT * 4 +
         (size_t)NB * KS * MS * kTileBytes + (size_t)((I32 || KS == 1) ? 1 : NB * MS * (KS - 1)) * (MT / MS) * 64 * 16;
}

template <int MT, int NB, int KS, int MS, int PU, int WR, int XR, typename OutT>
__global__ __launch_bounds__(64 * NB * KS * MS) void k_w4a8_wide(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, const int32_t* __restrict__ wq,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero, int M, int N, int K,
    OutT* __restrict__ y) {
  static_assert(PU % KS == 0, "every wave of a block takes the same number of units");
  static_assert(MT % MS == 0, "every wave of a block takes the same number of m-tiles");
  constexpr int L = WR % XR == 0 ? WR : WR * XR;   // ring turn: every slot index static
  constexpr bool kI32 = __is_same(OutT, int32_t);
  constexpr int UPW = PU / KS;                     // units per wave and phase
  constexpr int MTW = MT / MS;                     // m-tiles per wave
  constexpr int MR = 16 * MT, PB = 2 * kUnitBytes * PU, kThreads = 64 * NB * KS * MS;   // PB: token bytes per row
  constexpr int kPitch = PB + 16;                                                   // odd number of 16-byte chunks
  constexpr int kRowChunks = PB / 16, kChunks = MR * kRowChunks;
  constexpr int CPT = (kChunks + kThreads - 1) / kThreads;
  constexpr int GP = 2 * PU;                                                        // groups per phase
  extern __shared__ __attribute__((aligned(16))) u32 szl[];   // 16 NB x sz_pitch(G) words
  __shared__ __attribute__((aligned(16))) int8_t xbuf[2][MR * kPitch];
  __shared__ __attribute__((aligned(16))) int tsum[2][GP][MR];
  __shared__ __attribute__((aligned(16))) int8_t tiles[NB * KS * MS][kTileBytes];
  __shared__ v4f red[(kI32 || KS == 1) ? 1 : NB * MS * (KS - 1)][MTW][64];
  static_assert(sizeof(xbuf) + sizeof(tsum) + sizeof(tiles) + sizeof(red) ==
                w4a8_wide_static_lds<MT, NB, KS, MS, PU, kI32>(), "static LDS bookkeeping");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blk = wave % NB, ks = (wave / NB) % KS, ms = wave / (NB * KS);
  const int r = lane & 15, j = lane >> 4;
  const int G = K >> 7, Kw = K >> 3, RB = Kw * 4;
  const int wg_row0 = blockIdx.x * NB * 16, n_base = wg_row0 + blk * 16;
  const int units = (RB + kUnitBytes - 1) / kUnitBytes;
  const int phases = (units + PU - 1) / PU;

  const int rows_n = max(0, min(16, N - n_base));
  const rsrc_t wr = make_rsrc_uniform(wq + (int64_t)min(n_base, N - 1) * Kw, (u32)(rows_n * RB));
  const rsrc_t xr = make_rsrc(xq, (u32)(M * K));
  const UnitLanes ul = unit_lanes(lane, RB);

  using WSlot = v4i[UPW][2];
  struct XBatch {
    v4i x[CPT];
  };
  auto load_w = [&](WSlot& d, int p) {
#pragma unroll
    for (int v = 0; v < UPW; ++v) unit_load(d[v], wr, ul, p * PU + ks * UPW + v, p < phases, RB);
  };
  auto load_x = [&](XBatch& bt, int p) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + c * kThreads;
      const int row = chunk / kRowChunks, kb = p * PB + (chunk % kRowChunks) * 16;
      // rows past M and bytes past K read zeros (past the resource)
      bt.x[c] = bld16(xr, chunk < kChunks && kb < K ? (u32)(row * K + kb) : kOOB);
    }
  };

  // scales and zero points of the workgroup's 16 NB rows, with the first
  // weight phases and token batches issued behind their loads
  const int wg_rows = max(0, min(16 * NB, N - wg_row0));
  const rsrc_t sr = make_rsrc_uniform(wscale + (int64_t)min(wg_row0, N - 1) * G, (u32)(wg_rows * G * 2));
  const rsrc_t zr = make_rsrc_uniform(wzero + (int64_t)min(wg_row0, N - 1) * G, (u32)(wg_rows * G * 2));
  ScaleZeroStage<kThreads, 4> sz;
  sz.load(sr, zr, 16 * NB * G, 0);
  __builtin_amdgcn_sched_barrier(0);
  WSlot wring[WR];
  XBatch xring[XR];
#pragma unroll
  for (int q = 0; q < (WR > XR ? WR : XR) - 1; ++q) {
    if (q < WR - 1) load_w(wring[q], q);
    if (q < XR - 1) load_x(xring[q], q);
  }
  __builtin_amdgcn_sched_barrier(0);
  sz.finish(sr, zr, szl, G, 16 * NB * G);

  const u32* szrow = szl + (blk * 16 + r) * sz_pitch(G);
  int8_t* tile = tiles[wave];
  v4f yacc[MTW];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt) yacc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  const int n = n_base + r;
  auto process = [&](const XBatch& bt, const WSlot& w, int p) {
    int8_t* buf = xbuf[p & 1];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + c * kThreads;   // chunk % 8 == tid % 8 (kThreads % 8 == 0)
      const bool in = chunk < kChunks;
      // the 8 chunks of a group are held by 8 consecutive lanes
      int t = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) t = __builtin_amdgcn_sdot4(bt.x[c][e], 0x01010101, t, false);
      t = sum_lanes8(t);
      if (in) {
        const int row = chunk / kRowChunks, col = chunk % kRowChunks;
        st16(buf + row * kPitch + col * 16, shuffle_act16(bt.x[c]));
        if ((col & 7) == 0) tsum[p & 1][col >> 3][row] = t;
      }
    }
    // Panel p (and, at p = 0, the scales) complete once every wave is here;
    // the buffers phase p + 1 overwrites were last read at phase p - 1.
    lds_barrier();
#pragma unroll
    for (int v = 0; v < UPW; ++v) {
      v4i f[2];
      unit_transpose(tile, w[v], ul, f);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int gl = 2 * (ks * UPW + v) + s2, g = p * GP + gl;
        const bool gin = g < G;
        const u32 szw = gin ? szrow[g] : 0u;       // past G: zero codes, tokens and scale
        const int z = (int)f16_bits_to_f32((uint16_t)(szw >> 16));
        const v4i bw0 = unpack_u4_pair((u32)f[s2][0], (u32)f[s2][1]);
        const v4i bw1 = unpack_u4_pair((u32)f[s2][2], (u32)f[s2][3]);
        const float sc = f16_bits_to_f32((uint16_t)(szw & 0xFFFFu));
#pragma unroll
        for (int mw = 0; mw < MTW; ++mw) {
          const int mt = ms * MTW + mw;
          const int8_t* xf = buf + (16 * mt + r) * kPitch + 128 * gl + 32 * j;
          const v4i ts = *reinterpret_cast<const v4i*>(&tsum[p & 1][gl][16 * mt + 4 * j]);
          v4i acc;   // |z| <= 15, |token sum| <= 128 * 127: exact 24-bit products
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = __mul24(-z, ts[e]);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ld16(xf), bw0, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ld16(xf + 16), bw1, acc, 0, 0, 0);
          if constexpr (kI32) {
            if (gin && n < N) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int m = 16 * mt + 4 * j + e;
                if (m < M) y[((int64_t)m * G + g) * N + n] = acc[e];
              }
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) yacc[mw][e] = __builtin_fmaf(sc, (float)acc[e], yacc[mw][e]);
          }
        }
      }
    }
  };
  // every wave runs the same number of phases, so all reach every barrier;
  // loads for phases past the end read zeros without touching memory
  for (int p0 = 0; p0 < phases; p0 += L) {
#pragma unroll
    for (int s = 0; s < L; ++s) {
      const int p = p0 + s;
      if (p >= phases) break;
      load_w(wring[(s + WR - 1) % WR], p + WR - 1);
      load_x(xring[(s + XR - 1) % XR], p + XR - 1);
      __builtin_amdgcn_sched_barrier(0);
      process(xring[s % XR], wring[s % WR], p);
    }
  }

  if constexpr (!kI32) {
    if constexpr (KS > 1) {
      // the block's other waves hand their partial sums to wave ks = 0
      if (ks > 0) {
#pragma unroll
        for (int mw = 0; mw < MTW; ++mw) red[((ks - 1) * MS + ms) * NB + blk][mw][lane] = yacc[mw];
      }
      lds_barrier();
      if (ks > 0) return;
#pragma unroll
      for (int o = 0; o < KS - 1; ++o)
#pragma unroll
        for (int mw = 0; mw < MTW; ++mw) {
          const v4f t = red[(o * MS + ms) * NB + blk][mw][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) yacc[mw][e] += t[e];
        }
    }
    if (n < N) {
#pragma unroll
      for (int mw = 0; mw < MTW; ++mw)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * (ms * MTW + mw) + 4 * j + e;
          if (m < M) store_out<OutT>(y, (int64_t)m * N + n, yacc[mw][e] * xs[m]);
        }
    }
  }
}

template <int MT, int NB, int KS, int MS, typename OutT>
static bool launch_w4a8_wide_nb(const int8_t* xq, const float* xs, const int32_t* wq,
                                const uint16_t* ws, const uint16_t* wz, int M, int N, int K, OutT* y,
                                size_t lds, hipStream_t st) {
  constexpr int PU = KS, WR = 2, XR = 2;   // measured on MI355X (K = 4096, N = 11008 / 14336)
  if (w4a8_wide_static_lds<MT, NB, KS, MS, PU, __is_same(OutT, int32_t)>() + lds > kLdsBytesPerCU) return false;
  const int nblocks = (N + 15) / 16;
  const dim3 grid((unsigned)((nblocks + NB - 1) / NB)), block(64 * NB * KS * MS);
  k_w4a8_wide<MT, NB, KS, MS, PU, WR, XR, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, wz, M, N, K, y);
  return true;
}

// 2-4 weight blocks per workgroup (wide_waves); per block 4 waves (K split in
// 4, or in 2 with the m-tiles split in 2) where the workgroup stays at 12
// waves or fewer, else 2 (measured on MI355X: 16-wave workgroups were slower)
template <int MT, typename OutT>
static bool launch_w4a8_wide(const int8_t* xq, const float* xs, const int32_t* wq,
                             const uint16_t* ws, const uint16_t* wz, int M, int N, int K, OutT* y,
                             size_t lds, hipStream_t st) {
  constexpr int KS = MT <= 2 ? 4 : 2, MS = MT <= 2 ? 1 : 2;
  switch (wide_waves(N)) {
    case 2: return launch_w4a8_wide_nb<MT, 2, KS, MS, OutT>(xq, xs, wq, ws, wz, M, N, K, y, lds, st);
    case 3: return launch_w4a8_wide_nb<MT, 3, KS, MS, OutT>(xq, xs, wq, ws, wz, M, N, K, y, lds, st);
    default: return launch_w4a8_wide_nb<MT, 4, 2, 1, OutT>(xq, xs, wq, ws, wz, M, N, K, y, lds, st);
  }
}

// ---------------------------------------------------------------------------
// One or two token rows (MR): a matrix-vector product on the vector ALU's
// int8 dot products, where a 16x16 MFMA would spend 15 of its 16 rows on
// padding.
// Lane l of a wave covers bytes 16 l .. 16 l + 15 of every kilobyte c of a
// weight row: codes k = 2048 c + 32 l + [0, 32), a quarter of group
// g = 16 c + l / 4.  It keeps the matching 32 activation bytes of every c in
// registers, split once into the even- and odd-code bytes of each word (the
// order w & 0x0F0F0F0F and (w >> 4) & 0x0F0F0F0F unpack to), and the
// group's token sum (byte sums reduced over the group's four lanes).  A wave
// owns R consecutive weight rows and issues all their loads up front.  Per
// word of 8 codes: two masks, a shift and two v_dot4_i32_i8 -- exact int32.
// The group's four lanes add their sums (DPP), the zero point enters as
// -z * (token sum), and the group sum is scaled by s in binary32 as in the
// matrix-core kernels; the wave sums its lanes at the end.
// ---------------------------------------------------------------------------
constexpr int kGemvWaves = 4;

__device__ __forceinline__ int quad_sum_i(int t) {
  t += __builtin_amdgcn_mov_dpp(t, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  t += __builtin_amdgcn_mov_dpp(t, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  return t;
}

template <int MR, int R, int C, typename OutT>
__global__ __launch_bounds__(64 * kGemvWaves) void k_w4a8_gemv(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, const int32_t* __restrict__ wq,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero, int M, int N, int K,
    OutT* __restrict__ y) {
  constexpr bool kI32 = __is_same(OutT, int32_t);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x * kGemvWaves + wave) * R;
  if (n0 >= N) return;   // wave-uniform
  const int G = K >> 7, RB = K >> 1;   // groups and packed bytes per weight row
  const int rows = min(R, N - n0);
  const rsrc_t wr = make_rsrc_uniform(wq + (int64_t)n0 * (K >> 3), (u32)(rows * RB));
  const rsrc_t sr = make_rsrc_uniform(wscale + (int64_t)n0 * G, (u32)(rows * G * 2));
  const rsrc_t zr = make_rsrc_uniform(wzero + (int64_t)n0 * G, (u32)(rows * G * 2));
  const rsrc_t xr = make_rsrc_uniform(xq, (u32)(M * K));   // token rows past M read zeros

  // activations first, then scales and zero points, then the weight stream;
  // pieces past the row end read zeros (x through its resource's range, the
  // rest through kOOB: their resources span the wave's rows)
  v4i xv[MR][C][2];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 2048 * c + 32 * lane + 16 * h;
        xv[m][c][h] = bld16(xr, k < K ? (u32)(m * K + k) : kOOB);
      }
  uint16_t sb[R][C], zb[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int g = 16 * c + (lane >> 2);
      const u32 o = g < G ? (u32)(2 * (r * G + g)) : kOOB;
      sb[r][c] = bld2(sr, o);
      zb[r][c] = bld2(zr, o);
    }
  v4i wv[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int b = 1024 * c + 16 * lane;
      wv[r][c] = bld16_nt(wr, b < RB ? (u32)(r * RB + b) : kOOB);
    }
  __builtin_amdgcn_sched_barrier(0);

  // word i of the lane's piece holds codes 8i..8i+7: its activation bytes are
  // dwords 2i, 2i+1 of the 32 loaded bytes
  u32 xe[MR][C][4], xo[MR][C][4];
  int tsum[MR][C];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      int t = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32 d0 = (u32)xv[m][c][i >> 1][2 * (i & 1)], d1 = (u32)xv[m][c][i >> 1][2 * (i & 1) + 1];
        even_odd_bytes(d0, d1, xe[m][c][i], xo[m][c][i]);
        t = __builtin_amdgcn_sdot4((int)d0, 0x01010101, t, false);
        t = __builtin_amdgcn_sdot4((int)d1, 0x01010101, t, false);
      }
      tsum[m][c] = quad_sum_i(t);   // the group's token sum, in all four lanes
    }

  float yacc[MR][R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int m = 0; m < MR; ++m) yacc[m][r] = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      u32 lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32 w = (u32)wv[r][c][i];
        lo[i] = w & 0x0F0F0F0Fu;
        hi[i] = (w >> 4) & 0x0F0F0F0Fu;
      }
      // |z| <= 15 and |token sum| <= 128 * 127: the 24-bit multiply is exact
      const int z = (int)f16_bits_to_f32(zb[r][c]);
      const float s = f16_bits_to_f32(sb[r][c]);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        int a = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a = __builtin_amdgcn_sdot4((int)xe[m][c][i], (int)lo[i], a, false);
          a = __builtin_amdgcn_sdot4((int)xo[m][c][i], (int)hi[i], a, false);
        }
        const int acc = quad_sum_i(a) - __mul24(z, tsum[m][c]);
        if constexpr (kI32) {
          const int g = 16 * c + (lane >> 2);
          if ((lane & 3) == 0 && g < G && r < rows && m < M) y[((int64_t)m * G + g) * N + n0 + r] = acc;
        } else {
          yacc[m][r] = __builtin_fmaf(s, (float)acc, yacc[m][r]);
        }
      }
    }
  }

  if constexpr (!kI32) {
    // sum over the 16 quads: rotations by 4 and 8 within each row of 16
    // lanes, then the four rows; lane m R + r stores token row m, weight row r
    float mine = 0.f;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        int v = __float_as_int(yacc[m][r]);
        v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, false)));
        v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false)));
        const float t = (__int_as_float(__builtin_amdgcn_readlane(v, 0)) + __int_as_float(__builtin_amdgcn_readlane(v, 16))) +
                        (__int_as_float(__builtin_amdgcn_readlane(v, 32)) + __int_as_float(__builtin_amdgcn_readlane(v, 48)));
        mine = lane == m * R + r ? t : mine;
      }
    const int m = lane / R, r = lane - m * R;
    if (m < MR && m < M && r < rows) store_out<OutT>(y, (int64_t)m * N + n0 + r, mine * xs[m]);
  }
}

template <int MR, int R, int C, typename OutT>
static void launch_w4a8_gemv_rc(const int8_t* xq, const float* xs, const int32_t* wq, const uint16_t* ws,
                                const uint16_t* wz, int M, int N, int K, OutT* y, hipStream_t st) {
  const int waves = (N + R - 1) / R;
  const dim3 grid((unsigned)((waves + kGemvWaves - 1) / kGemvWaves)), block(64 * kGemvWaves);
  k_w4a8_gemv<MR, R, C, OutT><<<grid, block, 0, st>>>(xq, xs, wq, ws, wz, M, N, K, y);
}

// K up to 16384 (8 KB per weight row); rows per wave for about 8 kilobyte
// weight loads in flight per wave (4 and 16 measured alike or slower).
// Measured on MI355X against the matrix-core kernels it replaces at one row
// (A/B, graphs of 200 calls, weights rotated through 600 MB; us, K x N):
// 11008 x 4096 6.79-6.82 / 7.89-7.91, 4096 x 11008 5.90-5.91 / 6.96-7.04,
// 4096 x 12288 6.18-6.27 / 7.16, 4096 x 4096 3.73-3.75 / 4.90,
// 14336 x 4096 7.85 / 8.87-8.92, 8192 x 28672 20.53-20.54 / 26.24-26.31;
// the int32 group sums are the same bit for bit.
template <int MR, typename OutT>
static bool launch_w4a8_gemv_mr(const int8_t* xq, const float* xs, const int32_t* wq, const uint16_t* ws,
                                const uint16_t* wz, int M, int N, int K, OutT* y, hipStream_t st) {
  constexpr int L = 8;
  constexpr auto rows = [](int c) { return L / c < 1 ? 1 : L / c; };
  switch ((K / 2 + 1023) / 1024) {
    case 1: launch_w4a8_gemv_rc<MR, rows(1), 1, OutT>(xq, xs, wq, ws, wz, M, N, K, y, st); return true;
    case 2: launch_w4a8_gemv_rc<MR, rows(2), 2, OutT>(xq, xs, wq, ws, wz, M, N, K, y, st); return true;
    case 3: launch_w4a8_gemv_rc<MR, rows(3), 3, OutT>(xq, xs, wq, ws, wz, M, N, K, y, st); return true;
    case 4: launch_w4a8_gemv_rc<MR, rows(4), 4, OutT>(xq, xs, wq, ws, wz, M, N, K, y, st); return true;
    case 5: launch_w4a8_gemv_rc<MR, rows(5), 5, OutT>(xq, xs, wq, ws, wz, M, N, K, y, st); return true;
    case 6: launch_w4a8_gemv_rc<MR, rows(6), 6, OutT>(xq, xs, wq, ws, wz, M, N, K, y, st); return true;
    case 7: launch_w4a8_gemv_rc<MR, rows(7), 7, OutT>(xq, xs, wq, ws, wz, M, N, K, y, st); return true;
    case 8: launch_w4a8_gemv_rc<MR, rows(8), 8, OutT>(xq, xs, wq, ws, wz, M, N, K, y, st); return true;
    default: return false;
  }
}

// Two token rows: the unpack is shared, the dot products double.  Measured
// against the matrix-core kernels (us): K = 4096 with N = 4096 4.24-4.26 /
// 5.01, N = 11008 6.76-6.77 / 7.25-7.41, N = 12288 7.28-7.68 / 7.52-7.84;
// longer rows lose (K = 11008, N = 4096: 8.52-8.56 / 8.00-8.01), and so do
// four rows everywhere (K = 4096, N = 11008: 9.6 / 7.5-7.8).
template <typename OutT>
static bool launch_w4a8_gemv(const int8_t* xq, const float* xs, const int32_t* wq, const uint16_t* ws,
                             const uint16_t* wz, int M, int N, int K, OutT* y, hipStream_t st) {
  if (M == 1) return launch_w4a8_gemv_mr<1, OutT>(xq, xs, wq, ws, wz, M, N, K, y, st);
  if (M == 2 && K <= 4096) return launch_w4a8_gemv_mr<2, OutT>(xq, xs, wq, ws, wz, M, N, K, y, st);
  return false;
}

template <typename OutT>
static hipError_t gemm_w4a8_t(const int8_t* xq, const float* xs, const int32_t* wq,
                              const uint16_t* ws, const uint16_t* wz, int M, int N, int K, OutT* y,
                              hipStream_t st) {
  const size_t lds = (size_t)16 * sz_pitch(K / 128) * 4;
  if (M <= 2 && launch_w4a8_gemv<OutT>(xq, xs, wq, ws, wz, M, N, K, y, st)) return hipGetLastError();
  if (M <= 64 && wide_waves(N) >= 2) {
    // layers of more than 384 blocks: the token rows staged once per
    // workgroup of 2-4 weight blocks (unless K is too long for LDS).
    // Measured on MI355X against the decode kernels below (K = 4096, N =
    // 11008): 1 row 8.8 -> 7.1 us, 8 rows 9.4 -> 7.9, 16 rows 10.3 -> 7.7;
    // 17-64 rows against the multi-tile kernel: 32 rows 21.0 -> 10.6.  With
    // one block per workgroup (N < 6144) the kernels below were faster
    // (K = 11008, N = 4096, 17 rows: 13.0 against 18.0 us).
    const size_t lds_wide = (size_t)16 * wide_waves(N) * sz_pitch(K / 128) * 4;
    const bool done = M <= 16   ? launch_w4a8_wide<1, OutT>(xq, xs, wq, ws, wz, M, N, K, y, lds_wide, st)
                      : M <= 32 ? launch_w4a8_wide<2, OutT>(xq, xs, wq, ws, wz, M, N, K, y, lds_wide, st)
                                : launch_w4a8_wide<4, OutT>(xq, xs, wq, ws, wz, M, N, K, y, lds_wide, st);
    if (done) return hipGetLastError();
  }
  if (M <= 16 && 2 * lds <= kDecLdsMaxBytes && (N + 31) / 32 >= 256) {
    // wide layers (measured on MI355X, K = 4096: N = 11008 M = 16 14.4 ->
    // 11.0 us, M = 1 at N = 12288 10.1 -> 9.3 us); at N = 4096 its 128
    // workgroups leave half the CUs idle (11.0 -> 13.6 us), so not there
    constexpr int WAVES = 8;
    const dim3 grid((unsigned)((N + 31) / 32)), block(64 * WAVES);
    k_w4a8_dec2<WAVES, OutT><<<grid, block, 2 * lds, st>>>(xq, xs, wq, ws, wz, M, N, K, y);
    return hipGetLastError();
  }
  if (M <= 16 && lds <= kDecLdsMaxBytes) {
    constexpr int WAVES = 8, UB = 1;  // measured on MI355X
    const dim3 grid((unsigned)((N + 15) / 16)), block(64 * WAVES);
    const int mr = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    switch (mr) {
      case 1: k_w4a8_dec<1, WAVES, UB, false, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, wz, nullptr, nullptr, M, N, K, y); break;
      case 2: k_w4a8_dec<2, WAVES, UB, false, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, wz, nullptr, nullptr, M, N, K, y); break;
      case 4: k_w4a8_dec<4, WAVES, UB, false, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, wz, nullptr, nullptr, M, N, K, y); break;
      case 8: k_w4a8_dec<8, WAVES, UB, false, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, wz, nullptr, nullptr, M, N, K, y); break;
      default: k_w4a8_dec<16, WAVES, UB, false, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, wz, nullptr, nullptr, M, N, K, y); break;
    }
    return hipGetLastError();
  }
  if (M <= 64 && lds <= kDecLdsMaxBytes) {
    // 17..64 token rows: one weight stream for 2 or 4 tiles of 16 rows
    constexpr int WAVES = 8, UB = 1;
    const dim3 grid((unsigned)((N + 15) / 16)), block(64 * WAVES);
    if (M <= 32)
      k_w4a8_dec_mt<2, WAVES, UB, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, wz, M, N, K, y);
    else
      k_w4a8_dec_mt<4, WAVES, UB, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, wz, M, N, K, y);
    return hipGetLastError();
  }
  constexpr int MT = 1, NT = 1, WAVES = 8, U = 2;  // measured on MI355X
  dim3 grid((unsigned)((N + 16 * NT - 1) / (16 * NT)), (unsigned)((M + 16 * MT - 1) / (16 * MT)));
  k_w4a8<MT, NT, WAVES, U, OutT><<<grid, dim3(64 * WAVES), 0, st>>>(xq, xs, wq, ws, wz, M, N, K, y);
  return hipGetLastError();
}

// W4A8 with the INT8 outlier side path: the decode kernel over chunks of up
// to 16 token rows (the weight stream is re-read per chunk).
template <typename OutT>
static hipError_t gemm_w4a8_outl_t(const int8_t* xq, const float* xs, const int32_t* wq,
                                   const uint16_t* ws, const uint16_t* wz, const uint64_t* orec,
                                   const float* os8, int M, int N, int K, OutT* y,
                                   hipStream_t st) {
  constexpr int WAVES = 8, UB = 1;
  const int G = K / 128;
  const size_t lds = (size_t)16 * sz_pitch(G) * 4;
  if (lds > kDecLdsMaxBytes) return hipErrorInvalidValue;   // excluded by the API checks
  const dim3 grid((unsigned)((N + 15) / 16)), block(64 * WAVES);
  const int64_t ystride = __is_same(OutT, int32_t) ? (int64_t)(G + 1) * N : N;
  for (int m0 = 0; m0 < M; m0 += 16) {
    const int mc = std::min(16, M - m0);
    const int mr = mc <= 1 ? 1 : mc <= 2 ? 2 : mc <= 4 ? 4 : mc <= 8 ? 8 : 16;
    const int8_t* x = xq + (int64_t)m0 * K;
    const float* s = xs ? xs + m0 : nullptr;
    OutT* yy = y + m0 * ystride;
    switch (mr) {
      case 1: k_w4a8_dec<1, WAVES, UB, true, OutT><<<grid, block, lds, st>>>(x, s, wq, ws, wz, orec, os8, mc, N, K, yy); break;
      case 2: k_w4a8_dec<2, WAVES, UB, true, OutT><<<grid, block, lds, st>>>(x, s, wq, ws, wz, orec, os8, mc, N, K, yy); break;
      case 4: k_w4a8_dec<4, WAVES, UB, true, OutT><<<grid, block, lds, st>>>(x, s, wq, ws, wz, orec, os8, mc, N, K, yy); break;
      case 8: k_w4a8_dec<8, WAVES, UB, true, OutT><<<grid, block, lds, st>>>(x, s, wq, ws, wz, orec, os8, mc, N, K, yy); break;
      default: k_w4a8_dec<16, WAVES, UB, true, OutT><<<grid, block, lds, st>>>(x, s, wq, ws, wz, orec, os8, mc, N, K, yy); break;
    }
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_w4a8_outl(const int8_t* xq, const float* xs, const int32_t* wq,
                                 const uint16_t* ws, const uint16_t* wz, const uint64_t* orec,
                                 const float* os8, int64_t M, int64_t N, int64_t K, void* y,
                                 int y_dtype, hipStream_t st) {
  const int m = (int)M, n = (int)N, k = (int)K;
  switch (y_dtype) {
    case F32: return gemm_w4a8_outl_t<float>(xq, xs, wq, ws, wz, orec, os8, m, n, k, (float*)y, st);
    case F16: return gemm_w4a8_outl_t<_Float16>(xq, xs, wq, ws, wz, orec, os8, m, n, k, (_Float16*)y, st);
    case BF16: return gemm_w4a8_outl_t<uint16_t>(xq, xs, wq, ws, wz, orec, os8, m, n, k, (uint16_t*)y, st);
    default: return gemm_w4a8_outl_t<int32_t>(xq, xs, wq, ws, wz, orec, os8, m, n, k, (int32_t*)y, st);
  }
}

hipError_t launch_gemm_w4a8(const int8_t* xq, const float* xs, const int32_t* wq,
                            const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                            int64_t K, void* y, int y_dtype, hipStream_t st) {
  const int m = (int)M, n = (int)N, k = (int)K;
  switch (y_dtype) {
    case F32: return gemm_w4a8_t<float>(xq, xs, wq, ws, wz, m, n, k, (float*)y, st);
    case F16: return gemm_w4a8_t<_Float16>(xq, xs, wq, ws, wz, m, n, k, (_Float16*)y, st);
    case BF16: return gemm_w4a8_t<uint16_t>(xq, xs, wq, ws, wz, m, n, k, (uint16_t*)y, st);
    default: return gemm_w4a8_t<int32_t>(xq, xs, wq, ws, wz, m, n, k, (int32_t*)y, st);
  }
}

}  // namespace qg
