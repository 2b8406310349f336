// Per-token int8 quantization feeding the W4A8 GEMM through a token panel,
// for decode (M <= 16 token rows): the panel quantizer, the panel GEMM and
// the call that runs both.  「LLM推理降本五要素」 §2.2 (W4A8, group size 128,
// per-group scale and zero point); 「第4章：量化」 §1.1-1.3 (per-token
// symmetric codes, x_hat = (x_int - z) s) and §3.5 (dequantize inside the
// GEMM).
//
// The plain W4A8 kernel takes row-major codes, so each of its workgroups
// re-reads the token rows as half-used lines, permutes their bytes into the
// unpack order and forms the per-group token sums with extra matrix-core
// instructions -- all of it repeated by every workgroup of the layer.  Here
// the quantizer does that once: besides the codes and scales it writes
//   * a token panel: the codes of group g, half h (k = 128 g + 16 h ...) in
//     MFMA operand order, panel[g][h][r][j] = the 16 codes of row r at
//     k = 128 g + 32 j + 16 h + [0, 16), bytes permuted to the order in which
//     the packed weights unpack (even k of each 8 first, then odd k), so a
//     wave reads one operand as one contiguous kilobyte (whole lines) and a
//     row's codes of one (g, h) are 64 contiguous bytes;
//   * the token sums sums[g][r] = sum_{k in g} xq[r, k] (exact int32), which
//     carry the zero point: acc = sum xq q - z sum xq.
// Both live in device memory the caller provides; one panel can feed several
// GEMMs of the same input (the projections that share a layer's input).
//
// The GEMM streams each 16-row weight block with buffer-to-LDS DMA: every
// unit (16 rows x 128 bytes = two groups) of a wave's run is requested at
// once, each unit as two whole-line loads (8 rows x 128 B) landing in an
// XOR-swizzled 2 KB slot, from which the MFMA fragments are read without bank
// conflicts.  The block's scales and zero points and the token sums reach LDS
// the same way, requested ahead of the weights and waited for after them.
// Staged through registers instead, their loads must complete before the
// LDS stores: written after the weight requests, the compiler sank the loads
// behind them and waited for the whole stream; written before, every wave
// paid the loads' latency before its first weight request.  A wave whose run
// is one unit shorter than its ring repeats its last unit's loads (cache
// hits) with a zero scale instead of issuing out-of-range loads, which
// measured slow.
//
// At 16 token rows the panel a workgroup reads (16 K bytes) is twice its
// weight block (16 x K/2 bytes); that token traffic through each CU's
// vector-memory path, not HBM, bounds the kernel there (MI355X, 16 x 11008 x
// 4096: 9.4 us, 6.6 us with the token loads left out).

#include "qg_decode.hpp"
#include "qg_device.hpp"
#include "qg_launch.hpp"
#include "qg_quant.hpp"

#include <mutex>

namespace qg {

namespace {

// bytes [b0..b7] of (lo, hi) -> [b0 b2 b4 b6 | b1 b3 b5 b7]: the order in
// which w & 0x0F0F0F0F, (w >> 4) & 0x0F0F0F0F unpack 8 codes of a word
__device__ __forceinline__ v4i panel_order16(v4i x) {
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm((u32)x[1], (u32)x[0], 0x06040200u);
  r[1] = (int)__builtin_amdgcn_perm((u32)x[1], (u32)x[0], 0x07050301u);
  r[2] = (int)__builtin_amdgcn_perm((u32)x[3], (u32)x[2], 0x06040200u);
  r[3] = (int)__builtin_amdgcn_perm((u32)x[3], (u32)x[2], 0x07050301u);
  return r;
}

__device__ __forceinline__ v4i unpack_pair(u32 w0, u32 w1) {
  return v4i{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu), (int)(w1 & 0x0F0F0F0Fu),
             (int)((w1 >> 4) & 0x0F0F0F0Fu)};
}

// Outlier-retention side path (「LLM推理降本五要素」 §2.2) on the panel: a
// group's record holds three (index << 8 | code byte) slots; lane (row r,
// k-block j) of an MFMA covers the inputs k = 32 j + 16 h + [0, 16) of the
// group, held in the panel's byte order (within each 8: even k, then odd).
// The slots falling there are placed at the byte their k takes in that
// order, giving a sparse int8 operand whose product with the panel fragment
// accumulates sum_k x_q[m, k] * code exactly in int32.
__device__ __forceinline__ v4i outlier_operand_panel(u32 lo, u32 hi, int kb) {
  uint64_t b0 = 0, b1 = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const u32 slot = (i == 0 ? lo : i == 1 ? lo >> 16 : hi) & 0xFFFFu;
    const int pos = (int)(slot >> 8) - kb;   // k offset in the lane's 16, if in range
    const int at = (pos & 8) | ((pos & 1) << 2) | ((pos >> 1) & 3);   // its byte in the panel order
    const uint64_t v = (uint64_t)(slot & 0xFFu) << (8 * (at & 7));
    b0 |= (u32)pos < 8u ? v : 0;
    b1 |= (u32)(pos - 8) < 8u ? v : 0;
  }
  return v4i{(int)(u32)b0, (int)(u32)(b0 >> 32), (int)(u32)b1, (int)(u32)(b1 >> 32)};
}

// sum of the 16 signed bytes of v (exact)
__device__ __forceinline__ int byte_sum16(v4i v) {
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) s = __builtin_amdgcn_sdot4(v[i], 0x01010101, s, false);
  return s;
}

}  // namespace

// Panel layout (both kernels): panel[g][h][r][j], 16 bytes each, r < MR
// (MR = M rounded up to 1, 2, 4, 8 or 16), then the token sums sums[g][16]
// int32 at byte offset 2048 G: G (2048 + 64) bytes whatever M.
constexpr int kPanelRows = 16;

// ---------------------------------------------------------------------------
// Quantizer: one workgroup of NT threads per panel row, the row in
// registers.  Rows < M get the codes and scales of k_quant_per_token (same
// loads, scale, reciprocal and sym_code_t) and are written to xq (unless it
// is NULL), x_scale, the panel and the sums; rows M..MR-1 write zero codes
// and sums to the panel only (row 0 also zeroes sum rows MR..15), so that
// every byte of the panel is defined.  The grid is 16 workgroups whatever
// MR, workgroup b taking row 2 (b mod 8) + b / 8 (those past MR exit): the
// two rows that share each 128-byte panel line then run on one XCD
// (workgroups are dealt to the 8 XCDs in turn) and the line is completed in
// that XCD's L2 instead of being written in pieces from two.  Measured on
// MI355X (16 rows of K = 11008), 16-byte stores from rows spread over all
// XCDs made this kernel 0.6 us slower than the plain quantizer.
// ---------------------------------------------------------------------------
template <int DT, int CH, int NT>
__global__ __launch_bounds__(NT) void k_quant_panel(const void* __restrict__ x, int M, int64_t K,
                                                    int MR, int8_t* __restrict__ xq,
                                                    float* __restrict__ xs,
                                                    int8_t* __restrict__ panel, int* __restrict__ sums) {
  __shared__ float red[NT / kWave];
  const int row = 2 * (int)(blockIdx.x & 7) + (int)(blockIdx.x >> 3);
  if (row >= MR) return;   // the whole workgroup: before any barrier
  const bool real = row < M;
  const char* xr = reinterpret_cast<const char*>(x) + (real ? (int64_t)row * K * esize<DT>() : 0);
  const int nch = (int)(K >> 4);
  const rsrc_t rr = make_rsrc(xr, (uint32_t)(K * esize<DT>()));
  v4i raw[CH][4];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = threadIdx.x + c * NT;
    load_chunk16_rs<DT>(rr, real && idx < nch, idx, raw[c]);
  }
  float v[CH][16];
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    widen16<DT>(raw[c], v[c]);
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[c][e]));   // zeros past the end
  }
  amax = block_max_nonneg_once<NT>(amax, red);
  const float s = amax / 127.f, r = sym_code_r(amax, s);
  if (real && threadIdx.x == 0) xs[row] = amax > 0.f ? s : 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = threadIdx.x + c * NT;   // idx % 8 == threadIdx.x % 8 (NT % 8 == 0)
    const v4i code = codes16(v[c], s, r);
    // the 8 chunks of a group sit on 8 consecutive lanes (K % 128 == 0)
    int t = idx < nch ? byte_sum16(code) : 0;
    t += __shfl_xor(t, 1, kWave);
    t += __shfl_xor(t, 2, kWave);
    t += __shfl_xor(t, 4, kWave);
    if (idx < nch) {
      if (real && xq) st16(xq + (int64_t)row * K + (int64_t)idx * 16, code);
      const int g = idx >> 3, j = (idx & 7) >> 1, h = idx & 1;
      st16(panel + ((((int64_t)g * 2 + h) * MR + row) * 4 + j) * 16, panel_order16(code));
      if ((idx & 7) == 0) {
        sums[g * kPanelRows + row] = t;
        if (row == 0)   // sum rows past the panel rows: zeros too
          for (int rr = MR; rr < kPanelRows; ++rr) sums[g * kPanelRows + rr] = 0;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM on the panel: one workgroup per 16-row weight block, WAVES waves each
// owning a contiguous run of units, every unit of the run requested at once
// (RING >= the longest run).  I32 output: the per-group accumulators.
//
// LDS: the block's scales [16][G] and zero points [16][G] (fp16) and the
// token sums [G][16] (int32), each in whole kilobytes, then each wave's ring
// of 2 KB unit slots.  The three small arrays arrive by buffer-to-LDS loads
// issued before any weight request, one kilobyte per wave-instruction; each
// wave then issues its whole run and only afterwards waits for the small
// arrays (older than its run, so a wait that leaves the run's requests in
// flight) and meets the others at a barrier.
// ---------------------------------------------------------------------------
// OUTL: the INT8 outlier side path as in k_w4a8_dec, its records loaded with
// each unit and its operand laid out in the panel's byte order.
template <int WAVES, int RING, bool OUTL, typename OutT>
__global__ __launch_bounds__(64 * WAVES) void k_w4a8_fdec(
    const int8_t* __restrict__ panel, const int* __restrict__ tsum, const float* __restrict__ xs,
    const int32_t* __restrict__ wq, const uint16_t* __restrict__ wscale,
    const uint16_t* __restrict__ wzero, const uint64_t* __restrict__ orec,
    const float* __restrict__ os8, int M, int MR, int N, int K, OutT* __restrict__ y) {
  constexpr bool kI32 = __is_same(OutT, int32_t);
  // loads per unit: 2 weight DMAs, 4 token fragments (, 1 outlier record load)
  constexpr int PU = OUTL ? 7 : 6;
  static_assert(PU * RING <= 63, "vmcnt budget of wait_vmcnt");
  extern __shared__ __attribute__((aligned(16))) u32 smem[];
  __shared__ v4f red[kI32 ? 1 : WAVES][64];
  __shared__ v4i redo[OUTL ? WAVES : 1][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int n_base = blockIdx.x * 16;
  const int G = K >> 7, RB = K >> 1;
  const int GY = OUTL ? G + 1 : G;   // int32 output slices per token: groups (+ side sum)
  const int units = (RB + kUnitBytes - 1) / kUnitBytes;
  // run of units of this wave, the mapping rotated from one workgroup to the
  // next of the same XCD (workgroups are dealt to the 8 XCDs in turn), so
  // that they do not all read the same token lines at once; the launcher
  // guarantees WAVES <= units: every run holds at least one unit
  const int run = (wave + (int)(blockIdx.x >> 3)) % WAVES;
  const int ub = (int)((int64_t)units * run / WAVES), ue = (int)((int64_t)units * (run + 1) / WAVES);
  const int kb_sz = kb_of_chunks(2 * G), kb_sum = kb_of_chunks(4 * G);
  int8_t* lds = reinterpret_cast<int8_t*>(smem);
  const uint16_t* sl = reinterpret_cast<const uint16_t*>(lds);
  const uint16_t* zl = reinterpret_cast<const uint16_t*>(lds + 1024 * kb_sz);
  const int8_t* suml = lds + 2048 * kb_sz;
  int8_t* ring = lds + 1024 * (2 * kb_sz + kb_sum) + wave * RING * 2048;

  const int rows_n = min(16, N - n_base);
  const rsrc_t wr = make_rsrc(wq + (int64_t)n_base * (K >> 3), (u32)(rows_n * RB));
  const rsrc_t xr = make_rsrc(panel, (u32)(G * 128 * MR));
  const u32 xoff = r < MR ? (u32)((r * 4 + j) * 16) : kOOB;   // rows >= MR: zero tokens
  // outlier records of weight row r: unit q's two groups are 16 bytes at 16 q
  const rsrc_t orr = OUTL ? make_rsrc(orec + (int64_t)n_base * G, (u32)(rows_n * G * 8)) : wr;

  // 1. scales, zero points and token sums into LDS
  stage_block_sz<WAVES>(lds, make_rsrc(wscale + (int64_t)n_base * G, (u32)(rows_n * G * 2)),
                        make_rsrc(wzero + (int64_t)n_base * G, (u32)(rows_n * G * 2)), rows_n, G,
                        make_rsrc(tsum, (u32)(G * 64)), kb_sum);
  float sx[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!kI32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * j + i;
      sx[i] = xs[m < M ? m : M - 1];
    }
  }
  // every wave's small-array requests ahead of any weight request
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // 2. every unit of the run: two whole-line DMAs (rows 8h..8h+7, lane l:
  // row 8h + l/8, chunk (l % 8) ^ f(row)) and four token fragments.  With
  // the outlier side path, whose operand building is VALU-heavy and needs no
  // weights, the tokens and records of the whole run go first and the side
  // sums are formed while the weights are still on their way.
  v4i tk[RING][2][2], orc[OUTL ? RING : 1];
  auto weights = [&](int i) {
    const int q = min(ub + i, ue - 1);   // past the run: the last unit again
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * h + (lane >> 3);
      const int ch = (lane & 7) ^ ((row >> 1) & 7);
      const u32 o = 128 * q + 16 * ch < RB ? (u32)(row * RB + 128 * q + 16 * ch) : kOOB;
      dma16(wr, ring + i * 2048 + 1024 * h, o);
    }
  };
  auto tokens = [&](int i) {
    const int q = min(ub + i, ue - 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int g = 2 * q + s;   // g == G (odd G): past the panel, zeros
#pragma unroll
      for (int h = 0; h < 2; ++h) tk[i][s][h] = bld16(xr, xoff + (u32)((g * 2 + h) * 64 * MR));
    }
    if constexpr (OUTL) orc[i] = bld16(orr, (u32)(r * G * 8 + 16 * q));
  };
#pragma unroll
  for (int i = 0; i < RING; ++i) {
    if constexpr (OUTL) {
      tokens(i);
    } else {
      weights(i);
      tokens(i);
    }
  }
  if constexpr (OUTL) {
#pragma unroll
    for (int i = 0; i < RING; ++i) weights(i);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the small arrays are older than every request of the run (with the side
  // path: than every weight request, the tokens and records too)
  wait_vmcnt(OUTL ? 2 * RING : PU * RING);
  lds_barrier();
  v4i oacc = {0, 0, 0, 0};
  if constexpr (OUTL) {
    // a repeated unit past the run adds nothing; a group past G has zero tokens
#pragma unroll
    for (int i = 0; i < RING; ++i) {
      if (ub + i < ue) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u32 lo = (u32)orc[i][2 * s], hi = (u32)orc[i][2 * s + 1];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            oacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                tk[i][s][h], outlier_operand_panel(lo, hi, 32 * j + 16 * h), oacc, 0, 0, 0);
        }
      }
    }
  }

  // 3. consume the units in issue order
  int rsl[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) rsl[s] = r * 128 + (((4 * s + j) ^ ((r >> 1) & 7)) << 4);
  v4f yacc = {0.f, 0.f, 0.f, 0.f};
  const int n = n_base + r;
#pragma unroll
  for (int i = 0; i < RING; ++i) {
    const bool live = ub + i < ue;
    const int q = min(ub + i, ue - 1);
    wait_vmcnt((OUTL ? 2 : PU) * (RING - 1 - i));
    const int8_t* slot = ring + i * 2048;
    const v4i f0 = *reinterpret_cast<const v4i*>(slot + rsl[0]);
    const v4i f1 = *reinterpret_cast<const v4i*>(slot + rsl[1]);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const v4i f = s ? f1 : f0;
      const int g = 2 * q + s;
      const bool gin = g < G;
      const int gg = gin ? g : G - 1;   // g == G: zero tokens, zero sums below
      const int z = (int)f16_bits_to_f32(zl[r * G + gg]);
      v4i ts = *reinterpret_cast<const v4i*>(suml + 64 * gg + 16 * j);
      if (!gin) ts = v4i{0, 0, 0, 0};
      v4i acc;   // |z| <= 15, |token sum| <= 128 * 127: exact 24-bit products
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __mul24(-z, ts[e]);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(tk[i][s][0], unpack_pair((u32)f[0], (u32)f[1]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(tk[i][s][1], unpack_pair((u32)f[2], (u32)f[3]), acc, 0, 0, 0);
      if constexpr (kI32) {
        if (live && gin && n < N) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 4 * j + e;
            if (m < M) y[((int64_t)m * GY + g) * N + n] = acc[e];
          }
        }
      } else {
        const float sc = live && gin ? f16_bits_to_f32(sl[r * G + gg]) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) yacc[e] = __builtin_fmaf(sc, (float)acc[e], yacc[e]);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (!kI32) red[wave][lane] = yacc;
  if constexpr (OUTL) redo[wave][lane] = oacc;
  if constexpr (!kI32 || OUTL) {
    __syncthreads();
    if (tid < 64 && n < N) {
      v4i osum = {0, 0, 0, 0};
      if constexpr (OUTL) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) osum += redo[w][lane];
      }
      if constexpr (kI32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 4 * j + e;
          if (m < M) y[((int64_t)m * GY + G) * N + n] = osum[e];
        }
      } else {
        v4f sum = red[0][lane];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) sum += red[w][lane];
        const float s8 = OUTL ? os8[n] : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 4 * j + e;
          // y = s_x (sum_g s_g acc_g + s8 acc_o)
          const float t = OUTL ? __builtin_fmaf(s8, (float)osum[e], sum[e]) : sum[e];
          if (m < M) y[(int64_t)m * N + n] = Out<OutT>::cvt(t * sx[e]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

constexpr int kPanelMaxK = 16384;   // 64 units of 128 weight bytes: 16 waves x ring 4
constexpr int kMaxRing = 4;

// Panel rows for M token rows: M rounded up to 1, 2, 4, 8 or 16 (the quantizer
// and the GEMM both derive it from M).
int panel_rows(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

bool panel_shape(int64_t M, int64_t K) {
  return M >= 1 && M <= kPanelRows && K >= 128 && K % 128 == 0 && K <= kPanelMaxK;
}

struct GemmPlan {
  bool ok = false;
  int waves = 0, ring = 0;
  size_t lds = 0;
};

// Launch shape of the panel GEMM: 16 waves per workgroup while the 16-row
// blocks fit in one workgroup per CU (256), else 8 (more workgroups resident
// per CU), 16 again if 8 would need a ring deeper than 4; never more waves
// than units, so that every run holds at least one.
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan p;
  if (!panel_shape(M, K) || N < 1) return p;
  const int64_t G = K / 128, units = (K / 2 + kUnitBytes - 1) / kUnitBytes;
  const int64_t nblocks = (N + 15) / 16;
  int waves = nblocks <= 256 ? 16 : 8;
  if ((units + waves - 1) / waves > kMaxRing) waves = 16;
  while (waves > 1 && waves > units) waves /= 2;
  const int ring = (int)((units + waves - 1) / waves);
  if (ring > kMaxRing) return p;
  p.lds = (size_t)1024 * (2 * kb_of_chunks((int)(2 * G)) + kb_of_chunks((int)(4 * G))) +
          (size_t)waves * ring * 2048;
  if (p.lds + (size_t)waves * 64 * sizeof(v4f) > 160 * 1024) return p;
  p.ok = true;
  p.waves = waves;
  p.ring = ring;
  return p;
}

// When quantize_gemm_w4a8 takes the panel pair: on layers of 257-383 16-row
// weight blocks.  Measured on MI355X, whole calls (quantizer + GEMM) against
// the per-token quantizer + the plain W4A8 GEMM, weights rotated through
// 600 MB.  On 256 blocks or fewer the pair was slower at every size tried
// (K = 11008, N = 4096: 6-11%; K = 4096, N = 4096: 2-6%): the panel quantizer
// costs ~0.4 us more than the plain one, more than the panel GEMM gains
// there.  From 384 blocks the plain GEMM is the wide kernel, which is faster
// than the pair at every size tried (K = 4096, N = 11008: 1 row 10.3 against
// 9.1 us, 16 rows 13.2 against 10.3; N = 14336, 28672 likewise).  Where the
// plain GEMM is the int8 dot-product kernel (one token row, or two with
// K <= 4096) the plain pair is faster too (K = 4096, N = 5120: 1 row 6.86
// against 8.89 us, 2 rows 7.85 against 8.96; K = 11008, N = 5120, 1 row
// 11.2 against 18.6).
bool use_panel(int64_t M, int64_t N, int64_t K) {
  const int64_t nblocks = (N + 15) / 16;
  const bool dot_kernel = M == 1 || (M == 2 && K <= 4096);
  return !dot_kernel && plan_gemm(M, N, K).ok && nblocks > 256 && nblocks < 384;
}

template <int DT>
hipError_t quant_panel_dt(const void* x, int M, int64_t K, int8_t* xq, float* xs, int8_t* panel,
                          int* sums, hipStream_t st) {
  const int64_t nch = K / 16;   // K <= 16384: at most 1024 chunks
  const int MR = panel_rows(M);
  const dim3 grid((unsigned)kPanelRows);
  if (nch <= 256)
    k_quant_panel<DT, 1, 256><<<grid, 256, 0, st>>>(x, M, K, MR, xq, xs, panel, sums);
  else if (nch <= 512)
    k_quant_panel<DT, 1, 512><<<grid, 512, 0, st>>>(x, M, K, MR, xq, xs, panel, sums);
  else
    k_quant_panel<DT, 2, 512><<<grid, 512, 0, st>>>(x, M, K, MR, xq, xs, panel, sums);
  return hipGetLastError();
}

// Operands of one panel GEMM launch (orec and os8 only for the outlier form).
struct FdecArgs {
  const int8_t* panel;
  const int* sums;
  const float* xs;
  const int32_t* wq;
  const uint16_t* ws;
  const uint16_t* wz;
  const uint64_t* orec;
  const float* os8;
  int M, N, K;
};

template <int WAVES, bool OUTL, typename OutT>
void fdec_ring(int ring, const FdecArgs& a, OutT* y, size_t lds, hipStream_t st) {
  const dim3 grid((unsigned)((a.N + 15) / 16)), block(64 * WAVES);
  const int MR = panel_rows(a.M);
#define QG_FDEC(R)                                                                              \
  k_w4a8_fdec<WAVES, R, OUTL, OutT><<<grid, block, lds, st>>>(a.panel, a.sums, a.xs, a.wq, a.ws, \
                                                              a.wz, a.orec, a.os8, a.M, MR, a.N, \
                                                              a.K, y)
  switch (ring) {
    case 1: QG_FDEC(1); break;
    case 2: QG_FDEC(2); break;
    case 3: QG_FDEC(3); break;
    default: QG_FDEC(4); break;
  }
#undef QG_FDEC
}

template <bool OUTL, typename OutT>
hipError_t fdec_t(const GemmPlan& p, const FdecArgs& a, OutT* y, hipStream_t st) {
  switch (p.waves) {
    case 16: fdec_ring<16, OUTL, OutT>(p.ring, a, y, p.lds, st); break;
    case 8: fdec_ring<8, OUTL, OutT>(p.ring, a, y, p.lds, st); break;
    case 4: fdec_ring<4, OUTL, OutT>(p.ring, a, y, p.lds, st); break;
    case 2: fdec_ring<2, OUTL, OutT>(p.ring, a, y, p.lds, st); break;
    default: fdec_ring<1, OUTL, OutT>(p.ring, a, y, p.lds, st); break;
  }
  return hipGetLastError();
}

template <bool OUTL>
hipError_t fdec_y(const GemmPlan& p, const FdecArgs& a, void* y, int y_dtype, hipStream_t st) {
  switch (y_dtype) {
    case F32: return fdec_t<OUTL, float>(p, a, (float*)y, st);
    case F16: return fdec_t<OUTL, _Float16>(p, a, (_Float16*)y, st);
    case BF16: return fdec_t<OUTL, uint16_t>(p, a, (uint16_t*)y, st);
    default: return fdec_t<OUTL, int32_t>(p, a, (int32_t*)y, st);
  }
}

int* panel_sums(void* panel, int64_t K) {
  return reinterpret_cast<int*>(reinterpret_cast<int8_t*>(panel) + K / 128 * 128 * kPanelRows);
}

}  // namespace

int64_t panel_bytes(int64_t M, int64_t K) {
  return panel_shape(M, K) ? K / 128 * (128 * kPanelRows + 4 * kPanelRows) : 0;
}

bool gemm_w4a8_panel_ok(int64_t M, int64_t N, int64_t K) { return plan_gemm(M, N, K).ok; }

int64_t quantize_gemm_w4a8_workspace(int64_t M, int64_t N, int64_t K) {
  return use_panel(M, N, K) ? panel_bytes(M, K) : 0;
}

hipError_t launch_quant_panel(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* xq,
                              float* xs, void* panel, hipStream_t st) {
  int8_t* pp = reinterpret_cast<int8_t*>(panel);
  int* sums = panel_sums(panel, K);
  switch (x_dtype) {
    case F32: return quant_panel_dt<F32>(x, (int)M, K, xq, xs, pp, sums, st);
    case F16: return quant_panel_dt<F16>(x, (int)M, K, xq, xs, pp, sums, st);
    default: return quant_panel_dt<BF16>(x, (int)M, K, xq, xs, pp, sums, st);
  }
}

hipError_t launch_gemm_w4a8_panel(const void* panel, const float* xs, const int32_t* wq,
                                  const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                                  int64_t K, void* y, int y_dtype, hipStream_t st) {
  const FdecArgs a{reinterpret_cast<const int8_t*>(panel), panel_sums(const_cast<void*>(panel), K),
                   xs, wq, ws, wz, nullptr, nullptr, (int)M, (int)N, (int)K};
  return fdec_y<false>(plan_gemm(M, N, K), a, y, y_dtype, st);
}

hipError_t launch_gemm_w4a8_outl_panel(const void* panel, const float* xs, const int32_t* wq,
                                       const uint16_t* ws, const uint16_t* wz,
                                       const uint64_t* orec, const float* os8, int64_t M,
                                       int64_t N, int64_t K, void* y, int y_dtype,
                                       hipStream_t st) {
  const FdecArgs a{reinterpret_cast<const int8_t*>(panel), panel_sums(const_cast<void*>(panel), K),
                   xs, wq, ws, wz, orec, os8, (int)M, (int)N, (int)K};
  return fdec_y<true>(plan_gemm(M, N, K), a, y, y_dtype, st);
}

hipError_t launch_quantize_gemm_w4a8(const void* x, int x_dtype, const int32_t* wq,
                                     const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                                     int64_t K, void* y, int y_dtype, int8_t* xq, float* xs,
                                     void* workspace, hipStream_t st) {
  if (!use_panel(M, N, K)) {   // the two kernels in sequence
    if (hipError_t e = launch_quant_per_token(x, x_dtype, M, K, xq, xs, st)) return e;
    return launch_gemm_w4a8(xq, xs, wq, ws, wz, M, N, K, y, y_dtype, st);
  }
  if (hipError_t e = launch_quant_panel(x, x_dtype, M, K, xq, xs, workspace, st)) return e;
  return launch_gemm_w4a8_panel(workspace, xs, wq, ws, wz, M, N, K, y, y_dtype, st);
}

// ---------------------------------------------------------------------------
// The library's own panel, for the entry point that allocates nothing: a
// fixed array in device memory, one per GPU (each device holds its own copy
// until the process ends), large enough for the biggest panel (K = 16384).
// In host code the name `scratch` is only a stand-in, not a device address:
// kernels and copies get the address hipGetSymbolAddress returns for the
// device, looked up once per device with that device current and kept.
// Every call on a GPU shares its array; calls that overlap on one GPU race.
// No part of it needs to start at zero: the panel quantizer writes every
// byte the panel GEMM reads.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = (int64_t)(kPanelMaxK / 128) * (128 * kPanelRows + 4 * kPanelRows);
static __device__ __align__(256) int8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of `scratch` on the device `st` belongs to (the current
// device for the null stream).
hipError_t scratch_address(hipStream_t st, void** out) {
  int cur = 0, dev = 0;
  if (hipError_t e = hipGetDevice(&cur)) return e;
  dev = cur;
  if (st)
    if (hipError_t e = hipStreamGetDevice(st, &dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur)
      if (hipError_t e = hipSetDevice(dev)) return e;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

int64_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t launch_quantize_gemm_w4a8_noalloc(const void* x, int x_dtype, const int32_t* wq,
                                             const uint16_t* ws, const uint16_t* wz, int64_t M,
                                             int64_t N, int64_t K, void* y, int y_dtype,
                                             int8_t* xq, float* xs, hipStream_t st) {
  const int64_t need = quantize_gemm_w4a8_workspace(M, N, K);
  void* panel = nullptr;
  if (need > 0) {
    if (need > kScratchBytes) return hipErrorInvalidValue;   // the API rejects this first
    if (hipError_t e = scratch_address(st, &panel)) return e;
  }
  return launch_quantize_gemm_w4a8(x, x_dtype, wq, ws, wz, M, N, K, y, y_dtype, xq, xs, panel, st);
}

}  // namespace qg
