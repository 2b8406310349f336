// W8A8 GEMM: acc[m,n] = sum_k xq[m,k] wq[n,k] (int8 x int8 -> exact int32 on the
// int8 matrix cores), y[m,n] = (acc * s_x[m]) * s_w[n].
// 「第4章：量化」 §2.3 (W8A8: the GEMM runs on int8 units), §1.1 (x_hat = x_int s);
// 「LLM推理降本五要素」 §2.1 (at decode the layer waits on weight bandwidth).
//
// Three kernels:
//  * decode (M <= 8, and M <= 16 on layers of at most 256 16-row blocks):
//    the weight stream is the whole cost.  Whole-line weight units transposed
//    through LDS into MFMA operands, token rows staged in LDS once per
//    workgroup (or per phase of K when they are too long); the K loop is
//    split across the waves and the int32 partials meet in LDS.
//  * wide decode (M <= 64): one 16-row weight block per wave over the whole
//    K, several blocks per workgroup sharing each phase's token-row panel.
//  * large M (prefill): 256x256 output tiles, K in 128-byte stages brought
//    into LDS by buffer-to-LDS DMA (two alternating stage buffers, XOR-swizzled
//    16-byte chunks), 4 waves each owning a 128x128 sub-tile of 32x32x32 int8
//    MFMAs.
#include <algorithm>
#include <array>
#include <type_traits>

#include "qg_decode.hpp"
#include "qg_device.hpp"
#include "qg_launch.hpp"

namespace qg {

template <typename OutT>
__device__ __forceinline__ OutT w8a8_epilogue(int acc, float sx, float sw) {
  return Out<OutT>::cvt(((float)acc * sx) * sw);
}
template <>
__device__ __forceinline__ int32_t w8a8_epilogue<int32_t>(int acc, float, float) {
  return acc;
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 16) on whole-line weight units (see qg_decode.hpp): a
// unit is two 64-deep int8 MFMA steps of 16 weight rows.  The K range is
// walked in `phases` contiguous runs of units (one unless the token rows are
// too long for LDS).  Per phase the token rows' slice is staged in LDS (MR
// rows, MR >= M, rows past M as zeros); wave w then streams its contiguous
// share of the phase's units in batches of UB, two batches in flight, each
// unit transposed through the wave's tile and multiplied against the matching
// token fragments.  The int32 partials of the waves meet in LDS.
// ---------------------------------------------------------------------------
// GEN = false compiles the common case (one block per workgroup, one phase)
// with those counts as constants: the general form measured ~1 us slower on
// the 45 MB FFN-up stream.
template <int MR, int WAVES, int UB, bool GEN, typename OutT>
__global__ __launch_bounds__(64 * WAVES) void k_w8a8_dec(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, const int8_t* __restrict__ wq,
    const float* __restrict__ ws, int M, int N, int K, OutT* __restrict__ y, int phases_arg) {
  extern __shared__ __attribute__((aligned(16))) int8_t xl[];   // MR rows of one phase's slice
  __shared__ __attribute__((aligned(16))) int8_t tiles[WAVES][kTileBytes];
  __shared__ v4i red[WAVES][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  // this workgroup's 16-row weight blocks [bb0, bb0 + nb) (one unless the
  // grid is smaller than the block count); block blk gets waves blk,
  // blk + nb, ..., which split its K
  const int nblocks = (N + 15) / 16;
  const int bb0 = GEN ? (int)((int64_t)nblocks * blockIdx.x / gridDim.x) : (int)blockIdx.x;
  const int nb = GEN ? (int)((int64_t)nblocks * (blockIdx.x + 1) / gridDim.x) - bb0 : 1;
  const int blk = GEN ? wave % nb : 0, sub = GEN ? wave / nb : wave;
  const int subs = GEN ? (WAVES - blk + nb - 1) / nb : WAVES;
  const int phases = GEN ? phases_arg : 1;
  const int n_base = (bb0 + blk) * 16;
  const int units = (K + kUnitBytes - 1) / kUnitBytes;
  const int pitch = stage_pitch(kUnitBytes * ((units + phases - 1) / phases));

  const int rows_n = min(16, N - n_base);
  const rsrc_t wr = make_rsrc_uniform(wq + (int64_t)n_base * K, (u32)(rows_n * K));
  const rsrc_t xr = make_rsrc(xq, (u32)(M * K));
  const UnitLanes ul = unit_lanes(lane, K);

  // epilogue scales, fetched behind the first phase's staging and weight
  // loads (vector loads complete in issue order: fetched first, they would
  // delay the staging) and long before the tail needs them; int32 output
  // takes no scales, and its scale pointers may be null
  const int n_out = n_base + r;
  float sw = 0.f, sx[4] = {0.f, 0.f, 0.f, 0.f};
  auto fetch_scales = [&]() {
    if constexpr (!std::is_same<OutT, int32_t>::value) {
      sw = ws[n_out < N ? n_out : N - 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * j + i;
        sx[i] = xs[m < M ? m : M - 1];
      }
    }
  };

  // Rows r >= MR, units past this wave's run and fragments past K read valid
  // LDS (row 0 of the slice): their weight operand is zero, and rows >= M are
  // never stored.
  const int8_t* xrow = xl + (r < MR ? r : 0) * pitch;
  int8_t* tile = tiles[wave];
  v4i acc = {0, 0, 0, 0};
  v4i b0[UB][2], b1[UB][2];
  for (int p = 0; p < phases; ++p) {
    const int pu0 = (int)((int64_t)units * p / phases), pu1 = (int)((int64_t)units * (p + 1) / phases);
    const int ub = pu0 + (int)((int64_t)(pu1 - pu0) * sub / subs);
    const int ue = pu0 + (int)((int64_t)(pu1 - pu0) * (sub + 1) / subs);
    const int col0 = kUnitBytes * pu0, cols = min(kUnitBytes * pu1, K) - col0;
    auto load = [&](v4i (&b)[UB][2], int q0) {
#pragma unroll
      for (int v = 0; v < UB; ++v) unit_load(b[v], wr, ul, q0 + v, q0 + v < ue, K);
      __builtin_amdgcn_sched_barrier(0);
    };
    if (p > 0) __syncthreads();   // every wave is done with the previous slice
    // the slice's token rows into LDS; the phase's first weight batch is
    // issued behind the first round of their loads
    stage_slice<MR, 64 * WAVES>(xl, pitch, xr, K, col0, cols, [&]() { load(b0, ub); });
    if (p == 0) fetch_scales();
    lds_barrier();

    auto mma = [&](const v4i (&b)[UB][2], int q0) {
#pragma unroll
      for (int v = 0; v < UB; ++v) {
        v4i f[2];
        unit_transpose(tile, b[v], ul, f);
        const bool qin = q0 + v < ue;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int ka = kUnitBytes * (q0 + v) + 64 * s + 16 * j;
          const v4i a = ld16(xrow + (qin && ka < K ? ka - col0 : 0));
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, f[s], acc, 0, 0, 0);
        }
      }
    };
    for (int q0 = ub; q0 < ue; q0 += 2 * UB) {
      load(b1, q0 + UB);
      mma(b0, q0);
      load(b0, q0 + 2 * UB);
      mma(b1, q0 + UB);
    }
  }

  red[wave][lane] = acc;
  __syncthreads();
  if (sub == 0) {   // wave blk: its block's partials, in wave order
    v4i sum = red[blk][lane];
    for (int sb = 1; sb < subs; ++sb) sum += red[blk + nb * sb][lane];
    if (n_out < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * j + i;
        if (m < M) y[(int64_t)m * N + n_out] = w8a8_epilogue<OutT>(sum[i], sx[i], sw);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wide decode kernel (up to 64 token rows, MT m-tiles of 16): a workgroup owns
// NB 16-row weight blocks, streamed over the whole K as whole-line units, and
// moves through K in phases of PU units.  Each block has KS x MS waves: KS
// split a phase's units, MS split the m-tiles (reading the same weights), so
// that a SIMD holds more than one wave to hide the LDS and MFMA latencies;
// the KS partial sums (exact int32) meet in LDS at the end.  A phase's panel
// of token rows (16 MT rows x 128 PU bytes) is staged in LDS once for all
// waves (two-deep ring, one barrier per phase), so one token-row byte read
// from L2 serves 16 NB weight rows.
// ---------------------------------------------------------------------------
template <int MT, int NB, int KS, int MS, int PU>
__host__ __device__ constexpr size_t w8a8_wide_static_lds() {
  return (size_t)2 * 16 * MT * (kUnitBytes * PU + 16) + (size_t)NB * KS * MS * kTileBytes +
         (size_t)(KS == 1 ? 1 : NB * MS * (KS - 1)) * (MT / MS) * 64 * 16;
}

template <int MT, int NB, int KS, int MS, int PU, typename OutT>
__global__ __launch_bounds__(64 * NB * KS * MS) void k_w8a8_wide(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, const int8_t* __restrict__ wq,
    const float* __restrict__ ws, int M, int N, int K, OutT* __restrict__ y) {
  static_assert(PU % KS == 0, "every wave of a block takes the same number of units");
  static_assert(MT % MS == 0, "every wave of a block takes the same number of m-tiles");
  constexpr int UPW = PU / KS, MTW = MT / MS;                     // units, m-tiles per wave
  constexpr int MR = 16 * MT, PB = kUnitBytes * PU, kThreads = 64 * NB * KS * MS;
  constexpr int kPitch = PB + 16;                      // odd number of 16-byte chunks
  constexpr int kRowChunks = PB / 16, kChunks = MR * kRowChunks;
  constexpr int CPT = (kChunks + kThreads - 1) / kThreads;
  constexpr bool kFull = CPT * kThreads == kChunks;
  __shared__ __attribute__((aligned(16))) int8_t xbuf[2][MR * kPitch];
  __shared__ __attribute__((aligned(16))) int8_t tiles[NB * KS * MS][kTileBytes];
  __shared__ v4i red[KS == 1 ? 1 : NB * MS * (KS - 1)][MTW][64];
  static_assert(sizeof(xbuf) + sizeof(tiles) + sizeof(red) == w8a8_wide_static_lds<MT, NB, KS, MS, PU>(),
                "static LDS bookkeeping");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blk = wave % NB, ks = (wave / NB) % KS, ms = wave / (NB * KS);
  const int r = lane & 15, j = lane >> 4;
  const int n_base = (blockIdx.x * NB + blk) * 16;
  const int units = (K + kUnitBytes - 1) / kUnitBytes;
  const int phases = (units + PU - 1) / PU;

  // rows past N (including a whole wave's block past N) read zeros
  const int rows_n = max(0, min(16, N - n_base));
  const rsrc_t wr = make_rsrc_uniform(wq + (int64_t)min(n_base, N - 1) * K, (u32)(rows_n * K));
  const rsrc_t xr = make_rsrc(xq, (u32)(M * K));
  const UnitLanes ul = unit_lanes(lane, K);

  struct Batch {
    v4i w[UPW][2], x[CPT];
  };
  auto load = [&](Batch& bt, int p) {
#pragma unroll
    for (int v = 0; v < UPW; ++v) unit_load(bt.w[v], wr, ul, p * PU + ks * UPW + v, true, K);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + c * kThreads;
      const int row = chunk / kRowChunks, kb = p * PB + (chunk % kRowChunks) * 16;
      // rows >= M fall past the end of the resource and read zeros
      bt.x[c] = bld16(xr, kb < K ? (u32)(row * K + kb) : kOOB);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  int8_t* tile = tiles[wave];
  v4i acc[MTW];
#pragma unroll
  for (int mw = 0; mw < MTW; ++mw) acc[mw] = v4i{0, 0, 0, 0};
  auto process = [&](const Batch& bt, int p) {
    int8_t* buf = xbuf[p & 1];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + c * kThreads;
      if (kFull || chunk < kChunks)
        st16(buf + (chunk / kRowChunks) * kPitch + (chunk % kRowChunks) * 16, bt.x[c]);
    }
    // Panel p is complete once every wave is here; the buffer phase p + 1
    // overwrites was last read at phase p - 1, before this barrier.
    lds_barrier();
#pragma unroll
    for (int v = 0; v < UPW; ++v) {
      v4i f[2];
      unit_transpose(tile, bt.w[v], ul, f);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        // past K the weight operand is zero; keep the panel read in range
        const int kin = kUnitBytes * (ks * UPW + v) + 64 * s2 + 16 * j;
#pragma unroll
        for (int mw = 0; mw < MTW; ++mw) {
          const v4i a = ld16(buf + (16 * (ms * MTW + mw) + r) * kPitch + kin);
          acc[mw] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, f[s2], acc[mw], 0, 0, 0);
        }
      }
    }
  };

  Batch b0, b1;
  load(b0, 0);
  const int n_out = n_base + r;
  float sw = 0.f;
  if constexpr (!std::is_same<OutT, int32_t>::value) sw = ws[n_out < N ? n_out : N - 1];
  // every wave runs the same number of phases, so all reach every barrier
  for (int p = 0; p < phases; p += 2) {
    load(b1, p + 1);
    process(b0, p);
    load(b0, p + 2);
    process(b1, p + 1);
  }

  if constexpr (KS > 1) {
    // the block's other waves hand their partial sums to wave ks = 0
    if (ks > 0) {
#pragma unroll
      for (int mw = 0; mw < MTW; ++mw) red[((ks - 1) * MS + ms) * NB + blk][mw][lane] = acc[mw];
    }
    lds_barrier();
    if (ks > 0) return;
#pragma unroll
    for (int o = 0; o < KS - 1; ++o)
#pragma unroll
      for (int mw = 0; mw < MTW; ++mw) {
        const v4i t = red[(o * MS + ms) * NB + blk][mw][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mw][i] += t[i];
      }
  }
  if (n_out < N) {
#pragma unroll
    for (int mw = 0; mw < MTW; ++mw)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * (ms * MTW + mw) + 4 * j + i;
        if (m < M) {
          float sx = 0.f;
          if constexpr (!std::is_same<OutT, int32_t>::value) sx = xs[m];
          y[(int64_t)m * N + n_out] = w8a8_epilogue<OutT>(acc[mw][i], sx, sw);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Large-M kernel: 256x256 output tiles, K in 128-byte stages, 4 waves (2x2),
// each wave a 128x128 sub-tile of 32x32x32 int8 MFMAs (256 int32
// accumulators per lane, held in the accumulation registers).
//
// Operands reach LDS by buffer-load-to-LDS DMA (no register staging): per
// stage each wave issues 16 one-kilobyte DMA loads, each 8 rows x 128 bytes
// (whole cache lines).  Two 64 KB stage buffers alternate: the DMA of stage
// k+1 runs while stage k is multiplied.  Rows past M/N and bytes past K come
// back as zeros from the buffer resources' range check.
// LDS layout of a stage: A tile [256 rows][128 B] then B tile; row r's
// 16-byte chunk c sits at r*128 + 16*(c ^ f(r)), f(r) = (r >> 1) & 7, so 16
// consecutive rows reading the same chunk hit 16 different 16-byte bank
// groups.  The DMA writes lane l's 16 bytes to slot l of the kilobyte, so the
// swizzle is applied by choosing which chunk each lane fetches.
// ---------------------------------------------------------------------------
constexpr int TBM = 256, TBN = 256, TBK = 128;
// tile-rows per column-major group of the tile walk (see k_w8a8_tiled)
constexpr int kPrefillGroupRows = 4;
constexpr int kStageBytes = (TBM + TBN) * TBK;   // 64 KB

__shared__ __attribute__((aligned(16))) int8_t g_stage0[kStageBytes];
__shared__ __attribute__((aligned(16))) int8_t g_stage1[kStageBytes];

// gfx950 LDS: 64 banks x 4 bytes; a 16-byte-per-lane read serves 16 lanes
// per cycle.  With 128-byte rows, rows r and r+1 share a 256-byte bank row, so
// 16 consecutive rows reading the same chunk are conflict-free when the 8 rows
// of each parity get 8 different chunk slots: f(r) = (r >> 1) & 7.
__device__ __forceinline__ int swz_f(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int ch) { return row * TBK + ((ch ^ swz_f(row)) << 4); }

#define QG_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// DMA of one stage, spread over the multiply of the previous stage.  The
// stage is 64 one-kilobyte loads; with NW waves each issues 64/NW of them.
// Load q covers rows 8q..8q+7 of A (q < 32) or B (q >= 32); lane l fetches row
// 8q + (l >> 3), chunk (l & 7) ^ f(row).  f(row) takes bits 1-2 from the row
// within the 8-row block and bit 3 from the block's parity, so each lane
// needs two byte offsets (even and odd blocks); the row step is a scalar
// offset.
template <int NW>
struct PrefillDma {
  int8_t* buf;
  rsrc_t ar, br;
  u32 voff[2];
  int wave;
  __device__ __forceinline__ void issue(int i, int K) const {
    const int q = wave * (64 / NW) + i;
    int8_t* dst = buf + (q < 32 ? 0 : TBM * TBK) + (q & 31) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 32 ? ar : br, QG_LDS(dst), 16, voff[q & 1],
                                             (u32)(8 * (q & 31) * K), 0, 0);
  }
};

template <int NW>
__device__ __forceinline__ PrefillDma<NW> prefill_dma_setup(int8_t* buf, int kt, int K, rsrc_t ar,
                                                            rsrc_t br, int wave, int lane) {
  const int row_local = lane >> 3, slot = lane & 7;
  PrefillDma<NW> d{buf, ar, br, {0u, 0u}, wave};
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int k = kt * TBK + 16 * (slot ^ swz_f(8 * par + row_local));
    d.voff[par] = k < K ? (u32)(row_local * K + k) : kOOB;
  }
  return d;
}

template <int NW>
__device__ __forceinline__ void prefill_dma(int8_t* buf, int kt, int K, rsrc_t ar, rsrc_t br,
                                            int wave, int lane) {
  const PrefillDma<NW> d = prefill_dma_setup<NW>(buf, kt, K, ar, br, wave, lane);
#pragma unroll
  for (int i = 0; i < 64 / NW; ++i) d.issue(i, K);
}

// Wave tile: 4 row tiles (128 rows) x WJ column tiles (32*WJ columns) of
// 32x32 MFMAs; WJ = 4 with 4 waves (2x2), WJ = 2 with 8 waves (2x4).
template <int WJ>
__device__ __forceinline__ void prefill_frag(const int8_t* buf, int ks, int row_a, int row_b,
                                             int lane, v4i (&af)[4], v4i (&bf)[WJ]) {
  const int ch = ks * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    af[i] = *reinterpret_cast<const v4i*>(&buf[swz(row_a + i * 32 + (lane & 31), ch)]);
#pragma unroll
  for (int j = 0; j < WJ; ++j)
    bf[j] = *reinterpret_cast<const v4i*>(&buf[TBM * TBK + swz(row_b + j * 32 + (lane & 31), ch)]);
}

// Multiply one stage: 4 sub-steps of 32 k; the fragments of sub-step ks+1 are
// read from LDS while the MFMAs of sub-step ks run (two fragment sets).  The
// wave's DMA loads of the next stage are slotted in between MFMAs over the
// first half of the stage, so the wave never stalls on a burst of loads and
// the second half covers their latency.
template <int NW, int WJ>
__device__ __forceinline__ void prefill_mma(const int8_t* buf, int row_a, int row_b, int lane,
                                            v16i (&acc)[4][WJ], const PrefillDma<NW>& next,
                                            int K) {
  constexpr int kLoads = 64 / NW;              // DMA loads per wave per stage
  constexpr int kSlots = 2 * 4 * WJ;           // MFMAs in the first two sub-steps
  constexpr int kEvery = kSlots / kLoads;
  v4i af[2][4], bf[2][WJ];
  prefill_frag<WJ>(buf, 0, row_a, row_b, lane, af[0], bf[0]);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks < 3) prefill_frag<WJ>(buf, ks + 1, row_a, row_b, lane, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < WJ; ++j) {
        // weight fragment as the first operand: the accumulator comes out
        // transposed (lane = token row), see the epilogue
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[ks & 1][j], af[ks & 1][i], acc[i][j], 0, 0, 0);
        const int slot = (ks * 4 + i) * WJ + j;
        if (slot < kSlots && (slot % kEvery) == kEvery - 1) next.issue(slot / kEvery, K);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Wait until this wave's DMA loads have landed, then meet the other waves:
// after the barrier the whole stage is in LDS and every wave has finished
// reading the other buffer, which the next DMA overwrites.  One asm statement
// with a memory clobber, so no LDS access moves across it.
__device__ __forceinline__ void prefill_stage_sync() {
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

// Scales of the tile's 256 token rows and 256 weight rows, staged in LDS.
__shared__ __attribute__((aligned(16))) float g_tile_scale[TBM + TBN];

template <int NW, typename OutT>
__global__ __launch_bounds__(64 * NW) void k_w8a8_tiled(const int8_t* __restrict__ xq,
                                                        const float* __restrict__ xs,
                                                        const int8_t* __restrict__ wq,
                                                        const float* __restrict__ ws, int M,
                                                        int N, int K, OutT* __restrict__ y,
                                                        int vec_store) {
  constexpr int WJ = NW == 4 ? 4 : 2;           // column tiles per wave
  constexpr int WAVES_N = NW / 2;               // waves across the 256 columns
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: the DMA's LDS address (M0) and buffer resource
  // must be wave-uniform values
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int row_a = wm * 128, row_b = wn * 32 * WJ;

  // Tile order: the hardware hands consecutive workgroups to the 8 XCDs in
  // turn; renumber so each XCD walks a contiguous run of tiles, and walk
  // tiles in column-major groups of 4 tile-rows so tiles sharing A rows and B
  // columns run close together on the same XCD's L2.
  const int tiles_m = (M + TBM - 1) / TBM, tiles_n = (N + TBN - 1) / TBN;
  const int total = tiles_m * tiles_n;
  int bid = blockIdx.x;
  {
    const int per = total / 8, rem = total % 8;   // xcd x gets per + (x < rem) tiles
    const int xcd = bid % 8, idx = bid / 8;
    bid = xcd * per + (xcd < rem ? xcd : rem) + idx;
  }
  constexpr int GROUP = kPrefillGroupRows;
  const int group = bid / (GROUP * tiles_n);
  const int first_m = group * GROUP;
  const int gsize = (tiles_m - first_m) < GROUP ? (tiles_m - first_m) : GROUP;
  const int tm = first_m + (bid % (GROUP * tiles_n)) % gsize;
  const int tn = (bid % (GROUP * tiles_n)) / gsize;
  const int m0 = tm * TBM, n0 = tn * TBN;

  const rsrc_t ar = make_rsrc(xq + (int64_t)m0 * K, (u32)(min(TBM, M - m0) * K));
  const rsrc_t br = make_rsrc(wq + (int64_t)n0 * K, (u32)(min(TBN, N - n0) * K));

  v16i acc[4][WJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j) acc[i][j] = v16i{};

  constexpr bool kI32 = std::is_same<OutT, int32_t>::value;
  if constexpr (!kI32) {   // (int32 output takes no scales; its pointers may be null)
    for (int t = tid; t < TBM + TBN; t += 64 * NW) {
      const int m = m0 + t, n = n0 + t - TBM;
      g_tile_scale[t] = t < TBM ? (m < M ? xs[m] : 0.f) : (n < N ? ws[n] : 0.f);
    }
  }

  const int nk = (K + TBK - 1) / TBK;
  prefill_dma<NW>(g_stage0, 0, K, ar, br, wave, lane);
  for (int kt = 0; kt < nk; kt += 2) {
    // stages past nk are loaded as zeros and add nothing; multiplying them
    // (at most one extra stage, when nk is odd) keeps the loop branch-free
    prefill_stage_sync();
    prefill_mma<NW, WJ>(g_stage0, row_a, row_b, lane, acc,
                        prefill_dma_setup<NW>(g_stage1, kt + 1, K, ar, br, wave, lane), K);
    prefill_stage_sync();
    prefill_mma<NW, WJ>(g_stage1, row_a, row_b, lane, acc,
                        prefill_dma_setup<NW>(g_stage0, kt + 2, K, ar, br, wave, lane), K);
  }

  // The MFMAs ran with the weight fragment first, so accumulator (i, j) holds
  // the transposed 32x32 block: lane l has token row 32i + (l & 31) of the
  // wave tile, and register e the weight row (output column) 32j + 8(e >> 2)
  // + 4(l >> 5) + (e & 3) -- four consecutive output columns per e >> 2.
  //
  // Epilogue: the last (zero) DMA has landed and every wave is done with the
  // stage buffers, which now serve as wave-private 16 KB staging regions: a
  // pass writes 128 token rows x 128 bytes of output (two column tiles of
  // 2-byte outputs, one of 4-byte outputs) into the region, then reads it
  // back as whole 16-byte chunks and stores whole 128-byte lines of y.  Tiles
  // that cross the edge of y, or a y that is not 16-byte aligned per row,
  // take element stores instead.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  constexpr int E = (int)sizeof(OutT);
  constexpr int JP = E == 2 ? 2 : 1;               // column tiles per pass
  const int lr = lane & 31, lc = 4 * (lane >> 5);
  float sx[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!kI32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sx[i] = g_tile_scale[row_a + 32 * i + lr];
  }
  auto scaled4 = [&](int i, int j, int eb) {      // 4 consecutive outputs
    v4f sw = {0.f, 0.f, 0.f, 0.f};
    if constexpr (!kI32) sw = *reinterpret_cast<const v4f*>(&g_tile_scale[TBM + row_b + 32 * j + 8 * eb + lc]);
    OutT o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = w8a8_epilogue<OutT>(acc[i][j][4 * eb + t], sx[i], sw[t]);
    return std::array<OutT, 4>{o[0], o[1], o[2], o[3]};
  };
  const bool full = vec_store && m0 + TBM <= M && n0 + TBN <= N;
  if (full) {
    int8_t* reg = (wave < 4 ? g_stage0 : g_stage1) + (wave & 3) * 16384;
#pragma unroll
    for (int jp = 0; jp < WJ; jp += JP) {
#pragma unroll
      for (int jj = 0; jj < JP; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int eb = 0; eb < 4; ++eb) {
            const std::array<OutT, 4> o = scaled4(i, jp + jj, eb);
            const int row = 32 * i + lr, byte = E * (32 * jj + 8 * eb + lc);
            int8_t* d = reg + row * 128 + (((byte >> 4) ^ (row & 7)) << 4) + (byte & 15);
            if constexpr (E == 2) {
              uint16_t h[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) h[t] = __builtin_bit_cast(uint16_t, o[t]);
              *reinterpret_cast<uint2*>(d) = uint2{(u32)h[0] | ((u32)h[1] << 16), (u32)h[2] | ((u32)h[3] << 16)};
            } else {
              u32 w[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) w[t] = __builtin_bit_cast(u32, o[t]);
              st16(d, v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]});
            }
          }
      // one wave's LDS accesses execute in order: the reads below see the
      // writes above, and the next pass's writes follow these reads
      asm volatile("" ::: "memory");
      int8_t* ybase = reinterpret_cast<int8_t*>(y) +
                      ((int64_t)(m0 + row_a) * N + n0 + row_b + 32 * jp) * E;
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int row = 8 * it + (lane >> 3), ch = lane & 7;
        const v4i v = ld16(reg + row * 128 + ((ch ^ (row & 7)) << 4));
        st16(ybase + (int64_t)row * N * E + 16 * ch, v);
      }
      asm volatile("" ::: "memory");
    }
  } else {
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + row_a + 32 * i + lr;
        if (m >= M) continue;
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) {
          const std::array<OutT, 4> o = scaled4(i, j, eb);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int n = n0 + row_b + 32 * j + 8 * eb + lc + t;
            if (n < N) y[(int64_t)m * N + n] = o[t];
          }
        }
      }
  }
}

constexpr int kPrefillWaves = 8;

// Waves per weight block (K split KS ways, PU units per phase), measured on
// MI355X: with one block per workgroup (narrow layers, N < 6144) 4 (K = 11008,
// N = 4096, 64 rows 38.5 -> 19.2 us; K = N = 4096 16.8 -> 10.0 us), and 4 for
// 33-64 rows over 2-3 blocks (K = 4096, N = 8192, 64 rows 13.8 -> 12.7 us;
// N = 11008 15.3 -> 14.7).  Otherwise the single wave per block streams near
// the weight-read rate already and a split only adds its reduction.
template <int MT, int NB>
struct W8Split {
  static constexpr int KS = NB == 1 || (MT >= 3 && NB <= 3) ? 4 : 1;
  static constexpr int MS = 1;
  static constexpr int PU = KS > 1 ? 4 : (MT <= 2 ? 4 : 2);
};

template <int MT, int NB, typename OutT>
static void launch_w8a8_wide_nb(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws,
                                int M, int N, int K, OutT* y, hipStream_t st) {
  using S = W8Split<MT, NB>;
  static_assert(w8a8_wide_static_lds<MT, NB, S::KS, S::MS, S::PU>() <= kLdsBytesPerCU, "LDS of a CU");
  const int nblocks = (N + 15) / 16;
  const dim3 grid((unsigned)((nblocks + NB - 1) / NB)), block(64 * NB * S::KS * S::MS);
  k_w8a8_wide<MT, NB, S::KS, S::MS, S::PU, OutT><<<grid, block, 0, st>>>(xq, xs, wq, ws, M, N, K, y);
}

template <int MT, typename OutT>
static void launch_w8a8_wide(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws,
                             int M, int N, int K, OutT* y, hipStream_t st) {
  switch (wide_waves(N)) {
    case 1: launch_w8a8_wide_nb<MT, 1, OutT>(xq, xs, wq, ws, M, N, K, y, st); break;
    case 2: launch_w8a8_wide_nb<MT, 2, OutT>(xq, xs, wq, ws, M, N, K, y, st); break;
    case 3: launch_w8a8_wide_nb<MT, 3, OutT>(xq, xs, wq, ws, M, N, K, y, st); break;
    default: launch_w8a8_wide_nb<MT, 4, OutT>(xq, xs, wq, ws, M, N, K, y, st); break;
  }
}

// Token rows longer than kDecLdsMaxBytes (a long K: the down projection of
// an FFN) still stage whole in LDS up to kDecLdsBigBytes, at one workgroup
// per compute unit; beyond that the decode kernel walks K in phases, each
// staging its own slice of the rows.
constexpr size_t kDecLdsBigBytes = 112 * 1024;

// Compute units of an MI355X.
constexpr int kDecCUs = 256;

// LDS bytes of the decode kernel's token slice with `phases` phases (the
// kernel's own pitch: whole units per phase).
static size_t dec_lds(int mr, int K, int phases) {
  const int units = (K + kUnitBytes - 1) / kUnitBytes;
  return (size_t)mr * stage_pitch(kUnitBytes * ((units + phases - 1) / phases));
}

// Waves per 16-row workgroup of the decode kernel (they split K): more when
// few 16-row blocks would leave the chip short of loads in flight (measured
// on MI355X: K = 11008, N = 4096 and K = 4096, N = 11008; 16 waves is slower).
static int dec_waves(int N, int K, size_t lds) {
  if (lds > kDecLdsMaxBytes) return 8;
  return (N + 15) / 16 <= 384 && K >= 4096 ? 8 : 4;
}

template <int WAVES, bool GEN, typename OutT>
static void dec_mr(int mr, const int8_t* xq, const float* xs, const int8_t* wq, const float* ws,
                   int M, int N, int K, OutT* y, size_t lds, int phases, int groups,
                   hipStream_t st) {
  constexpr int UB = 2;
  const dim3 grid((unsigned)groups), block(64 * WAVES);
  switch (mr) {
    case 1: k_w8a8_dec<1, WAVES, UB, GEN, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, M, N, K, y, phases); break;
    case 2: k_w8a8_dec<2, WAVES, UB, GEN, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, M, N, K, y, phases); break;
    case 4: k_w8a8_dec<4, WAVES, UB, GEN, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, M, N, K, y, phases); break;
    case 8: k_w8a8_dec<8, WAVES, UB, GEN, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, M, N, K, y, phases); break;
    default: k_w8a8_dec<16, WAVES, UB, GEN, OutT><<<grid, block, lds, st>>>(xq, xs, wq, ws, M, N, K, y, phases); break;
  }
}

template <typename OutT>
static hipError_t gemm_w8a8_t(const int8_t* xq, const float* xs, const int8_t* wq,
                              const float* ws, int M, int N, int K, OutT* y, hipStream_t st) {
  if (M <= 64) {
    const int mr = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    // 9..16 token rows: the decode kernel when N gives at most 256 blocks of
    // 16 weight rows (one workgroup per CU) and K is long enough to share
    // out (measured on MI355X: N = 4096 6.4 us against the wide kernel's
    // 8.4, K = 6912 7.9 against 12.5); wider layers (N = 11008: 10.9 against
    // 11.3 us) and short K (K = N = 512: 4.1 against 6.3 us) keep the wide
    // kernel
    if (M <= 8 || (M <= 16 && (N + 15) / 16 <= 256 && K >= 2048)) {
      const int units = (K + kUnitBytes - 1) / kUnitBytes;
      int phases = 1;
      while (phases < units && dec_lds(mr, K, phases) > kDecLdsBigBytes) ++phases;
      const size_t lds = dec_lds(mr, K, phases);
      const int nblocks = (N + 15) / 16;
      // One-block workgroups of 4 waves: how many fit a CU (LDS, and 28
      // waves at this kernel's register count).
      const size_t wg_lds = lds + 4 * (kTileBytes + 64 * sizeof(v4i));
      const int per_cu = (int)std::min<size_t>(7, kLdsBytesPerCU / wg_lds);
      if (nblocks > per_cu * kDecCUs && nblocks <= 4 * kDecCUs && lds <= kDecLdsMaxBytes) {
        // more blocks than one-block workgroups can be resident at once: one
        // workgroup of 12 waves per CU over 3-4 blocks instead of a second
        // round of workgroups (measured on MI355X: N = 13824, K = 5120, M = 8
        // 15.9 us against 18.8; with all one-block workgroups resident they
        // are faster, e.g. N = 11008: 10.7 against 11.0 us)
        dec_mr<12, true, OutT>(mr, xq, xs, wq, ws, M, N, K, y, lds, phases, kDecCUs, st);
      } else {
        const int waves = dec_waves(N, K, lds);
        if (phases > 1) {
          if (waves >= 8) dec_mr<8, true, OutT>(mr, xq, xs, wq, ws, M, N, K, y, lds, phases, nblocks, st);
          else dec_mr<4, true, OutT>(mr, xq, xs, wq, ws, M, N, K, y, lds, phases, nblocks, st);
        } else {
          if (waves >= 8) dec_mr<8, false, OutT>(mr, xq, xs, wq, ws, M, N, K, y, lds, 1, nblocks, st);
          else dec_mr<4, false, OutT>(mr, xq, xs, wq, ws, M, N, K, y, lds, 1, nblocks, st);
        }
      }
    } else if (M <= 16) {
      launch_w8a8_wide<1, OutT>(xq, xs, wq, ws, M, N, K, y, st);
    } else if (M <= 32) {
      launch_w8a8_wide<2, OutT>(xq, xs, wq, ws, M, N, K, y, st);
    } else if (M <= 48) {
      launch_w8a8_wide<3, OutT>(xq, xs, wq, ws, M, N, K, y, st);
    } else {
      launch_w8a8_wide<4, OutT>(xq, xs, wq, ws, M, N, K, y, st);
    }
  } else {
    const int tiles = ((M + TBM - 1) / TBM) * ((N + TBN - 1) / TBN);
    // whole-line stores need every row of y to start on a 16-byte boundary
    const int vec = ((uintptr_t)y % 16 == 0) && ((size_t)N * sizeof(OutT)) % 16 == 0;
    k_w8a8_tiled<kPrefillWaves, OutT><<<dim3((unsigned)tiles), dim3(64 * kPrefillWaves), 0, st>>>(
        xq, xs, wq, ws, M, N, K, y, vec);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_w8a8(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws,
                            int64_t M, int64_t N, int64_t K, void* y, int y_dtype, hipStream_t st) {
  const int m = (int)M, n = (int)N, k = (int)K;
  switch (y_dtype) {
    case F32: return gemm_w8a8_t<float>(xq, xs, wq, ws, m, n, k, (float*)y, st);
    case F16: return gemm_w8a8_t<_Float16>(xq, xs, wq, ws, m, n, k, (_Float16*)y, st);
    case BF16: return gemm_w8a8_t<uint16_t>(xq, xs, wq, ws, m, n, k, (uint16_t*)y, st);
    default: return gemm_w8a8_t<int32_t>(xq, xs, wq, ws, m, n, k, (int32_t*)y, st);
  }
}

}  // namespace qg
