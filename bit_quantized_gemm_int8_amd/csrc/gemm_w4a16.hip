// W4A16 weight-only GEMM: 16-bit float activations x g=128 uint4 weights, the
// dequantization fused into the GEMM.
// 「第4章：量化」 §3.1 (weight-only 4-bit, activations stay 16-bit) and §3.5
// (a separate dequantize-then-GEMM pass is slower than fp16 at small batch;
// fuse it); 「Quantization & Flash Attention」 §2.2 (AWQ-folded weights).
//
// Per group g:  p[m,g,n] = sum_{k in g} x[m,k] (q[n,k] - z[n,g])  on the fp16
// (or bf16) matrix cores with binary32 accumulation, then
// y[m,n] = sum_g s[n,g] p[m,g,n] in binary32.  The operand (q - z) is an
// exact small integer; the scale multiplies the binary32 group sum, never
// the 16-bit operand, so the only roundings are those of binary32 sums.
//
// fp16 unpack: (w & 0x000F000F) | 0x64006400 is the fp16 pair
// (1024 + q_0, 1024 + q_4), and a packed fp16 add of -(1024 + z) leaves
// (q - z) exactly; the odd nibbles (w & 0x00F000F0) give 1024 + 16 q, which one
// packed fma by 1/16 and -(64 + z) takes to (q - z) exactly; w >> 8 gives the
// other four codes.  The activation halves are shuffled into the matching
// [0,4,1,5,2,6,3,7] order.
#include "qg_decode.hpp"
#include "qg_device.hpp"
#include "qg_launch.hpp"

#include <algorithm>

namespace qg {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// halves [h0..h7] of an activation fragment -> [h0 h4 h1 h5 h2 h6 h3 h7]
__device__ __forceinline__ v4i shuffle_halves(v4i x) {
  const u32 d0 = (u32)x[0], d1 = (u32)x[1], d2 = (u32)x[2], d3 = (u32)x[3];
  return v4i{(int)__builtin_amdgcn_perm(d2, d0, 0x05040100u),
             (int)__builtin_amdgcn_perm(d2, d0, 0x07060302u),
             (int)__builtin_amdgcn_perm(d3, d1, 0x05040100u),
             (int)__builtin_amdgcn_perm(d3, d1, 0x07060302u)};
}

// (x & mask) | bits in one VALU instruction (the compiler otherwise emits an
// AND and an OR).  The mask comes from an SGPR and the bits from a VGPR: a
// gfx9 VOP3 instruction reads at most one scalar operand.
__device__ __forceinline__ u32 and_or(u32 x, u32 mask, u32 bits) {
  u32 r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(bits));
  return r;
}

// The zero point z (an integer 0..15) as the two packed fp16 addends the
// unpack uses: -(1024 + z) and -(64 + z), both exact.
struct ZeroF16 {
  h2 lo, hi;
};
__device__ __forceinline__ ZeroF16 zero_f16(float zf) {
  const u32 a = f32_to_f16_bits(-(1024.f + zf)), b = f32_to_f16_bits(-(64.f + zf));
  return ZeroF16{__builtin_bit_cast(h2, a | (a << 16)), __builtin_bit_cast(h2, b | (b << 16))};
}

// 8 codes of word w -> (q - z) as fp16 halves in order [q0 q4 q1 q5 q2 q6 q3 q7]:
//   (w & 0x000F000F) | 0x64006400 = (1024 + q0, 1024 + q4), plus -(1024 + z);
//   (w & 0x00F000F0) | 0x64006400 = (1024 + 16 q1, 1024 + 16 q5), times 1/16
//       plus -(64 + z) in one packed fma;
//   the same of w >> 8 for (q2, q6) and (q3, q7).
// Every step is exact (small integers); 9 instructions per word.
__device__ __forceinline__ v4i unpack_f16(u32 w, const ZeroF16& zp) {
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const u32 w8 = w >> 8;
  const h2 d0 = __builtin_bit_cast(h2, and_or(w, 0x000F000Fu, 0x64006400u)) + zp.lo;
  const h2 d1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(w, 0x00F000F0u, 0x64006400u)),
                                          sixteenth, zp.hi);
  const h2 d2 = __builtin_bit_cast(h2, and_or(w8, 0x000F000Fu, 0x64006400u)) + zp.lo;
  const h2 d3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(w8, 0x00F000F0u, 0x64006400u)),
                                          sixteenth, zp.hi);
  return v4i{__builtin_bit_cast(int, d0), __builtin_bit_cast(int, d1), __builtin_bit_cast(int, d2),
             __builtin_bit_cast(int, d3)};
}

// bf16: (q - z) built exactly in binary32 (2^23 + q minus 2^23 + z), whose
// upper half is the bf16 value; same output order as unpack_f16.
__device__ __forceinline__ v4i unpack_bf16(u32 w, float zb /* 2^23 + z */) {
  v4i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(0x4B000000u | ((w >> (4 * i)) & 0xFu)) - zb;
    const float hi = __uint_as_float(0x4B000000u | ((w >> (4 * i + 16)) & 0xFu)) - zb;
    r[i] = (int)((__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u));
  }
  return r;
}

template <int MT, int NT, int U>
struct W4A16Batch {
  v4i wv[U][NT], xa[U][MT][4];
  uint16_t sbits[U][NT], zbits[U][NT];
};

template <int MT, int NT, int U>
__device__ __forceinline__ void w4a16_load(W4A16Batch<MT, NT, U>& bt, int g0, int ge, rsrc_t wr,
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
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 4; ++h) bt.xa[u][mt][h] = bld16(xr, gin ? xoff[mt] + 256 * g + 16 * h : kOOB);
  }
  // keep the whole batch of loads ahead of the multiplies that follow
  __builtin_amdgcn_sched_barrier(0);
}

template <int MT, int NT, int U, int XDT>
__device__ __forceinline__ void w4a16_mma(const W4A16Batch<MT, NT, U>& bt, int g0, int ge,
                                          v4f (&yacc)[MT][NT]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {   // groups >= ge hold zeros and add zero
    v4i a[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 4; ++h) a[mt][h] = shuffle_halves(bt.xa[u][mt][h]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float zf = f16_bits_to_f32(bt.zbits[u][t]);
      const float s = f16_bits_to_f32(bt.sbits[u][t]);
      v4i b[4];
      if constexpr (XDT == F16) {
        const ZeroF16 zp = zero_f16(zf);
#pragma unroll
        for (int h = 0; h < 4; ++h) b[h] = unpack_f16((u32)bt.wv[u][t][h], zp);
      } else {
        const float zb = 8388608.f + zf;
#pragma unroll
        for (int h = 0; h < 4; ++h) b[h] = unpack_bf16((u32)bt.wv[u][t][h], zb);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v4f p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if constexpr (XDT == F16)
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a[mt][h]),
                                                       __builtin_bit_cast(v8h, b[h]), p, 0, 0, 0);
          else
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[mt][h]),
                                                        __builtin_bit_cast(v8bf, b[h]), p, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) yacc[mt][t][i] = __builtin_fmaf(s, p[i], yacc[mt][t][i]);
      }
    }
  }
}

// Workgroup = WAVES waves owning 16*NT columns and 16*MT rows; groups split
// across waves, walked in double-buffered batches of U groups.  Lane l:
// row/column (l & 15); in a group it loads words 4j..4j+3 of its column
// (j = l >> 4), MFMA h (0..3) takes word 4j+h, i.e. k = 32j + 8h + 0..7.
template <int MT, int NT, int WAVES, int U, int XDT, typename OutT>
__global__ __launch_bounds__(64 * WAVES) void k_w4a16(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ wq,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero, int M, int N, int K,
    OutT* __restrict__ y) {
  __shared__ v4f red[WAVES][MT][NT][64];
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
  const rsrc_t xr = make_rsrc(x + (int64_t)m_base * K, (u32)(rows_m * K * 2));
  u32 woff[NT], soff[NT], xoff[MT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    woff[t] = (u32)(((16 * t + r) * Kw + 4 * j) * 4);
    soff[t] = (u32)((16 * t + r) * G * 2);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xoff[mt] = (u32)(((16 * mt + r) * K + 32 * j) * 2);

  v4f yacc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) yacc[mt][t] = v4f{0.f, 0.f, 0.f, 0.f};

  W4A16Batch<MT, NT, U> p0, p1;
  w4a16_load(p0, gb, ge, wr, woff, sr, zr, soff, xr, xoff);
  // Branch-free software pipeline: groups past this wave's range read zeros
  // (and add zero), so each batch waits only for its own loads.
  for (int g0 = gb; g0 < ge; g0 += 2 * U) {
    w4a16_load(p1, g0 + U, ge, wr, woff, sr, zr, soff, xr, xoff);
    w4a16_mma<MT, NT, U, XDT>(p0, g0, ge, yacc);
    w4a16_load(p0, g0 + 2 * U, ge, wr, woff, sr, zr, soff, xr, xoff);
    w4a16_mma<MT, NT, U, XDT>(p1, g0 + U, ge, yacc);
  }

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
      if (m < M) y[(int64_t)m * N + n] = Out<OutT>::cvt(sum[i]);
    }
  }
}

// Bytes of 16-bit token values that one weight unit (two g=128 groups)
// multiplies.
constexpr int kSliceUnitBytes = 2 * 128 * 2;

// A slice of the token rows into LDS, each 16-byte chunk already in the
// order of the unpacked codes: bytes col0 .. col0 + row_bytes of each of ROWS
// rows src_stride bytes apart, into rows of pitch bytes.  Chunks past the
// slice go (as zeros) into the row's padding; rows past the resource's end
// are zeros.  `after` runs once the first round of loads is issued.
template <int ROWS, int THREADS, typename A>
__device__ __forceinline__ void stage_slice_halves(int8_t* dst, int pitch, rsrc_t src,
                                                   int src_stride, int col0, int row_bytes,
                                                   A after) {
  constexpr int CPR = ROWS <= 4 ? 2 : 1;
  const int kc = row_bytes >> 4;
  v4i v[ROWS][CPR];
  auto load = [&](int c0) {
#pragma unroll
    for (int i = 0; i < CPR; ++i) {
      const int c = c0 + (int)threadIdx.x + i * THREADS;
#pragma unroll
      for (int m = 0; m < ROWS; ++m)
        v[m][i] = bld16(src, c < kc ? (u32)(m * src_stride + col0 + 16 * c) : kOOB);
    }
  };
  auto store = [&](int c0) {
#pragma unroll
    for (int i = 0; i < CPR; ++i) {
      const int c = c0 + (int)threadIdx.x + i * THREADS, cc = c < kc ? c : kc;
#pragma unroll
      for (int m = 0; m < ROWS; ++m) st16(dst + m * pitch + 16 * cc, shuffle_halves(v[m][i]));
    }
  };
  load(0);
  __builtin_amdgcn_sched_barrier(0);
  after();
  store(0);
  for (int c0 = CPR * THREADS; c0 < kc; c0 += CPR * THREADS) {
    load(c0);
    store(c0);
  }
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 16) on whole-line weight units (see qg_decode.hpp): a
// unit is two g=128 groups of 16 weight rows.  The token rows are staged whole
// in LDS, each 16-byte chunk already in the [0,4,1,5,2,6,3,7] order of the
// unpacked codes, and the rows' scales and zero points next to them; wave w
// streams its contiguous run of units in batches of UB, two batches in
// flight.  Rows r >= MR of the MFMA read token row 0 (never stored): with one
// token row every lane reads the same bytes, an LDS broadcast.
// ---------------------------------------------------------------------------
// GEN = true: the workgroup owns the 16-row blocks [bb0, bb0 + nb) given by
// its share of the grid (block blk gets waves blk, blk + nb, ..., which split
// its K); GEN = false compiles the one-block case with constant counts.
template <int MR, int WAVES, int UB, int XDT, bool GEN, typename OutT>
__global__ __launch_bounds__(64 * WAVES) void k_w4a16_dec(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ wq,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero, int M, int N, int K,
    OutT* __restrict__ y, int phases_arg) {
  constexpr int kThreads = 64 * WAVES;
  // LDS: MR token rows (pitch stage_pitch(2K)), then 16 nb x sz_pitch(G) words
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  __shared__ __attribute__((aligned(16))) int8_t tiles[WAVES][kTileBytes];
  __shared__ v4f red[WAVES][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int nblocks = (N + 15) / 16;
  const int bb0 = GEN ? (int)((int64_t)nblocks * blockIdx.x / gridDim.x) : (int)blockIdx.x;
  const int nb = GEN ? (int)((int64_t)nblocks * (blockIdx.x + 1) / gridDim.x) - bb0 : 1;
  const int blk = GEN ? wave % nb : 0, sub = GEN ? wave / nb : wave;
  const int subs = GEN ? (WAVES - blk + nb - 1) / nb : WAVES;
  const int n_base = (bb0 + blk) * 16;
  const int G = K >> 7, Kw = K >> 3, RB = Kw * 4;   // RB: packed bytes per weight row
  const int units = (RB + kUnitBytes - 1) / kUnitBytes;
  // K is walked in `phases` runs of units (one unless the token rows are too
  // long for LDS); each phase stages its slice of the token rows
  const int phases = GEN ? phases_arg : 1;
  const int xpitch =
      stage_pitch(min(2 * K, kSliceUnitBytes * ((units + phases - 1) / phases)));
  int8_t* xl = smem;
  u32* szl = reinterpret_cast<u32*>(smem + MR * xpitch);

  const int rows_n = min(16, N - n_base);
  const rsrc_t wr = make_rsrc_uniform(wq + (int64_t)n_base * Kw, (u32)(rows_n * RB));
  const UnitLanes ul = unit_lanes(lane, RB);

  v4i b0[UB][2], b1[UB][2];
  // scales and zero points, then per phase the slice of the token rows and
  // behind it the phase's first weight batch
  ScaleZeroStage<kThreads, 4> sz;
  const int srows = min(16 * nb, N - 16 * bb0);   // the workgroup's weight rows
  const rsrc_t sr = make_rsrc_uniform(wscale + (int64_t)16 * bb0 * G, (u32)(srows * G * 2));
  const rsrc_t zr = make_rsrc_uniform(wzero + (int64_t)16 * bb0 * G, (u32)(srows * G * 2));
  sz.load(sr, zr, 16 * nb * G, 0);
  const rsrc_t xr = make_rsrc(x, (u32)(M * K * 2));

  const int8_t* xrow = xl + (r < MR ? r : 0) * xpitch + 64 * j;
  const u32* szrow = szl + (16 * blk + r) * sz_pitch(G);
  int8_t* tile = tiles[wave];
  v4f yacc = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < phases; ++p) {
    const int pu0 = (int)((int64_t)units * p / phases), pu1 = (int)((int64_t)units * (p + 1) / phases);
    const int ub = pu0 + (int)((int64_t)(pu1 - pu0) * sub / subs);
    const int ue = pu0 + (int)((int64_t)(pu1 - pu0) * (sub + 1) / subs);
    const int col0 = kSliceUnitBytes * pu0, cols = min(kSliceUnitBytes * pu1, 2 * K) - col0;
    auto load = [&](v4i (&b)[UB][2], int q0) {
#pragma unroll
      for (int v = 0; v < UB; ++v) unit_load(b[v], wr, ul, q0 + v, q0 + v < ue, RB);
      __builtin_amdgcn_sched_barrier(0);
    };
    if (p > 0) __syncthreads();   // every wave is done with the previous slice
    stage_slice_halves<MR, kThreads>(xl, xpitch, xr, 2 * K, col0, cols, [&]() { load(b0, ub); });
    if (p == 0) sz.finish(sr, zr, szl, G, 16 * nb * G);
    lds_barrier();

    auto mma = [&](const v4i (&b)[UB][2], int q0) {
#pragma unroll
      for (int v = 0; v < UB; ++v) {
        v4i f[2];
        unit_transpose(tile, b[v], ul, f);
        // units past this wave's run: zero codes; their scale is taken as zero
        const bool qin = q0 + v < ue;
        const int q = qin ? q0 + v : 0;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int g = 2 * q + s;
          const u32 szw = qin && g < G ? szrow[g] : 0u;
          const float sc = f16_bits_to_f32((uint16_t)(szw & 0xFFFFu));
          const float zf = f16_bits_to_f32((uint16_t)(szw >> 16));
          v4i bw[4];
          if constexpr (XDT == F16) {
            const ZeroF16 zp = zero_f16(zf);
#pragma unroll
            for (int h = 0; h < 4; ++h) bw[h] = unpack_f16((u32)f[s][h], zp);
          } else {
            const float zb = 8388608.f + zf;
#pragma unroll
            for (int h = 0; h < 4; ++h) bw[h] = unpack_bf16((u32)f[s][h], zb);
          }
          // groups of this phase sit at 256 (g - 2 pu0) in the slice; a slot
          // past the run or past G reads the slice's start (its scale is zero)
          const int8_t* xf = xrow + (qin && g < G ? 256 * g - col0 : 0);
          v4f pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const v4i a = ld16(xf + 16 * h);
            if constexpr (XDT == F16)
              pacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                            __builtin_bit_cast(v8h, bw[h]), pacc, 0, 0, 0);
            else
              pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                             __builtin_bit_cast(v8bf, bw[h]), pacc, 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) yacc[i] = __builtin_fmaf(sc, pacc[i], yacc[i]);
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

  red[wave][lane] = yacc;
  __syncthreads();
  if (sub == 0) {   // wave blk: its block's partials, in wave order
    v4f sum = red[blk][lane];
    for (int sb = 1; sb < subs; ++sb) sum += red[blk + nb * sb][lane];
    const int n = n_base + r;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * j + i;
        if (m < M) y[(int64_t)m * N + n] = Out<OutT>::cvt(sum[i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wide decode kernel (up to 64 token rows, MT m-tiles of 16): a workgroup owns
// NB 16-row weight blocks and moves through K in phases of PU units (2 PU
// groups).  Each block has KS x MS waves: KS split a phase's units, MS split
// the m-tiles (reading the same weights), so that a SIMD holds more than one
// wave to hide the LDS and MFMA latencies; the KS partial sums meet in LDS at
// the end.  A phase's panel of token rows (16 MT rows x 256 PU halves, chunks
// already in the unpack order) is staged in LDS once for all waves (two-deep
// ring, one barrier per phase), and each unpacked weight fragment feeds the
// MFMAs of the wave's m-tiles.  Scales and zero points of the workgroup's
// rows are staged in LDS at the start.
// ---------------------------------------------------------------------------
template <int MT, int NB, int KS, int MS, int PU>
__host__ __device__ constexpr size_t w4a16_wide_static_lds() {
  return (size_t)2 * 16 * MT * (512 * PU + 16) + (size_t)NB * KS * MS * kTileBytes +
         (size_t)(KS == 1 ? 1 : NB * MS * (KS - 1)) * (MT / MS) * 64 * 16;
}

template <int MT, int NB, int KS, int MS, int PU, int XDT, typename OutT>
__global__ __launch_bounds__(64 * NB * KS * MS) void k_w4a16_wide(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ wq,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero, int M, int N, int K,
    OutT* __restrict__ y) {
  static_assert(PU % KS == 0, "every wave of a block takes the same number of units");
  static_assert(MT % MS == 0, "every wave of a block takes the same number of m-tiles");
  constexpr int UPW = PU / KS, MTW = MT / MS;                       // units, m-tiles per wave
  constexpr int MR = 16 * MT, PB = 512 * PU, kThreads = 64 * NB * KS * MS;   // PB: panel bytes per row
  constexpr int kPitch = PB + 16;                                   // odd number of 16-byte chunks
  constexpr int kRowChunks = PB / 16, kChunks = MR * kRowChunks;
  constexpr int CPT = (kChunks + kThreads - 1) / kThreads;
  constexpr bool kFull = CPT * kThreads == kChunks;
  extern __shared__ __attribute__((aligned(16))) u32 szl[];          // 16 NB x sz_pitch(G) words
  __shared__ __attribute__((aligned(16))) int8_t xbuf[2][MR * kPitch];
  __shared__ __attribute__((aligned(16))) int8_t tiles[NB * KS * MS][kTileBytes];
  __shared__ v4f red[KS == 1 ? 1 : NB * MS * (KS - 1)][MTW][64];
  static_assert(sizeof(xbuf) + sizeof(tiles) + sizeof(red) == w4a16_wide_static_lds<MT, NB, KS, MS, PU>(),
                "static LDS bookkeeping");
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
  const rsrc_t xr = make_rsrc(x, (u32)(M * K * 2));
  const UnitLanes ul = unit_lanes(lane, RB);

  struct Batch {
    v4i w[UPW][2], x[CPT];
  };
  auto load = [&](Batch& bt, int p) {
#pragma unroll
    for (int v = 0; v < UPW; ++v) unit_load(bt.w[v], wr, ul, p * PU + ks * UPW + v, true, RB);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + c * kThreads;
      const int row = chunk / kRowChunks, kb = p * PB + (chunk % kRowChunks) * 16;
      bt.x[c] = bld16(xr, kb < 2 * K ? (u32)(row * 2 * K + kb) : kOOB);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // scales and zero points of the workgroup's 16 NB rows, with the first
  // weight batch issued behind their loads
  const int wg_rows = max(0, min(16 * NB, N - wg_row0));
  const rsrc_t sr = make_rsrc_uniform(wscale + (int64_t)min(wg_row0, N - 1) * G, (u32)(wg_rows * G * 2));
  const rsrc_t zr = make_rsrc_uniform(wzero + (int64_t)min(wg_row0, N - 1) * G, (u32)(wg_rows * G * 2));
  ScaleZeroStage<kThreads, 4> sz;
  sz.load(sr, zr, 16 * NB * G, 0);
  __builtin_amdgcn_sched_barrier(0);
  Batch b0, b1;
  load(b0, 0);
  sz.finish(sr, zr, szl, G, 16 * NB * G);

  const u32* szrow = szl + (blk * 16 + r) * sz_pitch(G);
  int8_t* tile = tiles[wave];
  v4f yacc[MTW];
#pragma unroll
  for (int mw = 0; mw < MTW; ++mw) yacc[mw] = v4f{0.f, 0.f, 0.f, 0.f};
  auto process = [&](const Batch& bt, int p) {
    int8_t* buf = xbuf[p & 1];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + c * kThreads;
      if (kFull || chunk < kChunks)
        st16(buf + (chunk / kRowChunks) * kPitch + (chunk % kRowChunks) * 16, shuffle_halves(bt.x[c]));
    }
    // Panel p (and, at p = 0, the scales) complete once every wave is here;
    // the buffer phase p + 1 overwrites was last read at phase p - 1.
    lds_barrier();
#pragma unroll
    for (int v = 0; v < UPW; ++v) {
      v4i f[2];
      unit_transpose(tile, bt.w[v], ul, f);
      const int u = ks * UPW + v;   // unit within the phase
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int g = 2 * (p * PU + u) + s2;
        const u32 szw = g < G ? szrow[g] : 0u;     // past G: zero codes and scale
        const float zf = f16_bits_to_f32((uint16_t)(szw >> 16));
        v4i bw[4];
        if constexpr (XDT == F16) {
          const ZeroF16 zp = zero_f16(zf);
#pragma unroll
          for (int h = 0; h < 4; ++h) bw[h] = unpack_f16((u32)f[s2][h], zp);
        } else {
          const float zb = 8388608.f + zf;
#pragma unroll
          for (int h = 0; h < 4; ++h) bw[h] = unpack_bf16((u32)f[s2][h], zb);
        }
        const float sc = f16_bits_to_f32((uint16_t)(szw & 0xFFFFu));
        const int kin = 512 * u + 256 * s2 + 64 * j;
#pragma unroll
        for (int mw = 0; mw < MTW; ++mw) {
          const int8_t* xf = buf + (16 * (ms * MTW + mw) + r) * kPitch + kin;
          v4f pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const v4i a = ld16(xf + 16 * h);
            if constexpr (XDT == F16)
              pacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                            __builtin_bit_cast(v8h, bw[h]), pacc, 0, 0, 0);
            else
              pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                             __builtin_bit_cast(v8bf, bw[h]), pacc, 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) yacc[mw][i] = __builtin_fmaf(sc, pacc[i], yacc[mw][i]);
        }
      }
    }
  };
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
        for (int i = 0; i < 4; ++i) yacc[mw][i] += t[i];
      }
  }
  const int n = n_base + r;
  if (n < N) {
#pragma unroll
    for (int mw = 0; mw < MTW; ++mw)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * (ms * MTW + mw) + 4 * j + i;
        if (m < M) y[(int64_t)m * N + n] = Out<OutT>::cvt(yacc[mw][i]);
      }
  }
}

template <int MT, int NB, int KS, int MS, int PU, int XDT, typename OutT>
static bool launch_w4a16_wide_nb(const uint16_t* x, const int32_t* wq, const uint16_t* ws,
                                 const uint16_t* wz, int M, int N, int K, OutT* y, size_t lds,
                                 hipStream_t st) {
  if (w4a16_wide_static_lds<MT, NB, KS, MS, PU>() + lds > kLdsBytesPerCU) return false;
  const int nblocks = (N + 15) / 16;
  const dim3 grid((unsigned)((nblocks + NB - 1) / NB)), block(64 * NB * KS * MS);
  k_w4a16_wide<MT, NB, KS, MS, PU, XDT, OutT><<<grid, block, lds, st>>>(x, wq, ws, wz, M, N, K, y);
  return true;
}

// Waves per weight block (K split KS ways, m-tiles MS ways), measured on
// MI355X (K = 4096 and 11008; N = 4096, 12288, 14336): 2 (4 with one block per
// workgroup, narrow layers), or the m-tiles split where the K split would need
// too much LDS (PU = KS units of token rows per phase).  K = 4096, N = 12288:
// 17-32 rows 17.2 -> 12.2 us, 64 rows 25.6 -> 22.0; 16 rows on N = 14336
// 13.0 -> 10.2.
template <int MT, int NB>
struct W16Split {
  static constexpr int KS = MT == 1 ? (NB == 1 ? 4 : 2) : MT <= 3 ? 2 : 1;
  static constexpr int MS = MT == 2 ? (NB == 1 ? 2 : 1) : MT == 3 ? 1 : MT == 4 ? (NB == 1 ? 4 : 2) : 1;
  static constexpr int PU = KS > 1 ? KS : (MT == 1 ? 2 : 1);
};

template <int MT, int NB, int XDT, typename OutT>
static bool launch_w4a16_wide_split(const uint16_t* x, const int32_t* wq, const uint16_t* ws,
                                    const uint16_t* wz, int M, int N, int K, OutT* y, size_t lds,
                                    hipStream_t st) {
  using S = W16Split<MT, NB>;
  return launch_w4a16_wide_nb<MT, NB, S::KS, S::MS, S::PU, XDT, OutT>(x, wq, ws, wz, M, N, K, y, lds, st);
}

template <int MT, int XDT, typename OutT>
static bool launch_w4a16_wide(const uint16_t* x, const int32_t* wq, const uint16_t* ws,
                              const uint16_t* wz, int M, int N, int K, OutT* y, size_t lds,
                              hipStream_t st) {
  switch (wide_waves(N)) {
    case 1: return launch_w4a16_wide_split<MT, 1, XDT, OutT>(x, wq, ws, wz, M, N, K, y, lds, st);
    case 2: return launch_w4a16_wide_split<MT, 2, XDT, OutT>(x, wq, ws, wz, M, N, K, y, lds, st);
    case 3: return launch_w4a16_wide_split<MT, 3, XDT, OutT>(x, wq, ws, wz, M, N, K, y, lds, st);
    default: return launch_w4a16_wide_split<MT, 4, XDT, OutT>(x, wq, ws, wz, M, N, K, y, lds, st);
  }
}

// ---------------------------------------------------------------------------
// One fp16 token row (M = 1): a matrix-vector product, where a 16x16 MFMA
// would spend 15 of its 16 rows on padding.  It runs on the vector ALU.
//
// Lane l of a wave covers bytes 16 l .. 16 l + 15 of every kilobyte c of a
// weight row: codes k = 2048 c + 32 l + [0, 32), a quarter of group
// g = 16 c + l / 4.  The lane keeps the matching 32 activations of every c
// in registers, shuffled once into the unpack order.  A wave owns R
// consecutive weight rows and issues all its R x C one-kilobyte weight loads
// (whole cache lines) before the first multiply; no LDS, no barrier.
//
// Per packed word of 8 codes (nibble j = code j):
//   (w & 0x000F000F) | 0x64006400 = fp16 (1024 + q0, 1024 + q4), plus the
//       pair -(1024 + z): (q0 - z, q4 - z);
//   (w & 0x00F000F0) | 0x64006400 = (1024 + 16 q1, 1024 + 16 q5), times 1/16
//       plus -(64 + z) in one packed fma: (q1 - z, q5 - z);
//   the same of w >> 8 for codes (2, 6) and (3, 7).
// Every fp16 result is an exact small integer; v_dot2_f32_f16 adds
// x_a (q_a - z) + x_b (q_b - z) into a binary32 sum.  The four lanes of a
// group add their sums (DPP), the group sum is scaled by s in binary32 (as in
// the matrix-core kernels), and the lanes' totals are summed over the wave at
// the end.
// ---------------------------------------------------------------------------
constexpr int kGemvWaves = 4;

template <int CTRL>
__device__ __forceinline__ float mov_dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int R, int C, typename OutT>
__global__ __launch_bounds__(64 * kGemvWaves) void k_w4a16_gemv(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ wq,
    const uint16_t* __restrict__ wscale, const uint16_t* __restrict__ wzero, int N, int K,
    OutT* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x * kGemvWaves + wave) * R;
  if (n0 >= N) return;   // wave-uniform
  const int G = K >> 7, RB = K >> 1;   // groups and packed bytes per weight row
  const int rows = min(R, N - n0);
  const rsrc_t wr = make_rsrc_uniform(wq + (int64_t)n0 * (K >> 3), (u32)(rows * RB));
  const rsrc_t sr = make_rsrc_uniform(wscale + (int64_t)n0 * G, (u32)(rows * G * 2));
  const rsrc_t zr = make_rsrc_uniform(wzero + (int64_t)n0 * G, (u32)(rows * G * 2));
  const rsrc_t xr = make_rsrc_uniform(x, (u32)(K * 2));

  // Activations first (L2 hits, needed by the first multiply), then the
  // scales and zero points, then the weight stream in the order it is used.
  // Pieces past the row end read as zeros: x through its resource's range,
  // weights, scales and zero points through kOOB (their resources span the
  // wave's rows).
  v4i xv[C][4];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[c][i] = bld16(xr, (u32)(4096 * c + 64 * lane + 16 * i));
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

#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[c][i] = shuffle_halves(xv[c][i]);

  float yacc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    yacc[r] = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const ZeroF16 zp = zero_f16(f16_bits_to_f32(zb[r][c]));
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4i d = unpack_f16((u32)wv[r][c][i], zp);
        // (vector components pass through int: this compiler's bit_cast of
        // a component expression reads component 0 whatever the index)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          p0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, (int)xv[c][i][e]),
                                      __builtin_bit_cast(h2, (int)d[e]), p0, false);
          p1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, (int)xv[c][i][e + 1]),
                                      __builtin_bit_cast(h2, (int)d[e + 1]), p1, false);
        }
      }
      // the group's sum over its four lanes, identical in all four
      float p = p0 + p1;
      p += mov_dpp_f<0xB1>(p);   // quad_perm [1,0,3,2]
      p += mov_dpp_f<0x4E>(p);   // quad_perm [2,3,0,1]
      yacc[r] = __builtin_fmaf(f16_bits_to_f32(sb[r][c]), p, yacc[r]);
    }
  }

  // Sum over the 16 quads: rotations by 4 and 8 within each row of 16 lanes,
  // then the four rows.  Lane r stores weight row r's output.
  float mine = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float v = yacc[r];
    v += mov_dpp_f<0x124>(v);   // row_ror:4
    v += mov_dpp_f<0x128>(v);   // row_ror:8
    const float t = (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
    mine = lane == r ? t : mine;
  }
  if (lane < rows) y[n0 + lane] = Out<OutT>::cvt(mine);
}

template <int R, int C, typename OutT>
static void launch_w4a16_gemv_rc(const uint16_t* x, const int32_t* wq, const uint16_t* ws,
                                 const uint16_t* wz, int N, int K, OutT* y, hipStream_t st) {
  const int waves = (N + R - 1) / R;
  const dim3 grid((unsigned)((waves + kGemvWaves - 1) / kGemvWaves)), block(64 * kGemvWaves);
  k_w4a16_gemv<R, C, OutT><<<grid, block, 0, st>>>(x, wq, ws, wz, N, K, y);
}

// Weight rows of at most 2 KB (K <= 4096), where it measured faster than the
// matrix-core decode kernel on MI355X (A/B, graphs of 200 calls, weights
// rotated through 600 MB; us, this kernel / decode kernel): K = 4096 with
// N = 12288 7.73-7.84 / 7.82-8.13, N = 11008 6.81-6.86 / 7.18-7.60,
// N = 4096 4.14-4.15 / 4.49-4.52.  Longer rows lose: the dequantizing VALU
// work (13 instructions per 8 codes, against 11 with the matrix cores) no
// longer hides under the stream (K = 11008, N = 4096: 10.2 / 8.1; K = 8192,
// N = 28672: 26.8 / 25.0).  Four rows per wave (eight 1 KB loads in flight)
// at 2 KB per row, eight at 1 KB.
template <typename OutT>
static bool launch_w4a16_gemv(const uint16_t* x, const int32_t* wq, const uint16_t* ws,
                              const uint16_t* wz, int N, int K, OutT* y, hipStream_t st) {
  if (K > 2048) {
    if (K > 4096) return false;
    launch_w4a16_gemv_rc<4, 2, OutT>(x, wq, ws, wz, N, K, y, st);
  } else {
    launch_w4a16_gemv_rc<8, 1, OutT>(x, wq, ws, wz, N, K, y, st);
  }
  return true;
}

template <int WAVES, bool GEN, int XDT, typename OutT>
static void dec_w4a16_mr(int mr, const uint16_t* x, const int32_t* wq, const uint16_t* ws,
                         const uint16_t* wz, int M, int N, int K, OutT* y, size_t lds, int groups,
                         int phases, hipStream_t st) {
  constexpr int UB = 1;  // measured on MI355X
  const dim3 grid((unsigned)groups), block(64 * WAVES);
  switch (mr) {
    case 1: k_w4a16_dec<1, WAVES, UB, XDT, GEN, OutT><<<grid, block, lds, st>>>(x, wq, ws, wz, M, N, K, y, phases); break;
    case 2: k_w4a16_dec<2, WAVES, UB, XDT, GEN, OutT><<<grid, block, lds, st>>>(x, wq, ws, wz, M, N, K, y, phases); break;
    case 4: k_w4a16_dec<4, WAVES, UB, XDT, GEN, OutT><<<grid, block, lds, st>>>(x, wq, ws, wz, M, N, K, y, phases); break;
    case 8: k_w4a16_dec<8, WAVES, UB, XDT, GEN, OutT><<<grid, block, lds, st>>>(x, wq, ws, wz, M, N, K, y, phases); break;
    default: k_w4a16_dec<16, WAVES, UB, XDT, GEN, OutT><<<grid, block, lds, st>>>(x, wq, ws, wz, M, N, K, y, phases); break;
  }
}

// Compute units of an MI355X.
constexpr int kW16CUs = 256;

template <int XDT, typename OutT>
static hipError_t gemm_w4a16_t(const uint16_t* x, const int32_t* wq, const uint16_t* ws,
                               const uint16_t* wz, int M, int N, int K, OutT* y, hipStream_t st) {
  const int G = K / 128;
  if constexpr (XDT == F16) {
    if (M == 1 && launch_w4a16_gemv<OutT>(x, wq, ws, wz, N, K, y, st)) return hipGetLastError();
  }
  const int mr = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  const size_t lds = (size_t)mr * stage_pitch(2 * K) + (size_t)16 * sz_pitch(G) * 4;
  if (M <= 8 && lds <= kDecLdsMaxBytes) {
    const int nblocks = (N + 15) / 16;
    // one-block workgroups of 4 waves that fit a CU (LDS; at most 7 by registers)
    const size_t wg_lds = lds + 4 * (kTileBytes + 64 * sizeof(v4f));
    const int per_cu = (int)std::min<size_t>(7, kLdsBytesPerCU / wg_lds);
    const size_t lds_multi = (size_t)mr * stage_pitch(2 * K) + (size_t)64 * sz_pitch(G) * 4;
    if (nblocks > per_cu * kW16CUs && nblocks <= 4 * kW16CUs && lds_multi <= kDecLdsMaxBytes) {
      // more blocks than one-block workgroups can be resident at once: one
      // workgroup of 12 waves per CU over 3-4 blocks, the token rows staged
      // once (measured on MI355X: M = 8, K = 4096, N = 12288)
      dec_w4a16_mr<12, true, XDT, OutT>(mr, x, wq, ws, wz, M, N, K, y, lds_multi, kW16CUs, 1, st);
    } else if (nblocks <= 384) {
      // 8 waves split K when few 16-row blocks would leave the chip short of
      // loads in flight (measured on MI355X: K = 11008, N = 4096 takes 8.6 us
      // with 8 waves, 10.4 us with 4; N >= 11008 is best with 4)
      dec_w4a16_mr<8, false, XDT, OutT>(mr, x, wq, ws, wz, M, N, K, y, lds, nblocks, 1, st);
    } else {
      dec_w4a16_mr<4, false, XDT, OutT>(mr, x, wq, ws, wz, M, N, K, y, lds, nblocks, 1, st);
    }
    return hipGetLastError();
  }
  if (M <= 8) {
    // token rows too long for LDS at once: the decode kernel walks K in
    // phases, each staging its slice of the token rows (measured on MI355X,
    // K = 11008, N = 4096, 4 rows: 11.7 us against 14.1 with the wide kernel)
    const int nblocks = (N + 15) / 16;
    const int units = (K / 2 + kUnitBytes - 1) / kUnitBytes;
    auto tok_lds = [&](int ph) {
      return (size_t)mr * stage_pitch(std::min(2 * K, kSliceUnitBytes * ((units + ph - 1) / ph)));
    };
    const size_t sz16 = (size_t)16 * sz_pitch(G) * 4;
    int phases = 1;
    while (phases < units && tok_lds(phases) + sz16 > kDecLdsMaxBytes) ++phases;
    if (tok_lds(phases) + sz16 <= kDecLdsMaxBytes) {
      if (nblocks <= 384)
        dec_w4a16_mr<8, true, XDT, OutT>(mr, x, wq, ws, wz, M, N, K, y, tok_lds(phases) + sz16, nblocks, phases, st);
      else
        dec_w4a16_mr<4, true, XDT, OutT>(mr, x, wq, ws, wz, M, N, K, y, tok_lds(phases) + sz16, nblocks, phases, st);
      return hipGetLastError();
    }
  }
  const size_t lds_wide = (size_t)16 * wide_waves(N) * sz_pitch(G) * 4;
  if (M <= 64 && lds_wide <= kDecLdsMaxBytes) {
    bool done;
    if (M <= 16) done = launch_w4a16_wide<1, XDT, OutT>(x, wq, ws, wz, M, N, K, y, lds_wide, st);
    else if (M <= 32) done = launch_w4a16_wide<2, XDT, OutT>(x, wq, ws, wz, M, N, K, y, lds_wide, st);
    else if (M <= 48) done = launch_w4a16_wide<3, XDT, OutT>(x, wq, ws, wz, M, N, K, y, lds_wide, st);
    else done = launch_w4a16_wide<4, XDT, OutT>(x, wq, ws, wz, M, N, K, y, lds_wide, st);
    if (done) return hipGetLastError();
  }
  constexpr int MT = 1, NT = 1, WAVES = 8, U = 2;  // measured on MI355X
  dim3 grid((unsigned)((N + 16 * NT - 1) / (16 * NT)), (unsigned)((M + 16 * MT - 1) / (16 * MT)));
  k_w4a16<MT, NT, WAVES, U, XDT, OutT><<<grid, dim3(64 * WAVES), 0, st>>>(x, wq, ws, wz, M, N, K, y);
  return hipGetLastError();
}

template <int XDT>
static hipError_t gemm_w4a16_x(const uint16_t* x, const int32_t* wq, const uint16_t* ws,
                               const uint16_t* wz, int M, int N, int K, void* y, int y_dtype,
                               hipStream_t st) {
  switch (y_dtype) {
    case F32: return gemm_w4a16_t<XDT, float>(x, wq, ws, wz, M, N, K, (float*)y, st);
    case BF16: return gemm_w4a16_t<XDT, uint16_t>(x, wq, ws, wz, M, N, K, (uint16_t*)y, st);
    default: return gemm_w4a16_t<XDT, _Float16>(x, wq, ws, wz, M, N, K, (_Float16*)y, st);
  }
}

hipError_t launch_gemm_w4a16(const void* x, int x_dtype, const int32_t* wq, const uint16_t* ws,
                             const uint16_t* wz, int64_t M, int64_t N, int64_t K, void* y,
                             int y_dtype, hipStream_t st) {
  const uint16_t* xh = reinterpret_cast<const uint16_t*>(x);
  if (x_dtype == F16) return gemm_w4a16_x<F16>(xh, wq, ws, wz, (int)M, (int)N, (int)K, y, y_dtype, st);
  return gemm_w4a16_x<BF16>(xh, wq, ws, wz, (int)M, (int)N, (int)K, y, y_dtype, st);
}

}  // namespace qg
