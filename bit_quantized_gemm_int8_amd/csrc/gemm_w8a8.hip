// W8A8 GEMM: acc[m,n] = sum_k xq[m,k] wq[n,k] (int8 x int8 -> exact int32 on the
// int8 matrix cores), y[m,n] = (acc * s_x[m]) * s_w[n].
// 「第4章：量化」 §2.3 (W8A8: the GEMM runs on int8 units), §1.1 (x_hat = x_int s);
// 「LLM推理降本五要素」 §2.1 (at decode the layer waits on weight bandwidth).
//
// Two kernels:
//  * small M (decode, M <= 64): the weight stream is the whole cost.  Every
//    weight byte is used by at most 64 rows once, so weights go straight from
//    HBM into MFMA operand registers (16-byte streaming loads, many in flight
//    per lane); the K loop is split across the waves of a workgroup and the
//    int32 partials meet in LDS (exact, order-free).
//  * large M (prefill): 256x256 output tiles, K in 64-byte steps staged in LDS
//    (double-buffered, XOR-swizzled 16-byte chunks), 4 waves each owning a
//    128x128 sub-tile of 32x32x32 int8 MFMAs.
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
// Small-M kernel.  Workgroup = WAVES waves; it owns 16*NT output columns and
// 16*MT rows.  Lane l of a wave feeds MFMA row/column (l & 15) and the 16-byte
// k-slice (l >> 4) of each 64-deep step, from memory in the same order for
// both operands, so the int8 products pair up whatever order the matrix core
// sums them in.
// ---------------------------------------------------------------------------
template <int MT, int NT, int WAVES, int U, typename OutT>
__global__ __launch_bounds__(64 * WAVES) void k_w8a8_small_m(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, const int8_t* __restrict__ wq,
    const float* __restrict__ ws, int M, int N, int K, OutT* __restrict__ y) {
  __shared__ v4i red[WAVES][MT][NT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kq = (lane >> 4) * 16;
  const int n_base = blockIdx.x * 16 * NT;
  const int m_base = blockIdx.y * 16 * MT;
  const int steps = (K + 63) >> 6;
  const int sb = (int)((int64_t)steps * wave / WAVES);
  const int se = (int)((int64_t)steps * (wave + 1) / WAVES);

  const int8_t* wrow[NT];
  bool nok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n_base + 16 * t + r;
    nok[t] = n < N;
    wrow[t] = wq + (int64_t)(nok[t] ? n : 0) * K + kq;
  }
  const int8_t* xrow[MT];
  bool mok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m_base + 16 * mt + r;
    mok[mt] = m < M;
    xrow[mt] = xq + (int64_t)(mok[mt] ? m : 0) * K + kq;
  }

  v4i acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = v4i{0, 0, 0, 0};

  for (int s0 = sb; s0 < se; s0 += U) {
    v4i b[U][NT], a[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s0 + u) * 64;
      const bool kin = (s0 + u < se) && (k + kq < K);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        b[u][t] = (kin && nok[t]) ? ld16_stream(wrow[t] + k) : v4i{0, 0, 0, 0};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        a[u][mt] = (kin && mok[mt]) ? ld16(xrow[mt] + k) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[mt][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][mt], b[u][t], acc[mt][t], 0, 0, 0);
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][mt][t][lane] = acc[mt][t];
  __syncthreads();

  // 16x16 accumulator layout: lane l holds column (l & 15), rows 4*(l >> 4) + i.
  for (int it = threadIdx.x; it < MT * NT * 64; it += 64 * WAVES) {
    const int l = it & 63, t = (it >> 6) % NT, mt = (it >> 6) / NT;
    v4i sum = red[0][mt][t][l];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[w][mt][t][l];
    const int n = n_base + 16 * t + (l & 15);
    if (n >= N) continue;
    const float sw = ws ? ws[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m_base + 16 * mt + 4 * (l >> 4) + i;
      if (m < M) y[(int64_t)m * N + n] = w8a8_epilogue<OutT>(sum[i], xs ? xs[m] : 0.f, sw);
    }
  }
}

// ---------------------------------------------------------------------------
// Large-M kernel: 256x256x64 tiles, 4 waves (2x2), 32x32x32 int8 MFMAs.
// LDS holds, per stage, the A tile [256 rows][64 k] then the B tile; row r's
// 16-byte chunk c sits at r*64 + 16*(c ^ ((r >> 1) & 3)) so that the eight
// rows a group of lanes reads at once land in eight different bank groups.
// ---------------------------------------------------------------------------
constexpr int TBM = 256, TBN = 256, TBK = 64;

__device__ __forceinline__ int swz(int row, int ch) { return row * TBK + ((ch ^ ((row >> 1) & 3)) << 4); }

template <typename OutT>
__global__ __launch_bounds__(256) void k_w8a8_tiled(const int8_t* __restrict__ xq,
                                                    const float* __restrict__ xs,
                                                    const int8_t* __restrict__ wq,
                                                    const float* __restrict__ ws, int M, int N,
                                                    int K, OutT* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) int8_t smem[2][(TBM + TBN) * TBK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

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
    if (idx < per + (xcd < rem ? 1 : 0))
      bid = xcd * per + (xcd < rem ? xcd : rem) + idx;
  }
  constexpr int GROUP = 4;
  const int group = bid / (GROUP * tiles_n);
  const int first_m = group * GROUP;
  const int gsize = (tiles_m - first_m) < GROUP ? (tiles_m - first_m) : GROUP;
  const int tm = first_m + (bid % (GROUP * tiles_n)) % gsize;
  const int tn = (bid % (GROUP * tiles_n)) / gsize;
  const int m0 = tm * TBM, n0 = tn * TBN;

  v4i ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 2, k = k0 + (c & 3) * 16;
      const int m = m0 + row, n = n0 + row;
      ra[i] = (m < M && k < K) ? ld16(xq + (int64_t)m * K + k) : v4i{0, 0, 0, 0};
      rb[i] = (n < N && k < K) ? ld16(wq + (int64_t)n * K + k) : v4i{0, 0, 0, 0};
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 2, off = swz(row, c & 3);
      *reinterpret_cast<v4i*>(&smem[buf][off]) = ra[i];
      *reinterpret_cast<v4i*>(&smem[buf][TBM * TBK + off]) = rb[i];
    }
  };

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};

  const int nk = (K + TBK - 1) / TBK;
  gload(0);
  swrite(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * TBK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 2 + (lane >> 5);
      v4i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const v4i*>(&smem[buf][swz(row, ch)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 128 + j * 32 + (lane & 31);
        bf[j] = *reinterpret_cast<const v4i*>(&smem[buf][TBM * TBK + swz(row, ch)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) swrite(buf ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane l holds column (l & 31); register e holds
  // row 8*(e >> 2) + 4*(l >> 5) + (e & 3).
  const int col_in = lane & 31, rsub = 4 * (lane >> 5);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 128 + j * 32 + col_in;
    if (n >= N) continue;
    const float sw = ws ? ws[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + rsub + (e & 3);
        if (m < M) y[(int64_t)m * N + n] = w8a8_epilogue<OutT>(acc[i][j][e], xs ? xs[m] : 0.f, sw);
      }
    }
  }
}

template <typename OutT>
static hipError_t gemm_w8a8_t(const int8_t* xq, const float* xs, const int8_t* wq,
                              const float* ws, int M, int N, int K, OutT* y, hipStream_t st) {
  if (M <= 64) {
    constexpr int WAVES = 8, NT = 1, U = 4;
    dim3 block(64 * WAVES);
    const unsigned gx = (unsigned)((N + 16 * NT - 1) / (16 * NT));
    if (M <= 16)
      k_w8a8_small_m<1, NT, WAVES, U, OutT><<<dim3(gx, 1), block, 0, st>>>(xq, xs, wq, ws, M, N, K, y);
    else if (M <= 32)
      k_w8a8_small_m<2, NT, WAVES, U, OutT><<<dim3(gx, 1), block, 0, st>>>(xq, xs, wq, ws, M, N, K, y);
    else
      k_w8a8_small_m<4, NT, WAVES, U, OutT><<<dim3(gx, 1), block, 0, st>>>(xq, xs, wq, ws, M, N, K, y);
  } else {
    const int tiles = ((M + TBM - 1) / TBM) * ((N + TBN - 1) / TBN);
    k_w8a8_tiled<OutT><<<dim3((unsigned)tiles), dim3(256), 0, st>>>(xq, xs, wq, ws, M, N, K, y);
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
