// KV-cache INT8 quantization in position segments with per-channel scales.
// 「LLM推理降本五要素」 §5.2: cached keys/values are quantized in segments of
// 128 positions, each segment with its own scale per head-dim channel (scale
// buffer indexed [layer, kv head, position / 128, head dim]); a value becomes
// round(k / scale), clamped to int8.  「第4章：量化」 §1.2: symmetric scale
// s = max|x| / 127; §1.1: x_hat = x_int * s.
//
// Layout (one layer, one sequence): kv [T][H][D] token-major, the grouped
// [L/G][G][H][D] layout with G = 128 of 「现代AI加速技术全景解析」 §5.2;
// scales [H][ceil(T / 128)][D] fp32.
#include "qg_device.hpp"
#include "qg_launch.hpp"

#include <algorithm>

namespace qg {

constexpr int kKvSeg = 128;
constexpr int kKvThreads = 256;
constexpr int kKvMaxD = 256;

// 8 consecutive channels of one (position, head), as loaded: 16 bytes of
// 16-bit values or 32 bytes of binary32.  Kept raw until used, so that a
// batch of loads stays in flight.
template <int DT>
struct KvRaw {
  v4i d[DT == F32 ? 2 : 1];
};

template <int DT>
__device__ __forceinline__ void kv_f32(const KvRaw<DT>& r, float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (DT == F32) {
      v[e] = __int_as_float(r.d[0][e]);
      v[4 + e] = __int_as_float(r.d[1][e]);
    } else {
      const u32 u = (u32)r.d[0][e];
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

typedef int v2i __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Work item: one (segment, head, channel slice).  A slice is CPW chunks of 8
// channels: 8 chunks (one 128-byte line of bf16/f16 per position) when D / 8
// is a multiple of 8, else the whole head dim.  Items are numbered
// ((segment * H) + head) * slices + slice, so that the workgroups running at
// one time read neighbouring parts of the same 128 positions.
//
// A 256-thread workgroup takes items blockIdx.x, blockIdx.x + gridDim.x, ...
// and keeps two in registers: the loads of the next item are issued before
// the current one is reduced and stored, so the read and write streams
// overlap.  Every access goes through a buffer resource that spans the
// item's rows of the slice (the resource of an item past the last is empty):
// rows past the segment's end and items past the last read zeros and drop
// their stores, so no access sits under a branch and the compiler's waits
// count exactly the loads of the item being finished.
//
// Within an item, thread t owns chunk t % CPW of positions t / CPW + i * RP
// (RP = 256 / CPW positions per pass, i < KC passes; threads t >= RP * CPW
// load nothing).  Per-channel maxima meet in LDS (rows past the segment's end
// add zeros); one thread per channel forms its scale and the scale's
// reciprocal, and every thread stores its codes 8 bytes at a time.
// ---------------------------------------------------------------------------
struct KvItem {
  rsrc_t x, q, s;   // the item's cache rows, code rows and scale slice
};

template <int DT, int KC>
struct KvQuant {
  static constexpr int kEs = DT == F32 ? 4 : 2;   // bytes per cache element
  const uint8_t* kv;
  int8_t* q;
  float* scale;
  int T, H, D, S, n, cpw, nsplit, rp, cc, r0;
  // exact division by nsplit and by H for quotients below 2^31:
  // n / d = (n * mag) >> (31 + sh), mag = ceil(2^(31 + sh) / d), sh = ceil(log2 d)
  u32 smag, hmag;
  int ssh, hsh;
  int64_t row;      // elements per position (H * D)
  // per pass: byte offset of the thread's chunk from the slice's first
  // element, for the cache (xo) and the codes (qo); kOOB for threads that
  // load nothing.  The same for every item.
  u32 xo[KC], qo[KC];

  __device__ __forceinline__ void offsets() {
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      // positions from 128 on lie outside every segment; stopping there also
      // keeps e * 4 below 2^31 (row <= 2^22)
      const bool act = r0 < rp && r0 + i * rp < kKvSeg;
      const u32 e = (u32)((r0 + i * rp) * row + 8 * cc);
      xo[i] = act ? e * kEs : kOOB;
      qo[i] = act ? e : kOOB;
    }
  }

  __device__ __forceinline__ KvItem item(int it) const {
    KvItem w;
    const int sh = (int)(((uint64_t)(u32)it * smag) >> (31 + ssh)), split = it - sh * nsplit;
    const int seg = (int)(((uint64_t)(u32)sh * hmag) >> (31 + hsh)), h = sh - seg * H;
    const int c0 = 8 * cpw * split, t0 = seg * kKvSeg;
    const int tn = it < n ? min(kKvSeg, T - t0) : 0;
    const int64_t base = ((int64_t)t0 * H + h) * D + c0;
    // bytes from the slice's first element to the end of its last row
    const uint32_t span = tn > 0 ? (uint32_t)((int64_t)(tn - 1) * row + 8 * cpw) : 0u;
    w.x = make_rsrc(kv + base * kEs, span * kEs);
    w.q = make_rsrc(q + base, span);
    w.s = make_rsrc(scale + ((int64_t)h * S + seg) * D + c0, tn > 0 ? 32u * cpw : 0u);
    return w;
  }

  __device__ __forceinline__ void load(const KvItem& w, KvRaw<DT> (&v)[KC]) const {
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      v[i].d[0] = bld16(w.x, xo[i]);
      if constexpr (DT == F32) v[i].d[1] = bld16(w.x, xo[i] + 16);   // kOOB + 16: still out
    }
  }

  // Finish an item: per-channel maxima, scales and their reciprocals, codes
  // (sym_code_t: the correctly rounded quotient's integer, reached through
  // the reciprocal).  With bf16 caches about 0.3% of the values fall near a
  // tie and take the division -- quotients of 8-bit mantissas often land on
  // or near half-integers -- so the fallback is decided per value.
  __device__ __forceinline__ void process(const KvItem& w, const KvRaw<DT> (&raw)[KC],
                                          float* part, float* chs, float* chr) const {
    const int cw = 8 * cpw;
    const int tid = threadIdx.x;
    float v[KC][8];
#pragma unroll
    for (int i = 0; i < KC; ++i) kv_f32<DT>(raw[i], v[i]);
    float amax[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      amax[e] = fabsf(v[0][e]);
#pragma unroll
      for (int i = 1; i < KC; ++i) amax[e] = fmaxf(amax[e], fabsf(v[i][e]));
    }
    if (r0 < rp) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part[r0 * cw + 8 * cc + e] = amax[e];
    }
    __syncthreads();
    float sc = 0.f;
    if (tid < cw) {   // one channel per thread (cw <= 256): s = max / 127, r = 1 / s
      float a = 0.f;
      for (int r = 0; r < rp; ++r) a = fmaxf(a, part[r * cw + tid]);
      sc = a > 0.f ? a / 127.f : 0.f;
      chs[tid] = sc;
      chr[tid] = sym_code_r(a, sc);
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(sc), w.s, tid < cw ? 4u * tid : kOOB, 0,
                                          0);
    __syncthreads();
    float s[8], rc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s[e] = chs[8 * cc + e];
      rc[e] = chr[8 * cc + e];   // 0 for an all-zero channel: its codes come out 0
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      u32 c[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        c[h] = pack_code_bytes(sym_code_t(v[i][4 * h], s[4 * h], rc[4 * h]),
                               sym_code_t(v[i][4 * h + 1], s[4 * h + 1], rc[4 * h + 1]),
                               sym_code_t(v[i][4 * h + 2], s[4 * h + 2], rc[4 * h + 2]),
                               sym_code_t(v[i][4 * h + 3], s[4 * h + 3], rc[4 * h + 3]));
      // rows past the segment's end fall outside the resource: dropped
      __builtin_amdgcn_raw_buffer_store_b64(v2i{(int)c[0], (int)c[1]}, w.q, qo[i], 0, 0);
    }
  }
};

template <int DT, int KC>
__global__ __launch_bounds__(kKvThreads) void k_kv_quant_seg(const void* __restrict__ kv, int T,
                                                             int H, int D, int cpw,
                                                             int8_t* __restrict__ q,
                                                             float* __restrict__ scale,
                                                             u32 smag, int ssh, u32 hmag, int hsh) {
  __shared__ float part[kKvThreads * 8];   // [RP][8 * CPW] partial maxima (<= 2048)
  __shared__ __align__(16) float chs[kKvMaxD];   // per-channel scale of the slice
  __shared__ __align__(16) float chr[kKvMaxD];   // and its reciprocal
  KvQuant<DT, KC> k;
  k.kv = reinterpret_cast<const uint8_t*>(kv);
  k.q = q;
  k.scale = scale;
  k.T = T;
  k.H = H;
  k.D = D;
  k.S = (T + kKvSeg - 1) / kKvSeg;
  k.cpw = cpw;
  k.nsplit = (D >> 3) / cpw;
  k.smag = smag;
  k.ssh = ssh;
  k.hmag = hmag;
  k.hsh = hsh;
  k.n = k.S * H * k.nsplit;
  k.rp = kKvThreads / cpw;
  k.cc = (int)threadIdx.x % cpw;
  k.r0 = (int)threadIdx.x / cpw;
  k.row = (int64_t)H * D;
  k.offsets();
  const int G = gridDim.x;

  KvRaw<DT> va[KC], vb[KC];
  int cur = blockIdx.x;   // the launch makes gridDim.x <= the item count
  KvItem wa = k.item(cur), wb;
  k.load(wa, va);
  while (true) {
    wb = k.item(cur + G);          // empty past the last item
    k.load(wb, vb);
    k.process(wa, va, part, chs, chr);
    cur += G;
    if (cur >= k.n) break;
    wa = k.item(cur + G);
    k.load(wa, va);
    k.process(wb, vb, part, chs, chr);
    cur += G;
    if (cur >= k.n) break;
  }
}

// 8 outputs as 16 (16-bit types) or 32 (binary32) bytes
template <typename OutT>
__device__ __forceinline__ void kv_store8(OutT* p, const float (&x)[8]) {
  if constexpr (sizeof(OutT) == 4) {
    v4i a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = __float_as_int(x[e]);
      b[e] = __float_as_int(x[4 + e]);
    }
    st16(p, a);
    st16(p + 4, b);
  } else {
    v4i a;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const u32 lo = __builtin_bit_cast(uint16_t, Out<OutT>::cvt(x[2 * e]));
      const u32 hi = __builtin_bit_cast(uint16_t, Out<OutT>::cvt(x[2 * e + 1]));
      a[e] = (int)(lo | (hi << 16));
    }
    st16(p, a);
  }
}

// x_hat = code * s: the binary32 product (rounded once), then rounded to the
// output type; one thread per 8 channels of one (position, head),
// grid-stride.  FAST (fewer than 2^31 chunks): the chunk index is split into
// (position, head, channel chunk) by multiply-high divisions.
template <typename OutT, bool FAST>
__global__ __launch_bounds__(256) void k_kv_dequant_seg(const int8_t* __restrict__ q,
                                                        const float* __restrict__ scale, int T,
                                                        int H, int D, OutT* __restrict__ out,
                                                        u32 cmag, int csh, u32 hmag, int hsh) {
  const int S = (T + kKvSeg - 1) / kKvSeg, cpr = D >> 3;
  const int64_t n8 = (int64_t)T * H * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    int64_t th;
    int cc, t, hh;
    if constexpr (FAST) {
      // n8 < 2^31: exact multiply-high divisions by cpr and H
      const u32 iu = (u32)i;
      const u32 thu = (u32)(((uint64_t)iu * cmag) >> (31 + csh));
      cc = (int)(iu - thu * (u32)cpr);
      t = (int)(((uint64_t)thu * hmag) >> (31 + hsh));
      hh = (int)thu - t * H;
      th = thu;
    } else {
      th = i / cpr;
      cc = (int)(i - th * cpr);
      t = (int)(th / H);
      hh = (int)(th - (int64_t)t * H);
    }
    const uint2 c = *reinterpret_cast<const uint2*>(q + 8 * i);
    const float* sp = scale + ((int64_t)hh * S + t / kKvSeg) * D + 8 * cc;
    const v4i s0 = ld16(sp), s1 = ld16(sp + 4);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int code = (int)(int8_t)(((e < 4 ? c.x : c.y) >> (8 * (e & 3))) & 0xFFu);
      const float sv = __int_as_float(e < 4 ? s0[e] : s1[e - 4]);
      x[e] = (float)code * sv;
    }
    kv_store8<OutT>(out + 8 * i, x);
  }
}

// Exact division of n < 2^31 by d >= 1 as a multiply-high: n / d =
// (n * mag) >> (31 + sh) with sh = ceil(log2 d), mag = ceil(2^(31 + sh) / d)
// (mag * d - 2^(31 + sh) < d, so the error term stays below 1 / d).
static u32 kv_magic(int d, int& sh) {
  sh = 0;
  while ((1LL << sh) < d) ++sh;
  return (u32)((((uint64_t)1 << (31 + sh)) + (uint64_t)d - 1) / (uint64_t)d);
}

// Workgroups of the quantizer: about two items per workgroup, at most
// kKvMaxWgs (an even split over the 256 CUs).
constexpr int kKvMaxWgs = 1024;

template <int DT>
static hipError_t kv_quant_dt(const void* kv, int T, int H, int D, int8_t* q, float* s,
                              hipStream_t st) {
  const int cpr = D >> 3, cpw = cpr % 8 == 0 ? 8 : cpr;
  const int64_t items = (int64_t)((T + kKvSeg - 1) / kKvSeg) * H * (cpr / cpw);
  const unsigned grid = (unsigned)std::min<int64_t>((items + 1) / 2, kKvMaxWgs);
  // passes over the segment: ceil(128 / RP), taken up to a power of two
  const int rp = kKvThreads / cpw, need = (kKvSeg + rp - 1) / rp;
  int ssh, hsh;
  const u32 smag = kv_magic(cpr / cpw, ssh), hmag = kv_magic(H, hsh);
  if (need <= 1) k_kv_quant_seg<DT, 1><<<grid, kKvThreads, 0, st>>>(kv, T, H, D, cpw, q, s, smag, ssh, hmag, hsh);
  else if (need <= 2) k_kv_quant_seg<DT, 2><<<grid, kKvThreads, 0, st>>>(kv, T, H, D, cpw, q, s, smag, ssh, hmag, hsh);
  else if (need <= 4) k_kv_quant_seg<DT, 4><<<grid, kKvThreads, 0, st>>>(kv, T, H, D, cpw, q, s, smag, ssh, hmag, hsh);
  else if (need <= 8) k_kv_quant_seg<DT, 8><<<grid, kKvThreads, 0, st>>>(kv, T, H, D, cpw, q, s, smag, ssh, hmag, hsh);
  else k_kv_quant_seg<DT, 16><<<grid, kKvThreads, 0, st>>>(kv, T, H, D, cpw, q, s, smag, ssh, hmag, hsh);
  return hipGetLastError();
}

hipError_t launch_kv_quant_seg(const void* kv, int kv_dtype, int64_t T, int64_t H, int64_t D,
                               int8_t* kv_q, float* kv_scale, hipStream_t st) {
  const int t = (int)T, h = (int)H, d = (int)D;
  switch (kv_dtype) {
    case F32: return kv_quant_dt<F32>(kv, t, h, d, kv_q, kv_scale, st);
    case F16: return kv_quant_dt<F16>(kv, t, h, d, kv_q, kv_scale, st);
    default: return kv_quant_dt<BF16>(kv, t, h, d, kv_q, kv_scale, st);
  }
}

template <typename OutT>
static void kv_dequant_t(const int8_t* kv_q, const float* kv_scale, int T, int H, int D, OutT* out,
                         int64_t n8, hipStream_t st) {
  const unsigned grid = (unsigned)std::min<int64_t>((n8 + 255) / 256, 65536);
  int csh, hsh;
  const u32 cmag = kv_magic(D / 8, csh), hmag = kv_magic(H, hsh);
  if (n8 < ((int64_t)1 << 31))   // 32-bit chunk indices: multiply-high divisions
    k_kv_dequant_seg<OutT, true><<<grid, 256, 0, st>>>(kv_q, kv_scale, T, H, D, out, cmag, csh, hmag, hsh);
  else
    k_kv_dequant_seg<OutT, false><<<grid, 256, 0, st>>>(kv_q, kv_scale, T, H, D, out, cmag, csh, hmag, hsh);
}

hipError_t launch_kv_dequant_seg(const int8_t* kv_q, const float* kv_scale, int64_t T, int64_t H,
                                 int64_t D, void* out, int out_dtype, hipStream_t st) {
  const int64_t n8 = T * H * (D / 8);
  const int t = (int)T, h = (int)H, d = (int)D;
  switch (out_dtype) {
    case F32: kv_dequant_t<float>(kv_q, kv_scale, t, h, d, (float*)out, n8, st); break;
    case F16: kv_dequant_t<_Float16>(kv_q, kv_scale, t, h, d, (_Float16*)out, n8, st); break;
    default: kv_dequant_t<uint16_t>(kv_q, kv_scale, t, h, d, (uint16_t*)out, n8, st); break;
  }
  return hipGetLastError();
}

}  // namespace qg
