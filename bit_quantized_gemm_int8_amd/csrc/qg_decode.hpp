// Building blocks of the decode-shaped (M <= 16) GEMM kernels.
//
// At decode the layer is a stream of weight bytes, each used by at most 16
// token rows, so the kernels are shaped around reading the weights at full
// HBM efficiency.  A workgroup owns 16 weight rows (16 output columns) and the
// whole K.  The rows are read in units of 128 bytes per row (one cache line):
// two MFMA steps of int8 codes, or two g=128 groups of packed uint4 codes.
//
// Whole-line loads.  An MFMA operand wants lane l to hold row l & 15, so a
// direct fragment load touches 16 rows x 64 bytes -- half lines -- and
// measured 25-50% slower on MI355X than loads whose lanes cover whole 128-byte
// lines.  A unit is therefore fetched as two loads of 8 rows x 128 bytes
// (lane l: row 8h + (l >> 3), 16-byte chunk l & 7) and turned into MFMA
// fragments through a 2 KB wave-private LDS tile: written with the lane's
// chunk at an XOR-swizzled slot, read back as fragment s = chunk 4s + (l >> 4)
// of row l & 15.  Both directions are free of LDS bank conflicts (64 banks x
// 4 bytes): a write covers rows 2i, 2i+1 with all 16 chunk slots, a read the
// 16 rows of one chunk at 16 different slots.
//
// Work split.  The waves of a workgroup split the units into contiguous
// runs: a wave streaming its own stretch of every row measured faster than
// waves interleaving units of a shared stretch (DRAM page locality).
#pragma once

#include "qg_device.hpp"

namespace qg {

constexpr int kUnitBytes = 128;   // per weight row
constexpr int kTileBytes = 16 * kUnitBytes;
// Largest dynamic LDS a decode launch stages (token rows, scales): 80 KB, so
// that two workgroups still share the 160 KB of a CU.
constexpr size_t kDecLdsMaxBytes = 80 * 1024;
constexpr size_t kLdsBytesPerCU = 160 * 1024;   // LDS of one CDNA4 compute unit

__device__ __forceinline__ int unit_slot(int row, int chunk) {
  return row * kUnitBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Per-lane constants of the unit fetch and transpose.
struct UnitLanes {
  u32 goff[2];    // byte offset of the lane's chunk of unit 0 (load h) in the 16-row block
  int wslot[2];   // LDS slot the lane writes (load h)
  int rslot[2];   // LDS slot of the lane's fragment s
  int kchunk;     // byte offset of the lane's chunk within a unit
};

__device__ __forceinline__ UnitLanes unit_lanes(int lane, int row_bytes) {
  UnitLanes u;
  const int ch = lane & 7;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * h + (lane >> 3);
    u.goff[h] = (u32)(row * row_bytes + 16 * ch);
    u.wslot[h] = unit_slot(row, ch);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) u.rslot[s] = unit_slot(lane & 15, 4 * s + (lane >> 4));
  u.kchunk = 16 * ch;
  return u;
}

// Issue the two whole-line loads of unit q (bytes 128q .. 128q + 127 of each
// row) if `valid`.  Chunks past the row end, rows past the buffer resource's
// end and invalid units read zeros.
__device__ __forceinline__ void unit_load(v4i (&d)[2], rsrc_t wr, const UnitLanes& ul, int q,
                                          bool valid, int row_bytes) {
  const bool in = valid && kUnitBytes * q + ul.kchunk < row_bytes;
  const u32 o = (u32)(kUnitBytes * q);
  d[0] = bld16_nt(wr, in ? ul.goff[0] + o : kOOB);
  d[1] = bld16_nt(wr, in ? ul.goff[1] + o : kOOB);
}

// Write a fetched unit into the wave's tile and read back its two MFMA
// fragments.  One wave's LDS accesses execute in issue order, so the reads
// see the writes and the next unit's writes follow these reads; the asm
// statement keeps the compiler from reordering them.
__device__ __forceinline__ void unit_transpose(int8_t* tile, const v4i (&d)[2], const UnitLanes& ul,
                                               v4i (&f)[2]) {
  st16(tile + ul.wslot[0], d[0]);
  st16(tile + ul.wslot[1], d[1]);
  asm volatile("" ::: "memory");
  f[0] = ld16(tile + ul.rslot[0]);
  f[1] = ld16(tile + ul.rslot[1]);
  asm volatile("" ::: "memory");
}

// Row pitch (bytes) of token rows staged whole in LDS: an odd number of
// 16-byte chunks, so the 16 rows of a fragment read hit 16 different bank
// groups.
__host__ __device__ constexpr int stage_pitch(int row_bytes) {
  return ((row_bytes >> 4) & 1) ? row_bytes + 32 : row_bytes + 16;
}

// Copy ROWS token rows of `row_bytes` bytes (a multiple of 16) from global
// memory into LDS at pitch stage_pitch(row_bytes), every 16-byte chunk passed
// through `f`.  A round moves CPR chunks of every row per thread (2 for up to
// 4 rows, else 1: a 4096-element fp16 row, or 4096 int8 codes, in one round), all loads before their stores; `after` runs between the
// first round's loads and stores, so that loads the caller issues there
// overlap the staging.  Rows past the resource's end are staged as zeros.
template <int ROWS, int THREADS, typename F, typename A>
__device__ __forceinline__ void stage_rows(int8_t* dst, rsrc_t src, int row_bytes, F f, A after) {
  constexpr int CPR = ROWS <= 4 ? 2 : 1;
  const int kc = row_bytes >> 4, pitch = stage_pitch(row_bytes);
  v4i v[ROWS][CPR];
  auto load = [&](int c0) {
#pragma unroll
    for (int i = 0; i < CPR; ++i) {
      const int c = c0 + (int)threadIdx.x + i * THREADS;
#pragma unroll
      for (int m = 0; m < ROWS; ++m)
        v[m][i] = bld16(src, c < kc ? (u32)(m * row_bytes + 16 * c) : kOOB);
    }
  };
  auto store = [&](int c0) {
#pragma unroll
    for (int i = 0; i < CPR; ++i) {
      // a chunk past the row end is written (as zeros) into the row's padding
      const int c = c0 + (int)threadIdx.x + i * THREADS, cc = c < kc ? c : kc;
#pragma unroll
      for (int m = 0; m < ROWS; ++m) st16(dst + m * pitch + 16 * cc, f(v[m][i]));
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

// Like stage_rows, for a slice of longer rows: bytes col0 .. col0 + row_bytes
// of each of ROWS rows src_stride bytes apart, into LDS rows of pitch bytes
// (at least stage_pitch(row_bytes)).  Chunks past the slice are written as
// zeros into the row's padding; rows past the resource's end are zeros.
template <int ROWS, int THREADS, typename A>
__device__ __forceinline__ void stage_slice(int8_t* dst, int pitch, rsrc_t src, int src_stride,
                                            int col0, int row_bytes, A after) {
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
      for (int m = 0; m < ROWS; ++m) st16(dst + m * pitch + 16 * cc, v[m][i]);
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

// Scale and zero point of the weight rows of a workgroup (`rows` rows of G
// groups, fp16 bits, contiguous in global memory) staged in LDS as words
// s | z << 16 at pitch G + 1, an odd number of words, so that the 16 rows of
// one group read hit 16 different banks.  EPT elements per thread are loaded
// per round, all before their stores.  Elements past the buffer resources'
// ends read as zeros.
__host__ __device__ constexpr int sz_pitch(int G) { return G + 1; }

template <int THREADS, int EPT>
struct ScaleZeroStage {
  uint16_t s[EPT], z[EPT];
  int e0;
  __device__ __forceinline__ void load(rsrc_t sr, rsrc_t zr, int total, int c0) {
    e0 = c0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = c0 + (int)threadIdx.x + i * THREADS;
      s[i] = bld2(sr, e < total ? (u32)(2 * e) : kOOB);
      z[i] = bld2(zr, e < total ? (u32)(2 * e) : kOOB);
    }
  }
  __device__ __forceinline__ void store(u32* dst, int G, int total) const {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = e0 + (int)threadIdx.x + i * THREADS;
      if (e < total) {
        const int row = e / G;
        dst[row * sz_pitch(G) + (e - row * G)] = (u32)s[i] | ((u32)z[i] << 16);
      }
    }
  }
  // all rows: first round issued by the caller (so it can overlap other
  // loads), the rest here
  __device__ __forceinline__ void finish(rsrc_t sr, rsrc_t zr, u32* dst, int G, int total) {
    store(dst, G, total);
    for (int c0 = EPT * THREADS; c0 < total; c0 += EPT * THREADS) {
      load(sr, zr, total, c0);
      store(dst, G, total);
    }
  }
};

// Waves (16-row weight blocks) per workgroup of the wide decode kernels: the
// grid should come out near one workgroup per CU (256 on MI355X), so that the
// token rows are read by as few workgroups as the weight stream allows.
inline int wide_waves(int N) {
  const int nblocks = (N + 15) / 16;
  const int nb = (nblocks + 128) / 256;
  return nb < 1 ? 1 : nb > 4 ? 4 : nb;
}

// s_waitcnt vmcnt(n) for an n known once the caller's loop is unrolled (the
// switch folds to one case); n > 63 waits for everything.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define QG_WAITVM(i) case i: asm volatile("s_waitcnt vmcnt(" #i ")" ::: "memory"); break;
    QG_WAITVM(0) QG_WAITVM(1) QG_WAITVM(2) QG_WAITVM(3) QG_WAITVM(4) QG_WAITVM(5) QG_WAITVM(6)
    QG_WAITVM(7) QG_WAITVM(8) QG_WAITVM(9) QG_WAITVM(10) QG_WAITVM(11) QG_WAITVM(12)
    QG_WAITVM(13) QG_WAITVM(14) QG_WAITVM(15) QG_WAITVM(16) QG_WAITVM(17) QG_WAITVM(18)
    QG_WAITVM(19) QG_WAITVM(20) QG_WAITVM(21) QG_WAITVM(22) QG_WAITVM(23) QG_WAITVM(24)
    QG_WAITVM(25) QG_WAITVM(26) QG_WAITVM(27) QG_WAITVM(28) QG_WAITVM(29) QG_WAITVM(30)
    QG_WAITVM(31) QG_WAITVM(32) QG_WAITVM(33) QG_WAITVM(34) QG_WAITVM(35) QG_WAITVM(36)
    QG_WAITVM(37) QG_WAITVM(38) QG_WAITVM(39) QG_WAITVM(40) QG_WAITVM(41) QG_WAITVM(42)
    QG_WAITVM(43) QG_WAITVM(44) QG_WAITVM(45) QG_WAITVM(46) QG_WAITVM(47) QG_WAITVM(48)
    QG_WAITVM(49) QG_WAITVM(50) QG_WAITVM(51) QG_WAITVM(52) QG_WAITVM(53) QG_WAITVM(54)
    QG_WAITVM(55) QG_WAITVM(56) QG_WAITVM(57) QG_WAITVM(58) QG_WAITVM(59) QG_WAITVM(60)
    QG_WAITVM(61) QG_WAITVM(62) QG_WAITVM(63)
#undef QG_WAITVM
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// 16-byte buffer loads of every lane straight into LDS at lds + 16 lane (lds
// wave-uniform).  dma16: non-temporal, for data read once per call (the
// weights, their scales); dma16_keep: the default policy, for data other
// workgroups read too.  The builtin sits in plain device functions so that
// the host pass keeps the kernels that use it.
#define QG_LDS(p) ((__attribute__((address_space(3))) void*)(p))
__device__ __forceinline__ void dma16(rsrc_t r, int8_t* lds, u32 voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, QG_LDS(lds), 16, voff, 0, 0, kAuxNonTemporal);
}
__device__ __forceinline__ void dma16_keep(rsrc_t r, int8_t* lds, u32 voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, QG_LDS(lds), 16, voff, 0, 0, 0);
}

// Kilobytes of LDS that `chunks` 16-byte chunks take.
__host__ __device__ constexpr int kb_of_chunks(int chunks) { return (chunks + 63) / 64; }

// Scales and zero points of a 16-row weight block (rows_n rows of G fp16
// values each, contiguous; rows past rows_n read as zeros) into LDS as
// [16][G] arrays at lds and lds + 1024 kb (kb = kb_of_chunks(2 G)), then
// extra_kb kilobytes of the resource xr at lds + 2048 kb; kilobyte t by wave
// t mod WAVES with buffer-to-LDS loads, whose completion the caller waits
// for (vmcnt) before its barrier.  Buffer range checks work per dword: a
// dword only partly inside the range reads as zero, bytes inside it too
// (seen on MI355X).  A block cut short by N (2 G rows_n bytes, not always a
// multiple of 4) therefore stages its scales and zero points element by
// element; the caller's barrier must then also wait for LDS stores
// (lds_barrier).
template <int WAVES>
__device__ __forceinline__ void stage_block_sz(int8_t* lds, rsrc_t sr, rsrc_t zr, int rows_n,
                                               int G, rsrc_t xr, int extra_kb) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = kb_of_chunks(2 * G);
  const int t0 = rows_n == 16 ? 0 : 2 * kb;
  for (int t = t0 + wave; t < 2 * kb + extra_kb; t += WAVES) {
    const u32 o = (u32)(1024 * (t < kb ? t : t < 2 * kb ? t - kb : t - 2 * kb) + 16 * lane);
    if (t < kb) dma16(sr, lds + 1024 * t, o);
    else if (t < 2 * kb) dma16(zr, lds + 1024 * t, o);
    else dma16(xr, lds + 1024 * t, o);
  }
  if (rows_n < 16) {
    uint16_t* sw = reinterpret_cast<uint16_t*>(lds);
    uint16_t* zw = reinterpret_cast<uint16_t*>(lds + 1024 * kb);
    for (int el = (int)threadIdx.x; el < 16 * G; el += 64 * WAVES) {
      sw[el] = bld2(sr, (u32)(2 * el));
      zw[el] = bld2(zr, (u32)(2 * el));
    }
  }
}

// Barrier for LDS data written by the workgroup: waits for this wave's LDS
// accesses only, leaving its global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace qg
