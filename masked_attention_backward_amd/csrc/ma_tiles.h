// LDS tile layout and tile-level visibility shared by the forward and backward kernels.
//
// A staged tile is 64 rows x 128 columns of 16-bit elements, row-major, 256 bytes per
// row, with no padding.  The sixteen 16-byte chunks of a row are XOR-swizzled with
//     f(row) = ((row & 3) << 2) | ((row >> 2) & 3)
// so that
//   * a 16-byte read of one chunk by 16 lanes on 16 consecutive rows hits 16 distinct
//     chunk positions (MFMA operands taken along a row), and
//   * a ds_read_b64_tr_b16 group (4 consecutive rows x 32 columns per half-wave) spreads
//     its 4 rows over 4 distinct 16-byte groups (MFMA operands taken down a column).
#pragma once

#include <type_traits>

#include "ma_device.h"

namespace ma {

constexpr int TILE_ROWS = 64;
constexpr int TILE_ELEMS = TILE_ROWS * HD;   // 8192 elements = 16 KiB

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Element offset of (row, column) inside a staged tile.
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * HD + ((((col >> 3) ^ swz(row)) << 3) | (col & 7));
}

// Staged operand tiles live in one LDS array of two stages x two tiles (A, B): tile k of
// stage s starts at byte (2 s + k) * 16384; moving to the other stage flips the lane's
// offsets by 32 KiB.
constexpr int TILE_BYTES = TILE_ELEMS * 2;     // 16384
constexpr int STAGE_BYTES = 2 * TILE_BYTES;    // 32768

// Lane-dependent byte offsets of the MFMA operand fragments inside the staged tiles, with
// the current stage folded in.  Every fragment read is one of these offsets plus a
// compile-time constant (the array's LDS base, 16384 B for tile B, 8192 B per 32-row block,
// 4096 B per 16-row k-step), which the LDS instructions take as an immediate.
//   row[ks]        operand taken along a row: lane (c, h) reads columns [16 ks + 8 h, +8)
//                  of row c (add 8192 B for rows 32..63)
//   col[2 nb + i]  operand taken down a column with ds_read_b64_tr_b16: lane l = 32 h + c
//                  receives tile[row][32 nb + c] for the rows 16 t4 + 8 (s/4) + 4 h + (s%4),
//                  s = 0..7 (i = s/4; add 4096 B per t4), i.e. the k-slot order an
//                  accumulator tile has when it is fed back as an operand (accumulator
//                  register r = 8 (t4%2) + s of row block t4/2)
struct FragOff {
  int row[8];
  int col[8];
  __device__ __forceinline__ explicit FragOff(int lane) {
    const int c = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) row[ks] = 2 * (c * HD + (((2 * ks + h) ^ swz(c)) << 3));
    const int rin = (lane & 15) >> 2;
    const int cs = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      col[2 * nb] = 2 * tile_off(4 * h + rin, 32 * nb + cs);
      col[2 * nb + 1] = 2 * tile_off(8 + 4 * h + rin, 32 * nb + cs);
    }
  }
};

// Row-taken fragment of tile k (0 = A, 1 = B) of the current stage.
__device__ __forceinline__ u32x4 frag_row(const uint16_t* stages, const FragOff& f, int k, int ks, int mb) {
  return ld16(reinterpret_cast<const char*>(stages) + f.row[ks] + k * TILE_BYTES + mb * 8192);
}

// Column-taken (transposing) fragment of tile k of the current stage.
__device__ __forceinline__ u32x4 frag_col(const uint16_t* stages, const FragOff& f, int k, int t4, int nb) {
  typedef short short4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) short4v* lds_ptr;
  const char* base = reinterpret_cast<const char*>(stages) + k * TILE_BYTES + t4 * 4096;
  short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(base + f.col[2 * nb]));
  short4v y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(base + f.col[2 * nb + 1]));
  u32x2 xa = __builtin_bit_cast(u32x2, x);
  u32x2 ya = __builtin_bit_cast(u32x2, y);
  u32x4 o;
  o[0] = xa[0];
  o[1] = xa[1];
  o[2] = ya[0];
  o[3] = ya[1];
  return o;
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// LDS byte address of a pointer into a __shared__ array (taken once per kernel: the
// generic-to-LDS conversion carries a null check, so the kernels keep integer addresses).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_ptr)(p);
}

// Global -> LDS copies (LDS DMA): the wave-instruction reads 16 bytes (4 bytes for dma4)
// per lane from sbase + voff and writes them, lane after lane, to LDS starting at byte
// address `lds` (taken from M0).  They are issued from inline assembly on purpose: the
// compiler would treat each one as a possible write to any later-read LDS location and
// wait for it to complete before the next LDS read, which serialises the whole
// prefetch.  The kernels order these copies against their LDS reads themselves: an
// explicit vmcnt wait by every wave, then a workgroup barrier, before a stage is read.
// M0 (the LDS destination) is set inside each statement and declared clobbered; nothing
// else in these kernels reads M0 (on gfx950 LDS instructions do not use it), so no
// compiler-held value lives there across the copies.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "m0");
}
// The same with the non-temporal hint (data read once: streamed through L2 rather than kept).
__device__ __forceinline__ void dma16nt(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds)
               : "m0");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "m0");
}

// Cooperative load of one 64 x 128 tile (rows clamped into [0, nrows), row stride HD)
// straight from global memory into a swizzled LDS tile (global_load_lds_dwordx4: each
// wave-instruction fills 1 KiB = 4 rows of LDS, lane i writing bytes [16 i, 16 i + 16) of
// it).  The swizzle is applied on the global side: the lane that fills physical chunk p
// of row r fetches logical chunk p ^ f(r).  16 wave-instructions per tile, spread over
// the NW waves of the workgroup.
template <int NW>
__device__ __forceinline__ void tile_load_async(uint32_t tile_lds, const uint16_t* base, int row0, int nrows, int w,
                                                int lane) {
#pragma unroll
  for (int j = 0; j < (16 + NW - 1) / NW; ++j) {
    const int u = w + j * NW;
    if ((16 % NW) == 0 || u < 16) {
      const int row = 4 * u + (lane >> 4);
      const int p = lane & 15;
      const int g = min(row0 + row, nrows - 1);
      const uint32_t off = 2u * (uint32_t)(g * HD + ((p ^ swz(row)) << 3));
      dma16(base, off, __builtin_amdgcn_readfirstlane(tile_lds + (uint32_t)u * 1024u));
    }
  }
}

// 64 consecutive fp32 values straight into LDS by one wave (the per-row buffers are
// padded to a multiple of 64 rows).
__device__ __forceinline__ void row_load_async(uint32_t dst_lds, const float* src, int lane) {
  dma4(src, 4u * (uint32_t)lane, __builtin_amdgcn_readfirstlane(dst_lds));
}

// The global->LDS loads of one stage (tile A and tile B of 64 rows each, same rows of two
// tensors), prepared once and then issued one wave-instruction at a time, so that a wave
// can spread them over the matrix-core work of the tile it is computing instead of
// queueing all of them on the memory pipeline at once.  Instruction i < J fills rows
// [4u, 4u + 4) of tile A, u = w + i NW; instruction J + i does the same for tile B.
template <int NW>
struct StageLoads {
  static constexpr int J = (16 + NW - 1) / NW;   // instructions per tile for wave 0
  const uint16_t* srca;                          // head base of tensor A (wave-uniform)
  const uint16_t* srcb;                          // head base of tensor B
  uint32_t dst;                                  // LDS byte address of the stage (tile A; tile B follows)
  uint32_t off[J];                               // this lane's byte offset per instruction

  __device__ __forceinline__ void prepare(const uint16_t* a, const uint16_t* b, uint32_t stage_lds, int row0,
                                          int nrows, int w, int lane) {
    srca = a;
    srcb = b;
    dst = stage_lds;
    const int p = lane & 15;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int row = 4 * (w + j * NW) + (lane >> 4);
      off[j] = 2u * (uint32_t)(min(row0 + row, nrows - 1) * HD + ((p ^ swz(row)) << 3));
    }
  }
  // Number of instructions wave w issues (issue(i) for i >= count(w) does nothing).
  __device__ __forceinline__ static constexpr bool exists(int j, int w) { return (16 % NW) == 0 || w + j * NW < 16; }
  __device__ __forceinline__ void issue(int i, int w) const {
    const int j = i < J ? i : i - J;
    if (!exists(j, w)) return;
    const uint32_t d = dst + (uint32_t)((i < J ? 0 : TILE_BYTES) + (w + j * NW) * 1024);
    dma16(i < J ? srca : srcb, off[j], __builtin_amdgcn_readfirstlane(d));
  }
};

// Wait until at most N of this wave's vector-memory operations are outstanding (they
// complete in issue order, so everything issued before the last N is done).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}


struct TileRef {
  int head, tile;
  uint64_t bits;
};


// Work item decode of a window-path grid over (batch, query head, tile pair p) (dQ and the
// forward).
// Consecutive workgroups go to the eight XCDs in turn; when the (batch, kv head) pairs split
// evenly over them, XCD x serves the kv heads x, x + 8, ..., so the query heads that stream
// the same K/V tiles share that XCD's L2.  Lower p (heavier tiles) is dispatched first.
__device__ __forceinline__ void window_q_item(const AttnArgs& a, int wg, int& b, int& hq, int& p) {
  const int nbk = a.B * a.Hkv;
  if ((nbk & 7) == 0) {
    const int xcd = wg & 7, idx = wg >> 3;
    const int per = (nbk >> 3) * a.group;
    p = idx / per;
    const int rem = idx - p * per;
    const int m = rem / a.group, hs = rem - m * a.group;
    const int bk = xcd + 8 * m;
    b = bk / a.Hkv;
    hq = (bk - b * a.Hkv) * a.group + hs;
  } else {
    const int nbh = a.B * a.Hq;
    const int bh = wg % nbh;
    p = wg / nbh;
    b = bh / a.Hq;
    hq = bh % a.Hq;
  }
}

#define MA_STEP() __builtin_amdgcn_sched_barrier(0)


}  // namespace ma
