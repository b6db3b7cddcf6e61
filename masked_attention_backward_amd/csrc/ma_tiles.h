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

#include "ma_device.h"

namespace ma {

constexpr int TILE_ROWS = 64;
constexpr int TILE_ELEMS = TILE_ROWS * HD;   // 8192 elements = 16 KiB

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Element offset of (row, column) inside a staged tile.
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * HD + ((((col >> 3) ^ swz(row)) << 3) | (col & 7));
}

// MFMA operand taken along a row: lane (c, h) gets columns [16*ks + 8*h, +8) of row `row`.
__device__ __forceinline__ u32x4 frag_row(const uint16_t* tile, int row, int ks, int h) {
  return ld16(tile + row * HD + (((2 * ks + h) ^ swz(row)) << 3));
}

// MFMA operand taken down a column with the transposing LDS read.  Lane l = 32*h + c
// receives the eight values tile[row][col0 + c] for the rows
//     16*t4 + 8*(s/4) + 4*h + (s%4),   s = 0..7,
// i.e. the k-slot order an accumulator tile has when it is fed back as an operand
// (accumulator register r = 8*(t4%2) + s of row block t4/2).
__device__ __forceinline__ u32x4 frag_col(const uint16_t* tile, int t4, int col0, int lane) {
  const int h = lane >> 5;
  const int rin = (lane & 15) >> 2;
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int r1 = 16 * t4 + 4 * h + rin;
  const int r2 = r1 + 8;
  typedef short short4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) short4v* lds_ptr;
  short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(tile + tile_off(r1, col)));
  short4v y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(tile + tile_off(r2, col)));
  u32x2 xa = __builtin_bit_cast(u32x2, x);
  u32x2 ya = __builtin_bit_cast(u32x2, y);
  u32x4 o;
  o[0] = xa[0];
  o[1] = xa[1];
  o[2] = ya[0];
  o[3] = ya[1];
  return o;
}

// Cooperative copy of one 64 x 128 tile from global memory (rows clamped into
// [0, nrows), row stride HD) into registers, then into a swizzled LDS tile.
template <int NT>
struct TileStage {
  static constexpr int CPT = (TILE_ROWS * 16 + NT - 1) / NT;   // 16-byte chunks per thread
  u32x4 r[CPT];
  __device__ __forceinline__ void load(const uint16_t* base, int row0, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * NT;
      if (CPT * NT == TILE_ROWS * 16 || idx < TILE_ROWS * 16) {
        const int row = idx >> 4, ch = idx & 15;
        const int g = min(row0 + row, nrows - 1);
        r[i] = ld16(base + (size_t)g * HD + ch * 8);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * NT;
      if (CPT * NT == TILE_ROWS * 16 || idx < TILE_ROWS * 16) {
        const int row = idx >> 4, ch = idx & 15;
        st16(tile + row * HD + ((ch ^ swz(row)) << 3), r[i]);
      }
    }
  }
};

// Visibility of the elements of one (query-tile, key-tile) pair.
//   window:  query i sees key j iff 0 <= i - j < window, both inside their sequences
//   block:   a 64-bit mask over the 64 rows of the iterated tile (built by TileWalker)
struct WindowVis {
  int sq, skv, window;
  // true when every (i, j) in [q0, q0+nq) x [k0, k0+nk) is visible
  __device__ __forceinline__ bool full(int q0, int nq, int k0, int nk) const {
    return (q0 - (k0 + nk - 1) >= 0) && ((q0 + nq - 1) - k0 < window) && (q0 + nq <= sq) && (k0 + nk <= skv);
  }
  __device__ __forceinline__ bool vis(int i, int j) const {
    return ((unsigned)(i - j) < (unsigned)window) && (i < sq) && (j < skv);
  }
};

}  // namespace ma
