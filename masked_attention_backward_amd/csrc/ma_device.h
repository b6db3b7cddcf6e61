// Device helpers shared by the masked attention kernels (gfx950 / CDNA4 only).
//
// MFMA conventions used throughout (v_mfma_f32_32x32x16_{f16,bf16}, wave64):
//   lane l = 32*h + c  (c = l % 32, h = l / 32)
//   A operand (32 x 16, M x K): lane l holds row m = c, eight k-slots of half h.
//   B operand (16 x 32, K x N): lane l holds column n = c, the same eight k-slots.
//   C/D (32 x 32): lane l, accumulator r in [0,16): row 8*(r/4) + 4*h + (r%4), column c.
// The contraction pairs A-slot s of half h with B-slot s of half h, so any bijection of
// (h, s) onto the 16 k indices is valid as long as both operands use the same one.  The
// kernels exploit that: an accumulator tile (rows spread over registers) is fed back as
// the A or B operand of the next product with the k index permuted to match.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ma {

constexpr int HD = 128;          // head dimension (the only one supported)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Element-type traits: 16-bit storage, fp32 compute.
struct F16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  }
  // Two fp32 values -> two halves, round to nearest even (one v_cvt_pk_f16_f32).
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
  }
  static __device__ __forceinline__ float lo(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  }
  static __device__ __forceinline__ uint16_t one(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
  // Two products a s, b s rounded once each to half (mixed-precision FMA: the fp32 product is
  // not rounded first).
  static __device__ __forceinline__ uint32_t pack2s(float a, float b, float s) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)(a * s));
    const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(b * s));
    return lo | (hi << 16);
  }
};

struct BF16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
  // Two fp32 values -> two bfloat16, round to nearest even (one v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  }
  static __device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
  static __device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
  static __device__ __forceinline__ uint16_t one(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
  static __device__ __forceinline__ uint32_t pack2s(float a, float b, float s) { return pack2(a * s, b * s); }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Pack eight accumulator values acc[r0 .. r0+7] into one MFMA operand (eight 16-bit slots).
template <class T>
__device__ __forceinline__ u32x4 pack8(const f32x16& acc, int r0) {
  u32x4 o;
  o[0] = T::pack2(acc[r0 + 0], acc[r0 + 1]);
  o[1] = T::pack2(acc[r0 + 2], acc[r0 + 3]);
  o[2] = T::pack2(acc[r0 + 4], acc[r0 + 5]);
  o[3] = T::pack2(acc[r0 + 6], acc[r0 + 7]);
  return o;
}

// Bits [a, b) of a 64-bit word, 0 <= a <= b <= 64.
__device__ __forceinline__ uint64_t range_bits(int a, int b) {
  uint64_t hi = (b >= 64) ? ~0ull : ((1ull << b) - 1ull);
  uint64_t lo = (a >= 64) ? ~0ull : ((1ull << a) - 1ull);
  return hi & ~lo;
}

// Walks the 64-row tiles covered by an ascending list of kept blocks (one row of a
// selection table).  Each visited tile is reported once, in ascending order, with the
// bitmask of its rows that lie inside a kept block and inside the sequence.
// The list is read through the constant address space: the tables are written by an earlier
// launch and only read here, and the walk is wave-uniform, so each entry is a scalar load
// (scalar cache, counted by lgkmcnt) and never waits for the kernel's outstanding
// global->LDS tile copies (vmcnt).
typedef const __attribute__((address_space(4))) int* const_int_ptr;
struct TileWalker {
  const_int_ptr sel;
  int cnt, blk, len;
  int idx, last;
  int pj;   // entry(idx) when already loaded (whole-tile walk only; pj < 0: not loaded)
  __device__ TileWalker(const int* sel_, int cnt_, int blk_, int len_)
      : sel((const_int_ptr)sel_), cnt(cnt_), blk(blk_), len(len_), idx(0), last(-1), pj(-1) {}
  // Entry k of the list (wave-uniform k < cnt).
  __device__ int entry(int k) const { return sel[k]; }
  __device__ bool next(int& tile, uint64_t& bits) {
    if ((blk & 63) == 0) {
      // Blocks of whole 64-row tiles: a tile lies in one block, its bits are that block's rows
      // (all of them but in the sequence's last tile), and one entry load serves the tile; it
      // is issued one call ahead, so the caller does not wait for it.
      while (idx < cnt) {
        const int j = pj >= 0 ? pj : entry(idx);
        pj = -1;
        const int hi = min(j * blk + blk, len);
        const int t = max(j * (blk >> 6), last + 1);
        if (t * 64 >= hi) {
          ++idx;
          continue;
        }
        if (t * 64 + 64 >= hi) {   // the block's last tile
          ++idx;
          if (idx < cnt) pj = entry(idx);
        } else {
          pj = j;
        }
        last = t;
        tile = t;
        bits = range_bits(0, hi - t * 64);
        return true;
      }
      return false;
    }
    while (idx < cnt) {
      const int j = entry(idx);
      const int lo = j * blk;
      const int hi = min(lo + blk, len);
      int t = lo >> 6;
      if (t <= last) t = last + 1;
      if (t * 64 >= hi) {
        ++idx;
        continue;
      }
      const int t0 = t * 64, t1 = t0 + 64;
      uint64_t m = 0;
      for (int k = idx; k < cnt; ++k) {
        const int j2 = entry(k);
        const int lo2 = max(j2 * blk, t0);
        const int hi2 = min(min(j2 * blk + blk, len), t1);
        if (j2 * blk >= t1) break;
        if (lo2 < hi2) m |= range_bits(lo2 - t0, hi2 - t0);
      }
      last = t;
      tile = t;
      bits = m;
      return true;
    }
    return false;
  }
};

// Kernel argument block shared by the attention kernels.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  const float* lse2;     // lse * log2(e), written by the preprocess kernel
  const float* delta;
  const float* sink;
  void* dq;
  void* dk;
  void* dv;
  void* out_o;
  float* out_lse;
  const uint8_t* mask;   // [B, N, nqb, nkb]
  const int* sel_q;      // [B, N, nqb, nkb]
  const int* cnt_q;      // [B, N, nqb]
  const int* sel_k;      // [B, N, nkb, nqb]
  const int* cnt_k;      // [B, N, nkb]
  int B, Hq, Hkv, Sq, Skv, group;
  int window;
  int bx, by, nqb, nkb;
  float scale, scale_log2;
  int n_tiles;           // stationary tiles per head (window path)
  int pair;              // 1: workgroup p also runs tile n_tiles-1-p
  const int* cu;         // packed sequences: [B + 1] row offsets (nullptr: dense [B, H, S, D])
  int total;             // packed sequences: rows per head of every tensor
  int chunk;             // block path: selected query blocks per dK/dV workgroup (0: no limit);
                         // window path with a head split: tile visits per dK/dV workgroup
  int max_chunks;        // chunks per (kv head, key block or key tile) the dK/dV grid provides
                         // for (1: no split)
  float* dkv_part;       // split key blocks / tiles: fp32 partial dK (scaled) and dV,
                         // [2][B][Hkv][max_chunks][padded Skv][D]
  uint16_t* ds_bank;     // window path: dS of every live 32 x 32 block, written by dK/dV and
                         // read by the dQ GEMM (nullptr: dQ recomputes S and dP instead)
  int ds_kb;             // window path: ceil((window - 1) / 32), live key blocks below the diagonal
  long long ds_blocks;   // window path: live 32 x 32 blocks per (sequence, query head)
  int dq_nw;             // window path with a dS bank: waves per dQ workgroup (4 or 8)
  int ds_nka;            // block path with a dS bank: 32-row key blocks per 32-row query block
                         // (bank entry of (head, qa, ka): head * ds_blocks + qa * ds_nka + ka)
  const float* dsink_part;  // window path: the preprocess's dsink partials, [B][Hq][dsink_nblk]
  float* dsink_out;         // window path: dsink [Hq], reduced by the first dK/dV workgroup
                            // (nullptr: not reduced there)
  int dsink_nblk;           // window path: partials per (sequence, head)
};

// dsink[h] = - sum_b sum_blk part[b][h][blk], by one wave: lane-strided partial sums in a
// fixed order, then a butterfly over the 64 lanes (bit-identical run to run).
__device__ __forceinline__ void dsink_head_sum(const float* __restrict__ part, float* __restrict__ dsink, int B,
                                               int H, int nblk, int h, int lane) {
  float acc = 0.f;
  for (int b = 0; b < B; ++b)
    for (int i = lane; i < nblk; i += 64) acc += part[((size_t)b * H + h) * nblk + i];
  acc += __shfl_xor(acc, 32);
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 8);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 1);
  if (lane == 0) dsink[h] = -acc;
}

// Where the rows of sequence b lie in a tensor of H heads.  Dense: [B, H, S, D], S rows per
// sequence.  Packed: [H, total, D] with sequence b at rows cu[b] .. cu[b + 1] of every head;
// the offsets are clamped to [0, total] and the length to S (the longest sequence), so any
// offset table keeps every access inside the tensors and the padded per-row buffers.
// Row r of head h of the sequence is row base + h * head_stride + r.
struct SeqRows {
  size_t head_stride, base;
  int len;
};

__device__ __forceinline__ SeqRows seq_rows(const AttnArgs& a, int b, int H, int S) {
  if (a.cu) {
    const int s0 = min(max(a.cu[b], 0), a.total);
    const int s1 = min(max(a.cu[b + 1], s0), a.total);
    return SeqRows{(size_t)a.total, (size_t)s0, min(s1 - s0, S)};
  }
  return SeqRows{(size_t)S, (size_t)b * H * S, S};
}

enum { MASK_WINDOW = 0, MASK_BLOCK = 1 };

// The dS bank (window path).  Query block a (rows 32a .. 32a + 31 of a sequence) sees key
// blocks lo(a) = max(0, a - kb) .. a, kb = ceil((window - 1) / 32), exactly the blocks holding
// a visible (q, k) pair.  A (sequence, head) stores them query block after query block, key
// blocks ascending: block (a, b) is entry band_offset(a) + b - lo(a), 2048 bytes each, holding
// the 16-bit dS[q][k] of the block as two dQ-operand fragments (k-steps t = 0, 1; 64 lanes x
// 16 bytes each): lane 32 h + c holds dS[q = c][k = 16 t + 8 (s / 4) + 4 h + s % 4], s = 0..7,
// the k-slot order of a column-taken key tile.
__device__ __forceinline__ int band_lo(int a, int kb) { return max(0, a - kb); }
__device__ __host__ __forceinline__ long long band_offset(long long a, long long kb) {
  // sum over a' < a of (min(a', kb) + 1)
  return a <= kb + 1 ? a * (a + 1) / 2 : (kb + 1) * (kb + 2) / 2 + (a - kb - 1) * (kb + 1);
}
// Window path: windows of at least 256 tokens take the eight-wave dK/dV kernel over 128-row
// key tiles, shorter ones the four-wave kernel over 64-row key tiles (W = min(window, S)).
__device__ __host__ __forceinline__ bool window_wide(int W) { return W >= 256; }
__device__ __host__ __forceinline__ int window_key_rows(int W) { return window_wide(W) ? 128 : 64; }
// The 64-row query tiles key tile p visits: rows [c0, min(S, c0 + bc + W - 1)) of every query
// head of its group, c0 = bc p, bc = window_key_rows(W).
__device__ __host__ __forceinline__ int window_qtiles(int S, int W, int p) {
  const int bc = window_key_rows(W);
  const int c0 = p * bc;
  const int qend = S < c0 + bc + W - 1 ? S : c0 + bc + W - 1;
  const int n = ((qend + 63) >> 6) - (c0 >> 6);
  return n > 0 ? n : 0;
}
// Head split of key tiles when too few workgroups would fill the GPU: the workgroups key tile
// p's visits (query heads x query tiles) are spread over, whole query heads each, at most
// `target` visits per workgroup where the group allows (1: not split).
__device__ __host__ __forceinline__ int window_chunks(int S, int W, int group, int target, int p) {
  const int n = (group * window_qtiles(S, W, p) + target - 1) / target;
  return n < 1 ? 1 : (n > group ? group : n);
}
// The same in 32-bit arithmetic, exact while the head's bank holds fewer than 2^30 blocks.
__device__ __forceinline__ int band_offset32(int a, int kb) {
  return a <= kb + 1 ? (a * (a + 1)) >> 1 : (((kb + 1) * (kb + 2)) >> 1) + (a - kb - 1) * (kb + 1);
}

}  // namespace ma
