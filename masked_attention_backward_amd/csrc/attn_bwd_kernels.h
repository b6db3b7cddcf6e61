// Attention backward kernels for gfx950: a key/value-tile-stationary dK/dV kernel and a
// query-tile-stationary dQ kernel (the preprocess and dsink reduce are in attn_bwd.hip).
// Both recompute S = scale Q K^T and P = exp(S - lse) tile by tile (the FlashAttention-style
// recompute of the five-GEMM backward: S, P, dV += P^T dO, dP = dO V^T, dS = P (dP - Delta),
// dK += dS^T Q, dQ += dS K), as described on the page "[Example] Add GQA Sink Backward BHSD
// ..." (commit of the 9->6 kernel revision: QK^T, softmax, dV+dP, dS, dK+dQ; commit of the
// 4->2 revision: Delta = sum(O*dO), five GEMMs, dSink) and on the page "knowledge(triton) ...
// #174" (BlockSparseAttentionGrad skeleton: delta, then dq over the q-major table, then dk/dv
// over the kv-major table).
//
// Design on CDNA4, differing from the pages' Ascend kernels:
//   * dK/dV accumulate in registers of the workgroup that owns the key tile, and dQ in the
//     workgroup that owns the query tile, so there are no atomics and no fp32 partial
//     buffers in HBM: results are bit-identical run to run (the pages' single-kernel revision
//     accumulated dK/dV with fp32 atomics and a host-side cast).
//   * P and dS never leave registers: the accumulator tile of S (or S^T) is re-packed in place
//     as the A operand of the next MFMA, with the contraction index permuted to match (see
//     ma_device.h), and the other operand is read down the columns of the staged tile with
//     ds_read_b64_tr_b16.
//   * Both kernels run two waves per SIMD (at most 256 registers per lane), so one wave's LDS
//     reads, scalar work and softmax issue next to the other wave's matrix-core work; a
//     single wave per SIMD issues at most one instruction per cycle pair of the MFMA pipe's
//     32-cycle step and leaves the matrix core idle much of the time.
//   * Tiles come from HBM straight into LDS (global_load_lds_dwordx4), double-buffered: the
//     next tile's loads are issued right after the barrier that frees its stage.
#pragma once

#include "ma_launch.h"
#include "ma_tiles.h"

namespace ma {

// ------------------------------------------------------------------ tile sources
// Sequence of (query head, 64-row tile, row bitmask) a stationary workgroup visits.
// Heads [head, hend) in order, each over the tiles [tlo, thi); counters only, no division.
struct WindowSource {
  int head, hend, tlo, thi, tile;
  __device__ static WindowSource make(int head0, int nheads, int tlo, int nt) {
    return WindowSource{head0, nt > 0 ? head0 + nheads : head0, tlo, tlo + nt, tlo};
  }
  __device__ bool next(int& hd, int& t, uint64_t& bits) {
    if (head >= hend) return false;
    hd = head;
    t = tile;
    bits = 0;
    if (++tile >= thi) {
      tile = tlo;
      ++head;
    }
    return true;
  }
};

// Tiles [tlo, tlo + nt) from the last one down, each over the heads [head0, head0 + nheads)
// (tiles outer), or every tile of a head before the next head (heads outer).  The dK/dV
// workgroups of one kv head (all on one XCD) then read the same query tiles at about the same
// time: tiles outer on wide windows (for causal masks every walk ends at the last tile);
// heads outer on narrow windows, where neighbouring key tiles see overlapping runs of a few
// query tiles and one head's run for all resident workgroups fits the XCD's L2.
struct WindowSourceDesc {
  int head0, hend, tlo, thi, tile, head;
  bool heads_outer;   // narrow windows: every tile of a head, then the next head
  __device__ static WindowSourceDesc make(int head0, int nheads, int tlo, int nt, bool heads_outer = false) {
    return WindowSourceDesc{head0, head0 + nheads, tlo, tlo + nt - 1, tlo + nt - 1, head0, heads_outer};
  }
  __device__ bool next(int& hd, int& t, uint64_t& bits) {
    if (tile < tlo || head >= hend) return false;
    hd = head;
    t = tile;
    bits = 0;
    if (heads_outer) {
      if (--tile < tlo) {
        tile = thi;
        ++head;
      }
    } else if (++head >= hend) {
      head = head0;
      --tile;
    }
    return true;
  }
};

struct BlockSource {
  TileWalker walk;
  int head;
  __device__ bool next(int& hd, int& tile, uint64_t& bits) {
    hd = head;
    return walk.next(tile, bits);
  }
};

// The query tiles a key block of a K/V head sees on the block path: the rows of the kv-major
// table of every query head of its group, one head after the other (a single head for MHA).
// A workgroup may take only a chunk of that concatenated list: entries [first, first + count).
struct BlockGroupSource {
  const int* sel_k = nullptr;   // [B, Hq, nkb, nqb]
  const_int_ptr cnt_k = nullptr;   // [B, Hq, nkb] (scalar loads, see TileWalker)
  size_t row0 = 0;              // (b * Hq) * nkb + kblock: table row of query head 0
  int nkb = 0, nqb = 0, bx = 1, sq = 1;
  int head = 0, hend = 0;
  int skip = 0, left = 0;       // entries still to skip / still to walk
  TileWalker walk{nullptr, 0, 1, 1};
  __device__ void init(const AttnArgs& a, int b, int kvh, int kblock, int first, int count) {
    sel_k = a.sel_k;
    cnt_k = (const_int_ptr)a.cnt_k;
    row0 = (size_t)b * a.Hq * a.nkb + kblock;
    nkb = a.nkb;
    nqb = a.nqb;
    bx = a.bx;
    sq = a.Sq;
    head = kvh * a.group;
    hend = head + a.group;
    skip = first;
    left = count;
    start();
  }
  __device__ void start() {
    const size_t row = row0 + (size_t)head * nkb;
    // The row's entry `skip` is read together with its count (it is the walk's first entry
    // whenever the row has more than `skip` entries; in bounds either way).
    const int first = ((const_int_ptr)sel_k)[row * nqb + min(skip, nqb - 1)];
    const int n = cnt_k[row];
    const int s0 = min(skip, n);
    const int take = min(n - s0, left);
    walk = TileWalker(sel_k + row * nqb + s0, take, bx, sq);
    if (s0 == skip && take > 0) walk.pj = first;
    skip -= s0;
    left -= take;
  }
  __device__ bool next(int& hd, int& tile, uint64_t& bits) {
    while (true) {
      if (walk.next(tile, bits)) {
        hd = head;
        return true;
      }
      if (++head >= hend || left <= 0) return false;
      start();
    }
  }
};

// Number of chunks the key block's concatenated table rows split into (1 when unchunked).
__device__ __forceinline__ int block_chunks(const AttnArgs& a, int b, int kvh, int kblock) {
  if (a.chunk <= 0) return 1;
  const size_t row0 = ((size_t)b * a.Hq + (size_t)kvh * a.group) * a.nkb + kblock;
  int e = 0;
  const_int_ptr cnt = (const_int_ptr)a.cnt_k;
  for (int h = 0; h < a.group; ++h) e += cnt[row0 + (size_t)h * a.nkb];
  return max(1, (e + a.chunk - 1) / a.chunk);
}

// Query blocks whose size is not a multiple of 32 rows: two selected blocks of one head can
// share a 32-row query half, whose dS bank entry the dK/dV workgroup visiting that half stores
// once with the rows of both.  A chunk boundary between two such blocks would have two
// workgroups store that entry, each with only its own rows, so a boundary x (an index into the
// key block's concatenated table rows; x >= the entry count is returned as is) moves past every
// entry that shares a half with the entry before it in the same head.  Both neighbouring chunks
// compute the same boundary, so the chunks still cover every entry exactly once.
__device__ __forceinline__ int block_chunk_edge(const AttnArgs& a, int b, int kvh, int kblock, int x) {
  const size_t row0 = ((size_t)b * a.Hq + (size_t)kvh * a.group) * a.nkb + kblock;
  const_int_ptr cnt = (const_int_ptr)a.cnt_k;
  int base = 0;
  for (int h = 0; h < a.group; ++h) {
    const size_t row = row0 + (size_t)h * a.nkb;
    const int n = cnt[row];
    if (x < base + n) {
      const_int_ptr sel = (const_int_ptr)a.sel_k + row * a.nqb;
      int i = x - base;
      while (i > 0 && i < n && (min(sel[i - 1] * a.bx + a.bx, a.Sq) - 1) >> 5 == (sel[i] * a.bx) >> 5) ++i;
      return base + i;
    }
    base += n;
  }
  return x;
}

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ------------------------------------------------------------------------ epilogue
// Stores a wave's 32 x 128 tile of fp32 accumulators (accumulator nb: lane 32 h + c holds
// column 32 nb + c of rows 8 (r / 4) + 4 h + r % 4) times `mul` to rows [0, nrows) of a
// row-major 16-bit tensor at `dst` (row stride 128), in 16-byte pieces.  The values go through
// a column-major LDS area of 128 columns x 36 elements (9216 B, 8-byte aligned, owned by the
// wave): each lane writes its four consecutive rows of a column as 8 bytes, then one
// ds_read_b64_tr_b16 gives each lane of a 16-lane group four consecutive columns of one row
// (lane 4 r + a addresses rows 4 a .. 4 a + 3 of column C + r; lane j receives row j of
// columns C .. C + 3), and two of them make the lane's 16 bytes.  Both passes touch 32
// distinct 8-byte bank pairs per half-wave (the 72-byte column pitch).
constexpr int EPI_PITCH = 36;                            // elements per staged column
constexpr int EPI_ELEMS = 128 * EPI_PITCH;               // 4608 elements = 9216 B per wave

template <class T>
__device__ __forceinline__ void store_tile_rows(const f32x16 (&acc)[4], float mul, uint16_t* dst, int nrows,
                                                uint16_t* stage, int lane) {
  const int c = lane & 31, h = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const u32x2 v = {T::pack2s(acc[nb][4 * q4], acc[nb][4 * q4 + 1], mul),
                       T::pack2s(acc[nb][4 * q4 + 2], acc[nb][4 * q4 + 3], mul)};
      st8(stage + (32 * nb + c) * EPI_PITCH + 8 * q4 + 4 * h, v);
    }
  }
  typedef short short4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) short4v* lds_ptr;
  const int g = (lane >> 4) & 3, j = lane & 15, rr = j >> 2, aa = j & 3;
  const int row = 16 * (g & 1) + j;                       // the row this lane stores
  const uint16_t* rd = stage + rr * EPI_PITCH + 16 * (g & 1) + 4 * aa;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int col = 8 * (2 * s + (g >> 1));
    const short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(rd + col * EPI_PITCH));
    const short4v y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(rd + (col + 4) * EPI_PITCH));
    const u32x2 xa = __builtin_bit_cast(u32x2, x), ya = __builtin_bit_cast(u32x2, y);
    if (row < nrows) st16(dst + (size_t)row * HD + col, (u32x4){xa[0], xa[1], ya[0], ya[1]});
  }
}

// ----------------------------------------------------------------------- dK / dV
// Workgroup = 2 NK waves owning 32 NK consecutive key rows (NK = 4, 128 rows, on the window
// path; NK = ceil(by / 32) on the block path, so a workgroup never straddles two key blocks).
// The K and V rows stay in LDS next to two Q/dO stages; with at most 256 registers per lane
// every SIMD holds two waves, so one wave's LDS reads, scalar work and softmax issue next to
// the other's matrix-core work.  Wave w works on key block kb = w % NK (32 rows) and on query
// half qh = w / NK (32 of the 64 rows) of every visited query tile:
//   S[q][kv]  = Q K^T          A = Q rows (stage),   B = K rows (LDS)
//   dP[q][kv] = dO V^T         A = dO rows (stage),  B = V rows (LDS)
//   P = exp2(S scale log2e - lse log2e), dS = P (dP - Delta)   (accumulator layout: lane
//       column = key row, registers = query rows 8 (r / 4) + 4 h + r % 4 of the half)
//   dV[kv][d] += P^T dO        A = P^T (repacked accumulator), B = dO columns (tr read)
//   dK[kv][d] += dS^T Q        A = dS^T,                       B = Q columns (tr read)
// Waves w and w + NK accumulate partial dK/dV of the same key rows over disjoint query rows;
// the two partial sums are added through LDS at the end, in a fixed order (bit-identical
// results run to run).
template <int NK, int NSTAGE = 2>
struct DkdvShape {
  static constexpr int NWAVES = 2 * NK;
  static constexpr int KV_TILES = NK <= 2 ? 1 : 2;        // 64-row tiles of K (and of V) in LDS
  static constexpr int KV_OFF = NSTAGE * 2 * TILE_ELEMS;  // elements: the (Q, dO) stages first
  static constexpr int ROWS_OFF = KV_OFF + 2 * KV_TILES * TILE_ELEMS;
  static constexpr int ROWS_END = ROWS_OFF + NSTAGE * 2 * 64 * 2;   // + (lse2, Delta) rows per stage
  static constexpr int smem_elems() { return ROWS_END; }
  static_assert(NK * 32 * 64 * 16 <= ROWS_OFF * 2, "partial-sum exchange must fit in the tile area");
};

// Stage count of the dK/dV pipeline.  Key tiles of at most 64 rows (block path with small
// key blocks; narrow windows): one stage, so that two workgroups share a compute unit (two
// waves per SIMD; the loads of one workgroup are hidden behind the other's matrix-core work,
// and so are the prologue and epilogue of workgroups that walk only a few tiles).  128-row
// key tiles: two stages (the next tile's loads are issued while the current one is computed).
template <int MASK, int NK>
constexpr int dkdv_stages() { return NK <= 2 ? 1 : 2; }
// Waves per SIMD the dK/dV kernel's register budget is sized for (the second argument of
// __launch_bounds__ on this target): two for the one-stage variant (at most 256 registers per
// lane); the eight-wave workgroups of the other variants imply two by themselves.
template <int MASK, int NK>
constexpr int dkdv_waves_per_simd() { return dkdv_stages<MASK, NK>() == 1 ? 2 : 1; }

template <class T, int MASK, int NK, bool DS = false>
__device__ __forceinline__ void dkdv_tile(const AttnArgs& a, int b, int kvh, int c0, int kv_end, int kblock,
                                          uint16_t* smem, int chunk = 0, bool partial = false, int hoff = 0,
                                          int hcnt = 0) {
  constexpr int NSTAGE = dkdv_stages<MASK, NK>();
  using Sh = DkdvShape<NK, NSTAGE>;
  constexpr int NWV = Sh::NWAVES;
  constexpr int BC = 32 * NK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, h = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int kb = wu % NK, qh = wu / NK;
  uint16_t* stages = smem;
  uint16_t* kvs = smem + Sh::KV_OFF;
  float* sld = reinterpret_cast<float*>(smem + Sh::ROWS_OFF);
  const uint32_t stages_lds = __builtin_amdgcn_readfirstlane(lds_addr(stages));
  const uint32_t kvs_lds = __builtin_amdgcn_readfirstlane(lds_addr(kvs));
  const uint32_t sld_lds = __builtin_amdgcn_readfirstlane(lds_addr(sld));
  const SeqRows qs = seq_rows(a, b, a.Hq, a.Sq), ks = seq_rows(a, b, a.Hkv, a.Skv);
  const int sq = qs.len, skv = ks.len;
  kv_end = min(kv_end, skv);
  if (c0 >= kv_end) return;   // tile past the end of a shorter packed sequence (uniform)
  const size_t kvrow0 = ks.base + (size_t)kvh * ks.head_stride;
  const uint16_t* Kp = (const uint16_t*)a.k + kvrow0 * HD;
  const uint16_t* Vp = (const uint16_t*)a.v + kvrow0 * HD;
  const int sq_pad = (a.Sq + 63) & ~63;

  // K and V of rows [c0, c0 + 64 KV_TILES) into LDS (rows past the end clamped; never stored).
#pragma unroll
  for (int t = 0; t < Sh::KV_TILES; ++t) {
    tile_load_async<NWV>(kvs_lds + (uint32_t)(t * TILE_BYTES), Kp, c0 + 64 * t, skv, wu, lane);
    tile_load_async<NWV>(kvs_lds + (uint32_t)((Sh::KV_TILES + t) * TILE_BYTES), Vp, c0 + 64 * t, skv, wu, lane);
  }

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    dk[nb] = zero16();
    dv[nb] = zero16();
  }

  WindowSourceDesc wsrc{};
  BlockGroupSource bsrc{};
  if constexpr (MASK == MASK_WINDOW) {
    const int qend = min(sq, c0 + BC + a.window - 1);
    const int tlo = c0 >> 6;
    const int thi = (qend + 63) >> 6;
    // Narrow windows (64-row key tiles, a few query tiles each): heads outer, so that the
    // workgroups of neighbouring key tiles (one XCD) read the same head's query tiles at the
    // same time and share them in L2; wide windows: tiles outer (comment above).
    // A head split takes query heads hoff .. hoff + hcnt - 1 of the group only.
    wsrc = WindowSourceDesc::make(kvh * a.group + hoff, hcnt > 0 ? hcnt : a.group, tlo, max(0, thi - tlo), NK <= 2);
  } else {
    if (a.chunk > 0) {
      int first = chunk * a.chunk, count = a.chunk;
      if (DS && (a.bx & 31) != 0) {
        first = block_chunk_edge(a, b, kvh, kblock, first);
        count = block_chunk_edge(a, b, kvh, kblock, (chunk + 1) * a.chunk) - first;
      }
      bsrc.init(a, b, kvh, kblock, first, count);
    } else {
      bsrc.init(a, b, kvh, kblock, 0, 0x7fffffff);
    }
  }
  auto fetch = [&](TileRef& r) -> bool {
    if constexpr (MASK == MASK_WINDOW) return wsrc.next(r.head, r.tile, r.bits);
    else return bsrc.next(r.head, r.tile, r.bits);
  };
  // Copies of a visited tile: the lane offsets inside a 64-row tile are fixed (computed once;
  // the swizzle is applied on the global side); a visit only moves the wave-uniform bases to
  // its head and tile, and only a tile reaching past the sequence end clamps its rows.
  constexpr int J = StageLoads<NWV>::J;
  const int head0 = kvh * a.group;   // every visited head is head0 + (0 .. group - 1)
  const uint16_t* q0 = (const uint16_t*)a.q + (qs.base + (size_t)head0 * qs.head_stride) * HD;
  const uint16_t* o0 = (const uint16_t*)a.dout + (qs.base + (size_t)head0 * qs.head_stride) * HD;
  const size_t hstride = qs.head_stride * HD;
  const float* l0 = a.lse2 + ((size_t)b * a.Hq + head0) * sq_pad;
  const float* d0 = a.delta + ((size_t)b * a.Hq + head0) * sq_pad;
  uint32_t voff[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int row = 4 * (wu + j * NWV) + (lane >> 4);
    voff[j] = 2u * (uint32_t)(row * HD + (((lane & 15) ^ swz(row)) << 3));
  }
  auto issue = [&](const TileRef& r, int stg) {
    const int dh = r.head - head0;
    const size_t off = (size_t)dh * hstride + (size_t)r.tile * (64 * HD);
    const uint16_t* qb = q0 + off;
    const uint16_t* ob = o0 + off;
    const uint32_t dst = stages_lds + (uint32_t)(stg * STAGE_BYTES);
    if (r.tile * 64 + 64 <= sq) {
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (StageLoads<NWV>::exists(j, wu))
          dma16(qb, voff[j], __builtin_amdgcn_readfirstlane(dst + (uint32_t)((wu + j * NWV) * 1024)));
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (StageLoads<NWV>::exists(j, wu))
          dma16(ob, voff[j], __builtin_amdgcn_readfirstlane(dst + (uint32_t)(TILE_BYTES + (wu + j * NWV) * 1024)));
    } else {
      const int last = sq - 1 - r.tile * 64;   // last row of the tile inside the sequence
      uint32_t cl[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int row = 4 * (wu + j * NWV) + (lane >> 4);
        cl[j] = 2u * (uint32_t)(min(row, last) * HD + (((lane & 15) ^ swz(row)) << 3));
      }
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (StageLoads<NWV>::exists(j, wu))
          dma16(qb, cl[j], __builtin_amdgcn_readfirstlane(dst + (uint32_t)((wu + j * NWV) * 1024)));
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (StageLoads<NWV>::exists(j, wu))
          dma16(ob, cl[j], __builtin_amdgcn_readfirstlane(dst + (uint32_t)(TILE_BYTES + (wu + j * NWV) * 1024)));
    }
    const uint32_t rows = sld_lds + (uint32_t)(stg * 512);
    const size_t roff = (size_t)dh * sq_pad + r.tile * 64;
    if (wu == 0) row_load_async(rows, l0 + roff, lane);
    if (wu == NWV - 1) row_load_async(rows + 256, d0 + roff, lane);
  };

  // V is negated in LDS once it has landed (sign bit of every 16-bit element), right after
  // the first tile's barrier: dP is then accumulated as Delta + dO (-V)^T = Delta - dP,
  // starting from the staged Delta rows, and dS = P (dP - Delta) = -(P (Delta - dP)) costs no
  // subtraction.  The first tiles' loads go out together with K and V.
  auto negate_v = [&]() {
    u32x4* vt = reinterpret_cast<u32x4*>(kvs + Sh::KV_TILES * TILE_ELEMS);
    constexpr int NCH = Sh::KV_TILES * TILE_BYTES / 16;   // 16-byte chunks of V
    for (int ch = tid; ch < NCH; ch += NWV * 64) {
      u32x4 x = vt[ch];
      x ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      vt[ch] = x;
    }
  };

  const float sl2 = a.scale_log2;
  const int kj = c0 + 32 * kb + c;
  // Fragment offsets with the wave's blocks folded in, so every read takes a constant offset:
  // Q/dO rows and columns of query half qh (stage folded in as well, flipped every tile), and
  // K/V rows of key block kb (tile kb / 2, 32-row half kb % 2; V tiles follow the K tiles).
  FragOff fo(lane);
  FragOff fkv(lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    fo.row[i] += qh * 8192;
    fo.col[i] += qh * 8192;
    fkv.row[i] += (kb >> 1) * TILE_BYTES + (kb & 1) * 8192;
  }
  TileRef cur{};
  bool vcur = fetch(cur);
  if (vcur) issue(cur, 0);
  int it = 0;
  // Tiles where every (q, kv) of the workgroup is visible need no mask (rows past the
  // sequence end need none either: lse2 = +inf there; key columns past the end are never
  // stored).
  auto is_full = [&]() -> bool {
    if constexpr (MASK == MASK_WINDOW)
      return (cur.tile * 64 - (c0 + BC - 1) >= 0) && (cur.tile * 64 + 63 - c0 < a.window);
    else
      return cur.bits == ~0ull;
  };
  // One visit; the stage is a template constant (two stages: the loop alternates two copies).
  auto visit = [&](auto stc) {
    constexpr int stg = decltype(stc)::value;
      const bool masked = !is_full();
      // This tile's loads (and, first time round, K/V) landed; with two stages the other stage
      // is free once every wave has passed the barrier.
      wait_vmcnt<0>();
      __syncthreads();
      if (it == 0) {
        negate_v();
        __syncthreads();
      }
      const float* ld = sld + stg * 128 + qh * 32 + 4 * h;   // lse2 row; Delta row at +64
      // This tile's stage: a compile-time offset on every fragment read (the loop body exists
      // once per stage), so the lane offsets never change.
      const uint16_t* const sb = stages + stg * (STAGE_BYTES / 2);
      // The next tile.  One stage: found before this tile's LDS reads are issued (a table entry
      // read on the block path is a scalar load, whose wait would otherwise cover those reads as
      // well); two stages: found, and its loads issued, once the first reads are in flight.
      TileRef nxr{};
      bool vn = false;
      if constexpr (NSTAGE == 1) vn = fetch(nxr);

      // S = Q K^T and dP = dO V^T for this wave's 32 query rows x 32 key rows.
      typedef const __attribute__((address_space(3))) f32x4* lds_f32x4;
      f32x16 s, d;
      {
        // Delta of this wave's 32 query rows in accumulator order (register r = 4 g + e).
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 D4 = *(lds_f32x4)(ld + 64 + 8 * g);
  #pragma unroll
          for (int e = 0; e < 4; ++e) d[4 * g + e] = D4[e];
        }
      }
      u32x4 fq[2], fk[2], fd[2], fv[2];
      // Every operand is read one k-step (two MFMAs) before its MFMA; the loads of the next tile
      // are issued while the first reads are in flight.
      fq[0] = frag_row(sb, fo, 0, 0, 0);
      fk[0] = frag_row(kvs, fkv, 0, 0, 0);
      fd[0] = frag_row(sb, fo, 1, 0, 0);
      fv[0] = frag_row(kvs, fkv, Sh::KV_TILES, 0, 0);
      if constexpr (NSTAGE == 2) {
        vn = fetch(nxr);
        if (vn) issue(nxr, stg ^ 1);
      }
      MA_STEP();
      static_for<0, 8>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        if constexpr (ks + 1 < 8) {
          fq[(ks + 1) & 1] = frag_row(sb, fo, 0, ks + 1, 0);
          fk[(ks + 1) & 1] = frag_row(kvs, fkv, 0, ks + 1, 0);
        }
        s = T::mma(fq[ks & 1], fk[ks & 1], ks ? s : zero16());
        MA_STEP();
        if constexpr (ks + 1 < 8) {
          fd[(ks + 1) & 1] = frag_row(sb, fo, 1, ks + 1, 0);
          fv[(ks + 1) & 1] = frag_row(kvs, fkv, Sh::KV_TILES, ks + 1, 0);
        }
        d = T::mma(fd[ks & 1], fv[ks & 1], d);
        MA_STEP();
      });
      if (masked) {
        if constexpr (MASK == MASK_WINDOW) {
          const int qdiff = cur.tile * 64 + qh * 32 + 4 * h - kj;
          static_for<0, 16>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            constexpr int qo = 8 * (r / 4) + (r % 4);
            s[r] = ((unsigned)(qdiff + qo) < (unsigned)a.window) ? s[r] : -INFINITY;
          });
        } else {
          const uint64_t hb = cur.bits >> (qh * 32 + 4 * h);
          static_for<0, 16>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            constexpr int qo = 8 * (r / 4) + (r % 4);
            s[r] = ((hb >> qo) & 1ull) ? s[r] : -INFINITY;
          });
        }
      }
      MA_STEP();
      // log2 P = S scale log2e - lse log2e, in place.
      {
        f32x4 L[4];
  #pragma unroll
        for (int g = 0; g < 4; ++g) L[g] = *(lds_f32x4)(ld + 8 * g);
  #pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = fmaf(s[r], sl2, -L[r / 4][r % 4]);
      }
      // First dV/dK operands, read before the softmax rows that precede their MFMAs.
      u32x4 fb[2], fc[2];
      fb[0] = frag_col(sb, fo, 1, 0, 0);
      fc[0] = frag_col(sb, fo, 0, 0, 0);
      // P and dS enter the dV and dK products rounded to 16 bits.  Where some P of this wave's
      // 32 x 32 block exceeds 1/4, the rounding error of such large terms, summed over every
      // query row and head that attends strongly to one key, can approach the tolerance; those
      // blocks (rare: the first query rows of a sequence, sharply peaked rows) also add the
      // rounding residuals in a second product at the end of the tile (the page's compensated
      // hi + lo GEMM), which makes their P and dS exact to about 22 bits.  The test is a
      // ballot, uniform over the wave, so results stay deterministic.
      float lmax = s[0];
  #pragma unroll
      for (int r = 1; r < 16; ++r) lmax = fmaxf(lmax, s[r]);
      const bool comp = __builtin_amdgcn_ballot_w64(lmax > -2.0f) != 0;
      MA_STEP();
      // dS bank (window path): this wave's block, query block 2 tile + qh and key block
      // c0 / 32 + kb, is stored when it holds a visible pair (the bank's band), as this wave
      // holds it: the two A operands of the dK product, stored as soon as they are packed, so
      // that the stores complete under this tile's dV/dK MFMAs (stores count in vmcnt, which
      // the next tile's first wait drains).  Non-temporal: the bank is read once, by the dQ
      // kernel, and should not displace the query tiles the other workgroups still read.
      bool ds_live = false;   // wave-uniform
      bool ds_edge = false;   // wave-uniform: the block reaches past the last key row
      u32x4* ds_dst = nullptr;
      if constexpr (MASK == MASK_BLOCK && DS) {
        // Block path: entry (head, qa, ka) of the grid of 32-row query halves and key
        // sub-blocks, ka = kblock NK + kb (the 32 key rows c0 + 32 kb .. of this mask block's
        // workgroup; the global 32-row key block when by is a multiple of 32), stored when some
        // of its query rows are selected (unselected rows hold exact zeros); key columns past
        // the block's last row (the next block's, or past the end) are stored as zeros.
        const int qa = 2 * cur.tile + qh, ka = kblock * NK + kb;
        ds_live = ((cur.bits >> (32 * qh)) & 0xffffffffull) != 0 && c0 + 32 * kb < kv_end;
        ds_edge = c0 + 32 * kb + 32 > kv_end;
        const long long blk = ((long long)b * a.Hq + cur.head) * a.ds_blocks + (qa * a.ds_nka + ka);
        ds_dst = reinterpret_cast<u32x4*>(a.ds_bank + (ds_live ? blk : 0) * 1024) + lane;
      }
      if constexpr (MASK == MASK_WINDOW && DS) {
        const int qa = 2 * cur.tile + qh, kbk = (c0 >> 5) + kb;
        ds_live = kbk <= qa && qa - a.ds_kb <= kbk && qa * 32 < sq;
        // Entry within the head in 32-bit arithmetic (the launcher keeps a head's bank below
        // 2^30 blocks), the head's base in 64-bit.
        const int off = band_offset32(qa, a.ds_kb) + kbk - max(0, qa - a.ds_kb);
        const long long blk = ((long long)b * a.Hq + cur.head) * a.ds_blocks + off;
        ds_dst = reinterpret_cast<u32x4*>(a.ds_bank + (ds_live ? blk : 0) * 1024) + lane;
      }
      // Rows 0-7 feed the first four dV/dK k-step pairs and are done up front; rows 8-15 are
      // done one per MFMA between those eight MFMAs (with a dS bank, all sixteen up front, so
      // both bank stores go out before the dV/dK MFMAs and complete under them: the next tile's
      // first wait covers stores as well as loads).
      constexpr bool ROWS_UP_FRONT = DS;
      u32x4 pa[2], da[2];
      float pk = 0.f, dk2 = 0.f;
      auto srow = [&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const float v = fast_exp2(s[r]);
        const float dsv = -(v * d[r]);
        if constexpr ((r & 1) == 0) {
          pk = v;
          dk2 = dsv;
        } else {
          pa[r / 8][(r % 8) / 2] = T::pack2(pk, v);
          da[r / 8][(r % 8) / 2] = T::pack2(dk2, dsv);
        }
      };
      static_for<0, ROWS_UP_FRONT ? 16 : 8>(srow);
      if constexpr (ROWS_UP_FRONT) {
        if (MASK == MASK_BLOCK && ds_edge && kj >= kv_end) {
          // Key rows past the end: dS of these columns is garbage computed on clamped K rows;
          // zero it (it only feeds dK rows that are never stored, and the dQ product).
          da[0] = (u32x4){0u, 0u, 0u, 0u};
          da[1] = (u32x4){0u, 0u, 0u, 0u};
        }
        if (ds_live) {
          __builtin_nontemporal_store(da[0], ds_dst);
          __builtin_nontemporal_store(da[1], ds_dst + 64);
        }
      }
      // dV += P^T dO, dK += dS^T Q over this wave's 32 query rows.
      MA_STEP();
      static_for<0, 8>([&](auto jc) {
        constexpr int j = decltype(jc)::value, t = j / 4, nb = j % 4;
        if constexpr (j + 1 < 8) {
          fb[(j + 1) & 1] = frag_col(sb, fo, 1, (j + 1) / 4, (j + 1) % 4);
          fc[(j + 1) & 1] = frag_col(sb, fo, 0, (j + 1) / 4, (j + 1) % 4);
        }
        dv[nb] = T::mma(pa[t], fb[j & 1], dv[nb]);
        if constexpr (j < 4 && !ROWS_UP_FRONT) srow(std::integral_constant<int, 8 + 2 * j>{});
        MA_STEP();
        dk[nb] = T::mma(da[t], fc[j & 1], dk[nb]);
        if constexpr (j < 4 && !ROWS_UP_FRONT) srow(std::integral_constant<int, 9 + 2 * j>{});
        MA_STEP();
      });
      if (comp) {
        // Residual products of this tile: S and dP again from the stage (still resident), the
        // same mask and exponent, then dV += (P - hi(P))^T dO and dK += (dS - hi(dS))^T Q.
        f32x16 s2 = zero16(), d2;
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 D4 = *(lds_f32x4)(ld + 64 + 8 * g);
  #pragma unroll
          for (int e = 0; e < 4; ++e) d2[4 * g + e] = D4[e];
        }
  #pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          s2 = T::mma(frag_row(sb, fo, 0, ks, 0), frag_row(kvs, fkv, 0, ks, 0), s2);
          d2 = T::mma(frag_row(sb, fo, 1, ks, 0), frag_row(kvs, fkv, Sh::KV_TILES, ks, 0), d2);
        }
        if (masked) {
          if constexpr (MASK == MASK_WINDOW) {
            const int qdiff = cur.tile * 64 + qh * 32 + 4 * h - kj;
            static_for<0, 16>([&](auto rc) {
              constexpr int r = decltype(rc)::value;
              constexpr int qo = 8 * (r / 4) + (r % 4);
              s2[r] = ((unsigned)(qdiff + qo) < (unsigned)a.window) ? s2[r] : -INFINITY;
            });
          } else {
            const uint64_t hb = cur.bits >> (qh * 32 + 4 * h);
            static_for<0, 16>([&](auto rc) {
              constexpr int r = decltype(rc)::value;
              constexpr int qo = 8 * (r / 4) + (r % 4);
              s2[r] = ((hb >> qo) & 1ull) ? s2[r] : -INFINITY;
            });
          }
        }
        u32x4 pl[2], dl[2];
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 L4 = *(lds_f32x4)(ld + 8 * g);
  #pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const int r = 4 * g + e;
            const float v0 = fast_exp2(fmaf(s2[r], sl2, -L4[e]));
            const float v1 = fast_exp2(fmaf(s2[r + 1], sl2, -L4[e + 1]));
            const float d0 = -(v0 * d2[r]), d1 = -(v1 * d2[r + 1]);
            const uint32_t ph = T::pack2(v0, v1), dh = T::pack2(d0, d1);
            pl[r / 8][(r % 8) / 2] = T::pack2(v0 - T::lo(ph), v1 - T::hi(ph));
            dl[r / 8][(r % 8) / 2] = T::pack2(d0 - T::lo(dh), d1 - T::hi(dh));
          }
        }
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = j / 4, nb = j % 4;
          dv[nb] = T::mma(pl[t], frag_col(sb, fo, 1, t, nb), dv[nb]);
          dk[nb] = T::mma(dl[t], frag_col(sb, fo, 0, t, nb), dk[nb]);
        }
      }
      if constexpr (NSTAGE == 1) {
        // One stage: every wave is done reading it before the next tile's loads overwrite it.
        __syncthreads();
        if (vn) issue(nxr, 0);
      }
      cur = nxr;
      vcur = vn;
      ++it;
  };
  while (vcur) {
    visit(std::integral_constant<int, 0>{});
    if constexpr (NSTAGE == 2) {
      if (!vcur) break;
      visit(std::integral_constant<int, 1>{});
    }
  }
  wait_vmcnt<0>();   // K/V loads when there was no tile at all
  __syncthreads();

  // Waves w + NK hand their partial dK sums to waves w, which hand their partial dV sums back
  // (16-byte chunks, lane-major; key block kb's 32 KiB area holds dK's at its start and dV's
  // at +16 KiB); then waves w store dK and waves w + NK store dV, each adding the other half's
  // sums to its own (floating-point addition commutes: the bits do not depend on who adds).
  f32x4* red = reinterpret_cast<f32x4*>(smem) + (size_t)kb * 32 * 64 + lane;
  f32x4* mine = red + (qh == 0 ? 16 * 64 : 0);    // where this wave's partials go
  f32x4* theirs = red + (qh == 0 ? 0 : 16 * 64);  // where the other half's arrive
  f32x16 (&keep)[4] = qh == 0 ? dk : dv;           // the sums this wave stores
  {
    const f32x16 (&give)[4] = qh == 0 ? dv : dk;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        mine[(nb * 4 + q4) * 64] =
            (f32x4){give[nb][4 * q4], give[nb][4 * q4 + 1], give[nb][4 * q4 + 2], give[nb][4 * q4 + 3]};
    }
  }
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 o4 = theirs[(nb * 4 + q4) * 64];
#pragma unroll
      for (int e = 0; e < 4; ++e) keep[nb][4 * q4 + e] += o4[e];
    }
  }
  const float mul = qh == 0 ? a.scale : 1.f;
  if (partial) {
    // One chunk of a key block whose selected query blocks span several workgroups: fp32
    // partial sums, added in chunk order and cast by the dK/dV reduce kernel.
    const int skv_pad = (a.Skv + 63) & ~63;
    const size_t slab = (size_t)a.B * a.Hkv * a.max_chunks * skv_pad * HD;
    float* pk = a.dkv_part + (((size_t)b * a.Hkv + kvh) * a.max_chunks + chunk) * skv_pad * HD + (qh ? slab : 0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = c0 + 32 * kb + 8 * (r / 4) + 4 * h + r % 4;
        if (row < kv_end) pk[(size_t)row * HD + nb * 32 + c] = keep[nb][r] * mul;
      }
    }
  } else {
    // 16-byte stores through the area the partials arrived in (this wave alone read it; LDS
    // operations of one wave complete in order, so each staging write follows those reads).
    uint16_t* stage = reinterpret_cast<uint16_t*>(theirs - lane);
    const size_t row0 = kvrow0 + c0 + 32 * kb;
    const int nrows = kv_end - (c0 + 32 * kb);
    store_tile_rows<T>(keep, mul, (uint16_t*)(qh == 0 ? a.dk : a.dv) + row0 * HD, nrows, stage, lane);
  }
}

template <class T, int MASK, int NK, bool DS = false>
__global__ __launch_bounds__(2 * NK * 64, (dkdv_waves_per_simd<MASK, NK>())) void dkdv_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[DkdvShape<NK, dkdv_stages<MASK, NK>()>::smem_elems()];
  if constexpr (MASK == MASK_WINDOW) {
    // dsink of every query head (the preprocess that wrote the partials ran before this
    // kernel), one wave per head in turn, before this workgroup's own tiles.
    if (a.dsink_out != nullptr && blockIdx.x == 0) {
      const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
      for (int h = w; h < a.Hq; h += 2 * NK)
        dsink_head_sum(a.dsink_part, a.dsink_out, a.B, a.Hq, a.dsink_nblk, h, threadIdx.x & 63);
    }
  }
  const int nbh = a.B * a.Hkv;
  const int wg = blockIdx.x;
  const int bh = wg % nbh, p = wg / nbh;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  if constexpr (MASK == MASK_WINDOW) {
    constexpr int BC = 32 * NK;
    {
      if (a.max_chunks > 1) {
        // Head split (dense sequences, too few key tiles to fill the GPU): slot p holds chunk
        // max_chunks - 1 - p / n_tiles of key tile p % n_tiles, so the extra chunks of the
        // heaviest tiles are dispatched first; slots past a tile's chunk count return at once.
        const int kt = p % a.n_tiles, c = a.max_chunks - 1 - p / a.n_tiles;
        const int nch = window_chunks(a.Sq, a.window, a.group, a.chunk, kt);
        if (c >= nch) return;   // uniform: no loads or barriers issued yet
        const int h0 = c * a.group / nch, h1 = (c + 1) * a.group / nch;
        dkdv_tile<T, MASK, NK, DS>(a, b, kvh, kt * BC, a.Skv, 0, smem, c, nch > 1, h0, h1 - h0);
        return;
      }
    }
    // Workgroups of one (batch, kv head) are consecutive modulo B*Hkv: with B*Hkv = 8 they
    // all land on one XCD and share its L2.  Tile p is paired with tile n - 1 - p (equal
    // total work) when the launcher sets `pair`; n counts the tiles of this sequence, so a
    // shorter packed sequence pairs within itself (workgroups past its middle have no work).
    const int nk = a.cu ? (seq_rows(a, b, a.Hkv, a.Skv).len + BC - 1) / BC : a.n_tiles;
    const int p2 = nk - 1 - p;
    if (a.pair && p > p2) return;
    dkdv_tile<T, MASK, NK, DS>(a, b, kvh, p * BC, a.Skv, 0, smem);
    if (a.pair && p2 != p) {
      __syncthreads();
      dkdv_tile<T, MASK, NK, DS>(a, b, kvh, p2 * BC, a.Skv, 0, smem);
    }
  } else {
    // p = (max_chunks - 1 - chunk) * nkb + key block: the last chunks, which only the most
    // selected key blocks have, are dispatched first, so those blocks do not finish last.
    const int kblock = p % a.nkb, chunk = a.max_chunks - 1 - p / a.nkb;
    const int nch = block_chunks(a, b, kvh, kblock);
    if (chunk >= nch) return;   // uniform: no loads or barriers issued yet
    const int c0 = kblock * a.by;
    dkdv_tile<T, MASK, NK, DS>(a, b, kvh, c0, min(c0 + a.by, a.Skv), kblock, smem, chunk, nch > 1);
  }
}

// --------------------------------------------------------------------------- dQ
// Workgroup = NW waves owning 32 NW consecutive query rows (wave w: rows r0 + 32 w ..),
// two workgroups per compute unit (two LDS stages of K/V tiles, 64 KiB per workgroup; at
// most 256 registers per lane).  Per visited key tile of 64 rows, in two 32-row key blocks:
//   S^T[kv][q]  = K Q^T       A = K rows (LDS),  B = Q rows (registers)
//   dP^T[kv][q] = V dO^T      A = V rows (LDS),  B = dO rows (registers)
//   (accumulator layout: lane column = query row, registers = key rows)
//   dQ[q][d] += dS K          A = dS (repacked accumulator), B = K columns (tr read)
// Order: S/dP of block 0; S/dP of block 1 with block 0's softmax rows in between; dQ of
// block 0 with block 1's softmax rows in between; dQ of block 1.
// `masked` (uniform) selects the tiles that need the visibility test; it is applied to the
// block's S in place (masked entries become -inf, so exp2 gives exactly 0) behind a scalar
// branch, which keeps one loop body for all tiles.
template <class T, int MASK>
__device__ __forceinline__ void dq_compute(f32x16* acc, const FragOff& fo, const u32x4* qf, const u32x4* of,
                                            const uint16_t* stages, float sl2, float l2, float dd, int kdiff,
                                            int window, uint64_t hbits, bool masked) {
  // dP^T accumulates from -Delta (every register of a lane holds the same query row), so it
  // ends holding dP - Delta.
  f32x16 negd;
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = -dd;
  f32x16 s[2], d[2];
  u32x4 da[2][2];
  float pk[2] = {0.f, 0.f};
  // S/dP of block mb (16 MFMAs, operands read two MFMAs ahead); `extra(j)` runs after
  // MFMA j (softmax rows of the other block).
  auto sdp = [&](auto mc, auto&& extra) {
    constexpr int mb = decltype(mc)::value;
    u32x4 fa[2];
    fa[0] = frag_row(stages, fo, 0, 0, mb);
    fa[1] = frag_row(stages, fo, 1, 0, mb);
    MA_STEP();
    static_for<0, 16>([&](auto jc) {
      constexpr int j = decltype(jc)::value, ks = j / 2;
      const u32x4 op = fa[j & 1];
      if constexpr (j + 2 < 16) fa[j & 1] = frag_row(stages, fo, j & 1, (j + 2) / 2, mb);
      if constexpr ((j & 1) == 0) s[mb] = T::mma(op, qf[ks], ks ? s[mb] : zero16());
      else d[mb] = T::mma(op, of[ks], ks ? d[mb] : negd);
      extra(jc);
      MA_STEP();
    });
    if (masked) {
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        constexpr int ko = mb * 32 + 8 * (r / 4) + (r % 4);
        bool vis;
        if constexpr (MASK == MASK_WINDOW) vis = (unsigned)(kdiff - ko) < (unsigned)window;
        else vis = (hbits >> ko) & 1ull;
        s[mb][r] = vis ? s[mb][r] : -INFINITY;
      });
    }
    MA_STEP();
  };
  // Softmax row r of block mb (this lane's query row, key row = register).
  auto srow = [&](auto mc, auto rc) {
    constexpr int mb = decltype(mc)::value, r = decltype(rc)::value;
    const float v = fast_exp2(fmaf(s[mb][r], sl2, -l2));
    const float ds = v * d[mb][r];
    if constexpr ((r & 1) == 0) pk[mb] = ds;
    else da[mb][r / 8][(r % 8) / 2] = T::pack2(pk[mb], ds);
  };
  // dQ of block mb (8 MFMAs, K columns read two ahead); `extra(j)` runs after MFMA j.
  auto dqb = [&](auto mc, auto&& extra) {
    constexpr int mb = decltype(mc)::value;
    u32x4 fb[2];
    fb[0] = frag_col(stages, fo, 0, 2 * mb, 0);
    fb[1] = frag_col(stages, fo, 0, 2 * mb, 1);
    MA_STEP();
    static_for<0, 8>([&](auto jc) {
      constexpr int j = decltype(jc)::value, t = j / 4, nb = j % 4;
      const u32x4 op = fb[j & 1];
      if constexpr (j + 2 < 8) fb[j & 1] = frag_col(stages, fo, 0, 2 * mb + (j + 2) / 4, (j + 2) % 4);
      acc[nb] = T::mma(da[mb][t], op, acc[nb]);
      extra(jc);
      MA_STEP();
    });
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto none = [&](auto) {};
  // S/dP of block 0; S/dP of block 1 with block 0's softmax (one row per MFMA); dQ of block
  // 0 with block 1's softmax (two rows per MFMA); dQ of block 1.
  sdp(I0{}, none);
  sdp(I1{}, [&](auto jc) { srow(I0{}, jc); });
  dqb(I0{}, [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    srow(I1{}, std::integral_constant<int, 2 * j>{});
    srow(I1{}, std::integral_constant<int, 2 * j + 1>{});
  });
  dqb(I1{}, none);
}

// Stage count of the dQ pipeline: on the block path with query blocks of at most 64 rows one
// stage of K/V, so that four workgroups share a compute unit (two waves per SIMD); two stages
// elsewhere (two workgroups per compute unit).
template <int MASK, int NW>
constexpr int dq_stages() { return (MASK == MASK_BLOCK && NW <= 2) ? 1 : 2; }

template <class T, int MASK, int NW>
__device__ __forceinline__ void dq_tile(const AttnArgs& a, int b, int hq, int r0, int q_end, int qb,
                                         uint16_t* stages) {
  constexpr int NS = dq_stages<MASK, NW>();
  constexpr int BQ = 32 * NW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, h = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t stages_lds = __builtin_amdgcn_readfirstlane(lds_addr(stages));
  const SeqRows qs = seq_rows(a, b, a.Hq, a.Sq), ks = seq_rows(a, b, a.Hkv, a.Skv);
  const int sq = qs.len, skv = ks.len;
  q_end = min(q_end, sq);
  if (r0 >= q_end) return;   // tile past the end of a shorter packed sequence (uniform)
  const size_t qhead = (size_t)b * a.Hq + hq;
  const size_t qrow0 = qs.base + (size_t)hq * qs.head_stride;
  const int kvh = hq / a.group;
  const size_t kvrow0 = ks.base + (size_t)kvh * ks.head_stride;
  const uint16_t* Kp = (const uint16_t*)a.k + kvrow0 * HD;
  const uint16_t* Vp = (const uint16_t*)a.v + kvrow0 * HD;
  const int sq_pad = (a.Sq + 63) & ~63;

  const int qi = r0 + 32 * w + c;
  const int qr = min(qi, sq - 1);
  const uint16_t* Qp = (const uint16_t*)a.q + (qrow0 + qr) * HD;
  const uint16_t* Op = (const uint16_t*)a.dout + (qrow0 + qr) * HD;
  u32x4 qf[8], of[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qf[ks] = ld16(Qp + ks * 16 + 8 * h);
    of[ks] = ld16(Op + ks * 16 + 8 * h);
  }
  const float l2 = a.lse2[qhead * sq_pad + qr];
  const float dd = a.delta[qhead * sq_pad + qr];
  f32x16 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = zero16();

  WindowSource wsrc{};
  BlockSource bsrc{TileWalker(nullptr, 0, 1, 1), 0};
  if constexpr (MASK == MASK_WINDOW) {
    const int lo = max(0, r0 - a.window + 1);
    const int hi = min(skv, r0 + BQ);
    const int tlo = lo >> 6, thi = (hi + 63) >> 6;
    wsrc = WindowSource::make(0, 1, tlo, max(0, thi - tlo));
  } else {
    const size_t row = qhead * a.nqb + qb;
    bsrc = BlockSource{TileWalker(a.sel_q + row * a.nkb, ((const_int_ptr)a.cnt_q)[row], a.by, a.Skv), 0};
  }
  auto fetch = [&](TileRef& r) -> bool {
    if constexpr (MASK == MASK_WINDOW) return wsrc.next(r.head, r.tile, r.bits);
    else return bsrc.next(r.head, r.tile, r.bits);
  };
  auto issue = [&](int t, int stg) {
    const uint32_t dst = stages_lds + (uint32_t)(stg * STAGE_BYTES);
    tile_load_async<NW>(dst, Kp, t * 64, skv, wu, lane);
    tile_load_async<NW>(dst + TILE_BYTES, Vp, t * 64, skv, wu, lane);
  };

  const float sl2 = a.scale_log2;
  FragOff fo(lane);
  TileRef cur{};
  bool vcur = fetch(cur);
  if (vcur) issue(cur.tile, 0);
  int it = 0;
  // Key tiles that need no mask: every (q, kv) inside the window for all rows of the
  // workgroup (query rows past the end are never stored; key rows past the end always
  // fail the window test since Sq == Skv on the window path).
  auto is_full = [&]() -> bool {
    if constexpr (MASK == MASK_WINDOW)
      return (r0 - (cur.tile * 64 + 63) >= 0) && (r0 + BQ - 1 - cur.tile * 64 < a.window);
    else
      return cur.bits == ~0ull;
  };
  auto step = [&]() -> bool {
    const bool masked = !is_full();
    // This tile's loads landed (every wave), and every wave is done with the other stage.
    wait_vmcnt<0>();
    __syncthreads();
    TileRef nx{};
    const bool vn = fetch(nx);
    if constexpr (NS == 2) {
      if (vn) issue(nx.tile, (it + 1) & 1);
    }
    const int kdiff = qi - cur.tile * 64 - 4 * h;
    const uint64_t hbits = h ? (cur.bits >> 4) : cur.bits;
    dq_compute<T, MASK>(acc, fo, qf, of, stages, sl2, l2, dd, kdiff, a.window, hbits, masked);
    if constexpr (NS == 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        fo.row[i] ^= STAGE_BYTES;
        fo.col[i] ^= STAGE_BYTES;
      }
    } else {
      // One stage: every wave is done reading it before the next tile's loads overwrite it.
      __syncthreads();
      if (vn) issue(nx.tile, 0);
    }
    ++it;
    cur = nx;
    return vn;
  };
  while (vcur) vcur = step();

  // Epilogue: rows r0 + 32 w .. of dQ, staged through this wave's part of the (now idle) K/V
  // stages once every wave is done with them.
  __syncthreads();
  store_tile_rows<T>(acc, a.scale, (uint16_t*)a.dq + (qrow0 + r0 + 32 * w) * HD, q_end - (r0 + 32 * w),
                     stages + w * EPI_ELEMS, lane);
}

template <class T, int MASK, int NW>
__global__ __launch_bounds__(NW * 64, 2) void dq_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t stages[dq_stages<MASK, NW>() * 2 * TILE_ELEMS];
  const int wg = blockIdx.x;
  if constexpr (MASK == MASK_WINDOW) {
    constexpr int BQ = 32 * NW;
    int b, hq, p;
    window_q_item(a, wg, b, hq, p);
    // Heaviest query tiles first; with `pair`, tile n - 1 - p also runs tile p, n counting
    // the tiles of this sequence.
    const int nq = a.cu ? (seq_rows(a, b, a.Hq, a.Sq).len + BQ - 1) / BQ : a.n_tiles;
    const int t1 = nq - 1 - p;
    if (t1 < 0 || (a.pair && p > t1)) return;
    dq_tile<T, MASK, NW>(a, b, hq, t1 * BQ, a.Sq, 0, stages);
    const int t2 = p;
    if (a.pair && t2 != t1) {
      __syncthreads();
      dq_tile<T, MASK, NW>(a, b, hq, t2 * BQ, a.Sq, 0, stages);
    }
  } else {
    const int nbh = a.B * a.Hq;
    const int bh = wg % nbh, p = wg / nbh;
    const int b = bh / a.Hq, hq = bh % a.Hq;
    const int r0 = p * a.bx;
    dq_tile<T, MASK, NW>(a, b, hq, r0, min(r0 + a.bx, a.Sq), p, stages);
  }
}

// ------------------------------------------------------------------- dQ from the dS bank
// Window path with a dS bank: dQ[q][d] = scale sum_k dS[q][k] K[k][d], one GEMM per live
// 32 x 32 block, summed over the key blocks in ascending order (fixed, so results are
// bit-identical run to run).  Workgroup = NW waves owning 32 NW consecutive query rows (wave w:
// query block r0 / 32 + w).  Per 64-row key tile, one LDS stage holds the key tile and the two
// dS blocks of every wave, all copied straight from HBM (LDS DMA), one tile ahead with four
// waves (two workgroups per compute unit) and two tiles ahead with eight (wide windows: one
// workgroup of 256 query rows per compute unit, three stages, twice the bytes in flight per
// compute unit and each key tile shared by twice the rows).
// No softmax and no masking: masked entries of a stored block are exact zeros.
//
// A bank block holds dS as the dK/dV kernel's wave had it (lane 32 x + k: key k, slots s =
// query 16 u + 8 (s / 4) + 4 x + s % 4 of 1 KiB unit u); the dQ product needs it the other way
// round (lane = query row, slots = keys).  The transpose is one ds_read_b64_tr_b16 pair per
// k-step: in a 16-lane group, lane 4 r + a addresses the 8 bytes holding the four queries
// 16 u + 4 a + (0..3) of key k0 + r, and lane j receives query 16 u + j of keys k0 + (0..3).
// The copies place logical 16-byte chunk L = 32 x + 4 m + r (m = key / 4) of unit u at slot
//   P = 16 (m / 2) + 8 (u ^ (m % 2)) + 4 x + r,
// so that the 32 lanes of each half-wave read 32 distinct 8-byte bank pairs.
template <int NW>
struct DqDsShape {
  static constexpr int STAGES = NW == 8 ? 3 : 2;
  static constexpr int STAGE_B = TILE_BYTES + NW * 4096;   // key tile, then 2 dS blocks per wave
  static constexpr int elems() { return STAGES * STAGE_B / 2; }
};

template <class T, int NW>
__device__ __forceinline__ void dq_ds_tile(const AttnArgs& a, int b, int hq, int r0, int q_end, uint16_t* smem) {
  using Sh = DqDsShape<NW>;
  constexpr int DQS_STAGES = Sh::STAGES;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, h = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const SeqRows qs = seq_rows(a, b, a.Hq, a.Sq), ks = seq_rows(a, b, a.Hkv, a.Skv);
  const int sq = qs.len, skv = ks.len;
  q_end = min(q_end, sq);
  if (r0 >= q_end) return;   // tile past the end of a shorter packed sequence (uniform)
  const size_t qrow0 = qs.base + (size_t)hq * qs.head_stride;
  const int kvh = hq / a.group;
  const uint16_t* Kp = (const uint16_t*)a.k + (ks.base + (size_t)kvh * ks.head_stride) * HD;

  // Key blocks of this wave (qa) and of the workgroup; 64-row key tiles [tlo, thi].
  const int a0 = r0 >> 5, qa = a0 + wu;
  const int a1 = min((q_end - 1) >> 5, a0 + NW - 1);
  const bool rows = qa <= a1;
  const int mlo = band_lo(qa, a.ds_kb), mhi = rows ? qa : -1;
  const int tlo = band_lo(a0, a.ds_kb) >> 1, thi = a1 >> 1;
  // The copies are issued by the first ISS waves only, wave w also copying the dS blocks of
  // waves w + ISS, w + 2 ISS, ... (eight waves: half of them issue; measured 3 % faster than
  // all eight, fewer waves with copies in flight per CU).
  constexpr int ISS = NW == 8 ? 4 : NW;
  constexpr int CPW = NW / ISS;   // waves whose dS blocks one issuing wave copies
  // Bank entry of key block kb of wave wv is bank[i] + kb * 1024 elements for kb in
  // [lo[i], hi[i]] (wv = wu + i ISS); waves without rows copy the head's first block (never
  // read).
  const uint16_t* bank[CPW];
  int lo[CPW], hi[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int qw = qa + i * ISS;
    const bool rw = qw <= a1;
    lo[i] = band_lo(qw, a.ds_kb);
    hi[i] = rw ? qw : -1;
    bank[i] = a.ds_bank +
              (((long long)b * a.Hq + hq) * a.ds_blocks + (rw ? band_offset(qw, a.ds_kb) - lo[i] : 0)) * 1024;
  }

  // Copy sources: the lane filling slot P of unit u fetches logical chunk L(P, u).
  auto src_chunk = [&](int u) -> uint32_t {
    const int m = 2 * (lane >> 4) + (((lane >> 3) & 1) ^ u);
    return (uint32_t)(u * 1024 + (32 * ((lane >> 2) & 1) + 4 * m + (lane & 3)) * 16);
  };
  const uint32_t so0 = src_chunk(0), so1 = src_chunk(1);
  // Transposing reads: byte offset of this lane's 8 bytes for k-step 0 (first slot quad) of a
  // block; + 512 per k-step, + 256 for the second slot quad.
  const int g = (lane >> 4) & 1, ia = lane & 3, ir = (lane >> 2) & 3;
  const int dso = g * 1024 + 128 * (g ^ h) + 64 * (ia & 1) + 16 * ir + 8 * (ia >> 1);

  auto issue = [&](int t, int s) {
    if (wu >= ISS) return;
    const uint32_t st = smem_lds + (uint32_t)(s * Sh::STAGE_B);
    tile_load_async<ISS>(st, Kp, t * 64, skv, wu, lane);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int kb = hi[i] >= 0 ? min(max(2 * t + mb, lo[i]), hi[i]) : 0;
        const uint16_t* blk = bank[i] + (long long)kb * 1024;
        const uint32_t d = st + (uint32_t)(TILE_BYTES + (wu + i * ISS) * 4096 + mb * 2048);
        if constexpr (NW == 8) {   // bank blocks are read once (measured faster with three stages)
          dma16nt(blk, so0, __builtin_amdgcn_readfirstlane(d));
          dma16nt(blk, so1, __builtin_amdgcn_readfirstlane(d + 1024));
        } else {
          dma16(blk, so0, __builtin_amdgcn_readfirstlane(d));
          dma16(blk, so1, __builtin_amdgcn_readfirstlane(d + 1024));
        }
      }
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = zero16();
  FragOff fo(lane);
  typedef short short4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) short4v* lds_ptr;
  auto ds_frag = [&](const char* blk, int tt) -> u32x4 {
    const short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(blk + dso + 512 * tt));
    const short4v y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(blk + dso + 512 * tt + 256));
    const u32x2 xa = __builtin_bit_cast(u32x2, x), ya = __builtin_bit_cast(u32x2, y);
    return (u32x4){xa[0], xa[1], ya[0], ya[1]};
  };

  // Loads of the first DQS_STAGES - 1 tiles; then per tile: wait for its loads (the later
  // tiles' 2 * (16 / NW + 4) copies per wave may stay in flight), barrier, issue the loads of
  // the tile DQS_STAGES - 1 ahead into the stage freed by the barrier, multiply.
  constexpr int PER_TILE = 16 / ISS + 4 * CPW;   // copies per issuing wave per tile
  static_assert(16 % ISS == 0 && NW % ISS == 0, "copies must split evenly over the issuing waves");
#pragma unroll
  for (int j = 0; j < DQS_STAGES - 1; ++j)
    if (tlo + j <= thi) issue(tlo + j, j);
  int s = 0;
  for (int t = tlo; t <= thi; ++t) {
    const int ahead = min(thi - t, DQS_STAGES - 2);   // tiles after t already issued
    if constexpr (DQS_STAGES == 2) {
      wait_vmcnt<0>();
    } else {
      if (ahead <= 0) wait_vmcnt<0>();
      else if (ahead == 1) wait_vmcnt<PER_TILE>();
      else wait_vmcnt<2 * PER_TILE>();
    }
    __syncthreads();
    if (t + DQS_STAGES - 1 <= thi) issue(t + DQS_STAGES - 1, s == 0 ? DQS_STAGES - 1 : s - 1);
    const uint16_t* kt = smem + s * (Sh::STAGE_B / 2);
    const char* dsb = reinterpret_cast<const char*>(smem) + s * Sh::STAGE_B + TILE_BYTES + wu * 4096;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int kb = 2 * t + mb;
      if (kb >= mlo && kb <= mhi) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const u32x4 fa = ds_frag(dsb + mb * 2048, tt);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) acc[nb] = T::mma(fa, frag_col(kt, fo, 0, 2 * mb + tt, nb), acc[nb]);
        }
      }
    }
    s = s == DQS_STAGES - 1 ? 0 : s + 1;
  }

  // Epilogue: rows r0 + 32 w .. of dQ, staged through this wave's part of the (now idle)
  // stages once every wave is done with them.
  __syncthreads();
  store_tile_rows<T>(acc, a.scale, (uint16_t*)a.dq + (qrow0 + r0 + 32 * w) * HD, q_end - (r0 + 32 * w),
                     smem + w * EPI_ELEMS, lane);
}

template <class T, int NW>
__global__ __launch_bounds__(NW * 64, 2) void dq_ds_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[DqDsShape<NW>::elems()];
  constexpr int BQ = 32 * NW;
  int b, hq, p;
  window_q_item(a, blockIdx.x, b, hq, p);
  // Heaviest query tiles first; with `pair`, tile n - 1 - p also runs tile p (n counting the
  // tiles of this sequence).
  const int nq = a.cu ? (seq_rows(a, b, a.Hq, a.Sq).len + BQ - 1) / BQ : a.n_tiles;
  const int t1 = nq - 1 - p;
  if (t1 < 0 || (a.pair && p > t1)) return;
  dq_ds_tile<T, NW>(a, b, hq, t1 * BQ, a.Sq, smem);
  if (a.pair && p != t1) {
    __syncthreads();
    dq_ds_tile<T, NW>(a, b, hq, p * BQ, a.Sq, smem);
  }
}

// Block path with a dS bank (block sizes multiples of 32): dQ of query block qb (bx rows; NW =
// bx / 32 waves, wave w owning the 32-row query block qa = qb bx / 32 + w) from the bank.  The
// key tiles come from the query block's row of the q-major table (ascending, so the sum over
// key blocks has a fixed order); a selected mask block covers whole 32-row key blocks, so each
// 64-row tile's two 32-row halves are either selected (one GEMM each, dS copied from the bank)
// or skipped.  Stages as in dq_ds_tile (key tile + two dS blocks per wave, transposing reads).
template <class T, int NW>
__device__ __forceinline__ void dq_ds_block_tile(const AttnArgs& a, int b, int hq, int qb, uint16_t* smem) {
  constexpr int STAGE_B = TILE_BYTES + NW * 4096;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const SeqRows qs = seq_rows(a, b, a.Hq, a.Sq), ks = seq_rows(a, b, a.Hkv, a.Skv);
  const int sq = qs.len, skv = ks.len;
  const int r0 = qb * a.bx, q_end = min(r0 + a.bx, sq);
  const size_t qrow0 = qs.base + (size_t)hq * qs.head_stride;
  const int kvh = hq / a.group;
  const uint16_t* Kp = (const uint16_t*)a.k + (ks.base + (size_t)kvh * ks.head_stride) * HD;
  const int qa = (r0 >> 5) + wu;
  const bool rows = qa * 32 < q_end;
  const uint16_t* bank =
      a.ds_bank + (((long long)b * a.Hq + hq) * a.ds_blocks + (long long)(rows ? qa : 0) * a.ds_nka) * 1024;
  const size_t qhead = (size_t)b * a.Hq + hq;
  TileWalker walk(a.sel_q + (qhead * a.nqb + qb) * a.nkb, a.cnt_q[qhead * a.nqb + qb], a.by, a.Skv);

  auto src_chunk = [&](int u) -> uint32_t {
    const int m = 2 * (lane >> 4) + (((lane >> 3) & 1) ^ u);
    return (uint32_t)(u * 1024 + (32 * ((lane >> 2) & 1) + 4 * m + (lane & 3)) * 16);
  };
  const uint32_t so0 = src_chunk(0), so1 = src_chunk(1);
  const int g = (lane >> 4) & 1, ia = lane & 3, ir = (lane >> 2) & 3;
  const int dso = g * 1024 + 128 * (g ^ h) + 64 * (ia & 1) + 16 * ir + 8 * (ia >> 1);
  auto half_live = [](uint64_t bits, int mb) { return ((bits >> (32 * mb)) & 0xffffffffull) != 0; };
  auto issue = [&](const TileRef& r, int s) {
    const uint32_t st = smem_lds + (uint32_t)(s * STAGE_B);
    tile_load_async<NW>(st, Kp, r.tile * 64, skv, wu, lane);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (rows && half_live(r.bits, mb)) {
        const uint16_t* blk = bank + (long long)(2 * r.tile + mb) * 1024;
        const uint32_t d = st + (uint32_t)(TILE_BYTES + wu * 4096 + mb * 2048);
        // Bank blocks are read once: non-temporal (measured 2 % faster on bigbird).
        dma16nt(blk, so0, __builtin_amdgcn_readfirstlane(d));
        dma16nt(blk, so1, __builtin_amdgcn_readfirstlane(d + 1024));
      }
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = zero16();
  FragOff fo(lane);
  typedef short short4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) short4v* lds_ptr;
  auto ds_frag = [&](const char* blk, int tt) -> u32x4 {
    const short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(blk + dso + 512 * tt));
    const short4v y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(blk + dso + 512 * tt + 256));
    const u32x2 xa = __builtin_bit_cast(u32x2, x), ya = __builtin_bit_cast(u32x2, y);
    return (u32x4){xa[0], xa[1], ya[0], ya[1]};
  };

  TileRef cur{}, nx{};
  bool vcur = walk.next(cur.tile, cur.bits);
  if (vcur) issue(cur, 0);
  int s = 0;
  while (vcur) {
    wait_vmcnt<0>();   // this tile's copies (the next tile's go out after the barrier)
    __syncthreads();
    const bool vn = walk.next(nx.tile, nx.bits);
    if (vn) issue(nx, s ^ 1);
    const uint16_t* kt = smem + s * (STAGE_B / 2);
    const char* dsb = reinterpret_cast<const char*>(smem) + s * STAGE_B + TILE_BYTES + wu * 4096;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (rows && half_live(cur.bits, mb)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const u32x4 fa = ds_frag(dsb + mb * 2048, tt);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) acc[nb] = T::mma(fa, frag_col(kt, fo, 0, 2 * mb + tt, nb), acc[nb]);
        }
      }
    }
    s ^= 1;
    cur = nx;
    vcur = vn;
  }
  __syncthreads();
  store_tile_rows<T>(acc, a.scale, (uint16_t*)a.dq + (qrow0 + r0 + 32 * w) * HD, q_end - (r0 + 32 * w),
                     smem + w * EPI_ELEMS, lane);
}

template <class T, int NW>
__global__ __launch_bounds__(NW * 64, 2) void dq_ds_block_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (TILE_BYTES + NW * 4096) / 2];
  const int nbh = a.B * a.Hq;
  const int wg = blockIdx.x;
  const int bh = wg % nbh, qb = wg / nbh;
  dq_ds_block_tile<T, NW>(a, bh / a.Hq, bh % a.Hq, qb, smem);
}

// Block path with a dS bank when bx or by is not a multiple of 32 (the dK/dV kernel's 32-row
// query halves then straddle query blocks, and its key sub-blocks c0 + 32 kb are off the
// 32-row grid).  Every wave owns one 32-row query half qa (rows 32 qa ..) and works alone:
// it walks, in ascending order, the union of the key blocks selected by the (at most three)
// query blocks its rows fall in, and for each key block the sub-blocks that hold key rows,
// one GEMM per sub-block from its dS bank entry (qa, kb NK + j).  The entry exists exactly
// when one of those query blocks selects kb (the dK/dV kernel stored it then), and its rows
// of query blocks that do not select kb are exact zeros.
// The walk is latency-bound (a few dozen dependent sub-blocks per wave, little arithmetic
// each), so the copies go in granules of 16 keys, one MFMA k-step: 4 KiB of K rows and the
// 1 KiB of the dS entry those keys need, through a ring of DQU_SLOTS granule slots private to
// the wave (LDS DMA, vmcnt waits only: no barriers), DQU_SLOTS - 1 granules in flight.
// In a slot, K rows sit at 0 .. 4 KiB with the swizzle of a staged tile's first 16 rows (the
// swizzle repeats every 16 rows, so the k-step's fragments read as k-step 0), and the dS
// granule at 4 KiB: the 512 bytes of k-step tt of the entry's unit 0, then those of unit 1.
constexpr int DQU_SLOT_BYTES = 4096 + 1024;
constexpr int DQU_SLOTS = 5;
constexpr int DQU_WAVE_BYTES = DQU_SLOTS * DQU_SLOT_BYTES;   // 25 KiB per wave
constexpr int DQU_WAVES = 2;                                 // waves (query halves) per workgroup
static_assert(DQU_WAVE_BYTES >= EPI_ELEMS * 2, "the epilogue stages through the wave's slots");

// vmcnt wait for a count known only at run time (multiples of five, the copies per granule).
__device__ __forceinline__ void wait_vmcnt_granules(int pending) {
  static_assert(DQU_SLOTS == 5, "one case per granule count");
  switch (pending) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<5>(); break;
    case 2: wait_vmcnt<10>(); break;
    case 3: wait_vmcnt<15>(); break;
    default: wait_vmcnt<20>(); break;
  }
}

template <class T>
__device__ __forceinline__ void dq_ds_blocku_wave(const AttnArgs& a, int b, int hq, int qa, uint16_t* buf,
                                                  int lane) {
  const int h = lane >> 5;
  const SeqRows qs = seq_rows(a, b, a.Hq, a.Sq), ks = seq_rows(a, b, a.Hkv, a.Skv);
  const int sq = qs.len, skv = ks.len;
  const int q0 = qa * 32;
  if (q0 >= sq) return;   // wave-uniform; no barriers follow
  const uint32_t buf_lds = __builtin_amdgcn_readfirstlane(lds_addr(buf));
  const size_t qrow0 = qs.base + (size_t)hq * qs.head_stride;
  const int kvh = hq / a.group;
  const uint16_t* Kp = (const uint16_t*)a.k + (ks.base + (size_t)kvh * ks.head_stride) * HD;
  const uint16_t* bank =
      a.ds_bank + (((long long)b * a.Hq + hq) * a.ds_blocks + (long long)qa * a.ds_nka) * 1024;
  const int nks = (a.by + 31) >> 5;   // key sub-blocks per mask block

  // The query blocks of rows [q0, min(q0 + 32, sq)): at most three (bx >= 16).
  const size_t qhead = (size_t)b * a.Hq + hq;
  const int qb0 = q0 / a.bx, qb1 = min(a.nqb - 1, (min(q0 + 32, sq) - 1) / a.bx);
  const_int_ptr sel[3];
  int cnt[3], pos[3] = {0, 0, 0}, head[3];
  constexpr int kDone = 0x7fffffff;
  // head[i]: entry pos[i] of list i (kDone past its end).  A list's next entry is loaded when
  // its head is consumed and first used by the following merge, several granules later, so
  // the scalar loads stay off the wave's path (a row's entries past its count are in bounds:
  // the table pads every row to nkb entries, and the index is clamped to the row).
  auto entry = [&](int i) -> int { return pos[i] < cnt[i] ? sel[i][min(pos[i], a.nkb - 1)] : kDone; };
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int qb = min(qb0 + i, qb1);
    sel[i] = (const_int_ptr)a.sel_q + (qhead * a.nqb + qb) * a.nkb;
    cnt[i] = qb0 + i <= qb1 ? ((const_int_ptr)a.cnt_q)[qhead * a.nqb + qb] : 0;
    head[i] = entry(i);
  }
  // Next key block of the union (ascending; -1 when done).
  auto next_kb = [&]() -> int {
    const int m = min(head[0], min(head[1], head[2]));
    if (m == kDone) return -1;
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (head[i] == m) {
        ++pos[i];
        head[i] = entry(i);
      }
    return m;
  };

  // dS copy sources: the lane filling byte 16 l of a slot's dS granule (unit l / 32, k-step tt)
  // fetches the entry's 16-byte chunk that the sub-block layout places at slot 32 tt + l % 32
  // of that unit.
  auto ds_src = [&](int tt) -> uint32_t {
    const int u = lane >> 5, P = 32 * tt + (lane & 31);
    const int m = 2 * (P >> 4) + (((P >> 3) & 1) ^ u);
    return (uint32_t)(u * 1024 + (32 * ((P >> 2) & 1) + 4 * m + (P & 3)) * 16);
  };
  const uint32_t dsrc0 = ds_src(0), dsrc1 = ds_src(1);
  const int g = (lane >> 4) & 1, ia = lane & 3, ir = (lane >> 2) & 3;
  const int dso = 4096 + g * 512 + 128 * (g ^ h) + 64 * (ia & 1) + 16 * ir + 8 * (ia >> 1);
  // Key rows of a granule: unit u (four rows) per instruction, row 4 u + lane / 16 of the 16.
  uint32_t kcol[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 4 * u + (lane >> 4);
    kcol[u] = (uint32_t)((((lane & 15) ^ swz(row)) << 3));
  }
  // Granule cursor: key block kb, sub-block j, k-step tt (kb < 0: no granule left).
  int kb = next_kb(), j = 0, tt = 0;
  auto issue = [&](int slot) {
    const int row0 = kb * a.by + 32 * j + 16 * tt;
    const uint32_t d = buf_lds + (uint32_t)(slot * DQU_SLOT_BYTES);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int gr = min(row0 + 4 * u + (lane >> 4), skv - 1);
      dma16(Kp, 2u * ((uint32_t)gr * HD + kcol[u]), __builtin_amdgcn_readfirstlane(d + (uint32_t)(u * 1024)));
    }
    const uint16_t* blk = bank + (long long)(kb * nks + j) * 1024;
    dma16nt(blk, tt ? dsrc1 : dsrc0, __builtin_amdgcn_readfirstlane(d + 4096u));
    // Advance: the entry's second k-step if it holds key rows of the block (its dS columns are
    // zeros otherwise), else the next sub-block holding key rows, else the next key block of
    // the union.
    const int kend = min(kb * a.by + a.by, skv);
    if (tt == 0 && row0 + 16 < kend) {
      tt = 1;
    } else {
      tt = 0;
      ++j;
      if (j >= nks || kb * a.by + 32 * j >= kend) {
        kb = next_kb();
        j = 0;
      }
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = zero16();
  FragOff fo(lane);
  typedef short short4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) short4v* lds_ptr;

  int inflight = 0, slot_in = 0, slot_out = 0;
  while (inflight < DQU_SLOTS - 1 && kb >= 0) {
    issue(slot_in);
    slot_in = slot_in == DQU_SLOTS - 1 ? 0 : slot_in + 1;
    ++inflight;
  }
  while (inflight > 0) {
    if (kb >= 0) {
      // The slot refilled held the granule computed last: its LDS reads are done first.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(slot_in);
      slot_in = slot_in == DQU_SLOTS - 1 ? 0 : slot_in + 1;
      ++inflight;
    }
    wait_vmcnt_granules(inflight - 1);   // the oldest granule landed; the younger ones may fly
    const char* sb = reinterpret_cast<const char*>(buf) + slot_out * DQU_SLOT_BYTES;
    const short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(sb + dso));
    const short4v y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(sb + dso + 256));
    const u32x2 xa = __builtin_bit_cast(u32x2, x), ya = __builtin_bit_cast(u32x2, y);
    const u32x4 fa = (u32x4){xa[0], xa[1], ya[0], ya[1]};
    const uint16_t* kt = reinterpret_cast<const uint16_t*>(sb);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = T::mma(fa, frag_col(kt, fo, 0, 0, nb), acc[nb]);
    slot_out = slot_out == DQU_SLOTS - 1 ? 0 : slot_out + 1;
    --inflight;
  }
  // Epilogue through the wave's own slots (every copy landed, every read done).
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  store_tile_rows<T>(acc, a.scale, (uint16_t*)a.dq + (qrow0 + q0) * HD, min(32, sq - q0), buf, lane);
}

template <class T>
__global__ __launch_bounds__(DQU_WAVES * 64) void dq_ds_blocku_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[DQU_WAVES * DQU_WAVE_BYTES / 2];
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  // DQU_WAVES 32-row halves per workgroup.  Workgroups of one (batch, head) are consecutive
  // modulo B Hq, so with B Hq a multiple of 8 each lands on the XCD that holds its head's K
  // rows and bank blocks in L2.
  const int nbh = a.B * a.Hq;
  const int bh = blockIdx.x % nbh, t = blockIdx.x / nbh;
  dq_ds_blocku_wave<T>(a, bh / a.Hq, bh % a.Hq, DQU_WAVES * t + w, smem + w * (DQU_WAVE_BYTES / 2), lane);
}

// Launch of one (element type, mask kind, NW) variant: dK/dV with 2 NW waves (NW key blocks
// of 32 rows), dQ with NW waves (NW query blocks of 32 rows).
template <class T, int MASK, int NW>
inline void launch_dkdv_only(const AttnArgs& a, int grid, hipStream_t st) {
  if (a.ds_bank) {
    hipLaunchKernelGGL((dkdv_kernel<T, MASK, NW, true>), dim3(grid), dim3(2 * NW * 64), 0, st, a);
    return;
  }
  hipLaunchKernelGGL((dkdv_kernel<T, MASK, NW>), dim3(grid), dim3(2 * NW * 64), 0, st, a);
}

template <class T, int MASK, int NW>
inline void launch_dq_only(const AttnArgs& a, int grid, hipStream_t st) {
  if constexpr (MASK == MASK_WINDOW) {
    if (a.ds_bank) {
      if (a.dq_nw == 8)
        hipLaunchKernelGGL((dq_ds_kernel<T, 8>), dim3(grid), dim3(8 * 64), 0, st, a);
      else
        hipLaunchKernelGGL((dq_ds_kernel<T, NW>), dim3(grid), dim3(NW * 64), 0, st, a);
      return;
    }
  } else {
    if (a.ds_bank) {
      hipLaunchKernelGGL((dq_ds_block_kernel<T, NW>), dim3(grid), dim3(NW * 64), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((dq_kernel<T, MASK, NW>), dim3(grid), dim3(NW * 64), 0, st, a);
}

// Each variant is compiled in an object of its own (attn_bwd_variant.hip built once per
// variant), so the build of the large unrolled kernels runs in parallel.
template <class T, int MASK, int NW>
void launch_dkdv_variant(const AttnArgs& a, int grid, hipStream_t st);
template <class T, int MASK, int NW>
void launch_dq_variant(const AttnArgs& a, int grid, hipStream_t st);

}  // namespace ma
