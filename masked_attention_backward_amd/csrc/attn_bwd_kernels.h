// Attention backward kernels for gfx950: preprocess (Delta, dsink partials), a fixed-order
// dsink reduce, a key/value-tile-stationary dK/dV kernel and a query-tile-stationary dQ
// kernel.  Both main kernels recompute S = scale*Q K^T and P = exp(S - lse) tile by tile
// (the FlashAttention-style recompute of the five-GEMM backward: S, P, dV += P^T dO,
// dP = dO V^T, dS = P (dP - Delta), dK += dS^T Q, dQ += dS K), as described on the page
// "[Example] Add GQA Sink Backward BHSD ..." (commit of the 9->6 kernel revision: QK^T,
// softmax, dV+dP, dS, dK+dQ; commit of the 4->2 revision: Delta = sum(O*dO), five GEMMs,
// dSink) and on the page "knowledge(triton) ... #174" (BlockSparseAttentionGrad skeleton:
// delta, then dq over the q-major table, then dk/dv over the kv-major table).
//
// Design on CDNA4, differing from the pages' Ascend kernels:
//   * dK/dV accumulate in registers of the workgroup that owns the key tile, and dQ in
//     the workgroup that owns the query tile, so there are no atomics and no fp32
//     partial buffers: results are bit-identical run to run (the pages' single-kernel
//     revision accumulated dK/dV with fp32 atomics and a host-side cast).
//   * P and dS never leave registers: the accumulator tile of S^T (or S) is re-packed in
//     place as the A/B operand of the next MFMA, with the contraction index permuted to
//     match (see ma_device.h), and the other operand is read down the columns of the
//     staged tile with ds_read_b64_tr_b16.
//   * Q/dO (or K/V) tiles are double-buffered in LDS; the next tile's global loads are
//     issued before the current tile's MFMAs.
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

// Tiles [tlo, thi) from the last one down, each over the heads [head0, head0 + nheads).  The
// dK/dV workgroups of one kv head (all on one XCD) then read the same query tile at the same
// time wherever their live ranges overlap (for causal masks they all end at the last tile).
struct WindowSourceDesc {
  int head0, hend, tlo, tile, head;
  __device__ static WindowSourceDesc make(int head0, int nheads, int tlo, int nt) {
    return WindowSourceDesc{head0, head0 + nheads, tlo, tlo + nt - 1, head0};
  }
  __device__ bool next(int& hd, int& t, uint64_t& bits) {
    if (tile < tlo) return false;
    hd = head;
    t = tile;
    bits = 0;
    if (++head >= hend) {
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

// ----------------------------------------------------------------------- dK / dV
// Workgroup = NW waves owning 32*NW consecutive key rows (wave w: rows c0+32w .. +32).
// Per visited (query head, query tile of 64 rows), in two 32-row query blocks mb:
//   S[q][kv]  = Q K^T          A = Q rows (LDS),   B = K rows (registers)
//   dP[q][kv] = dO V^T         A = dO rows (LDS),  B = V rows (registers)
//   P = exp2(S*scale*log2e - lse*log2e), dS = P (dP - Delta)   (accumulator layout:
//       lane column = key row, registers = query rows)
//   dV[kv][d] += P^T dO        A = P^T (repacked accumulator), B = dO columns (tr read)
//   dK[kv][d] += dS^T Q        A = dS^T,                       B = Q columns (tr read)
// The instruction stream of one tile is a program of 64 slots, one MFMA each, separated
// by scheduling barriers (one wave per SIMD issues in order, so the work placed between
// two MFMAs has to fit in the 32 cycles the matrix core spends on one of them):
//   slots  0-15  S/dP of block 0            (slot 2k: S k-step k, slot 2k+1: dP k-step k)
//   slots 16-31  S/dP of block 1
//   slots 32-47  dV/dK of block 0           (slot 32+2j: dV, 32+2j+1: dK; j = 4 t4 + nb)
//   slots 48-63  dV/dK of block 1
// Every operand read from LDS is issued four slots before its MFMA.  The softmax of a
// block is done one accumulator row (register r) per slot, spread over the slots between
// the end of the block's S/dP and the first dV/dK slot that consumes the row's k-step
// (the row timetable below); lse2/Delta of each group of four rows are read from LDS
// three slots before the group's first row.  The global->LDS loads of the tile two ahead
// are spread over the slots as well.  At slot DKDV_SYNC_SLOT every wave waits for its own
// loads of the next tile and the workgroup meets at a barrier; the operand reads of the
// last DKDV_LA slots then already fetch the next tile's first fragments, so consecutive
// tiles run back to back.
template <class T, int NW>
struct DkdvCtx {
  u32x4 kf[8], vf[8];
  f32x16 dk[4], dv[4];
  u32x4 fr[4];                   // operand fragments in flight (carried from one tile to the next)
};

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Slot of the softmax of accumulator row r of block mb (block 0: rows on two of every
// three slots from 17; block 1: the two free slots left before 40, then one row per
// slot).  A row pair (r, r+1) is packed into the operands right after row r+1.
__host__ __device__ constexpr int dkdv_row_slot(int mb, int r) {
  return mb == 0 ? 17 + (3 * r) / 2 : (r == 0 ? 34 : r == 1 ? 37 : 38 + r);
}
constexpr int DKDV_LA = 4;        // LDS operand reads run this many slots ahead
constexpr int DKDV_LD_LEAD = 3;   // lse2/Delta reads run this many slots ahead of a group
constexpr int DKDV_SLOTS = 64;
constexpr int DKDV_SYNC_SLOT = DKDV_SLOTS - DKDV_LA;

// Operand of slot s of a tile: row fragments for S/dP, column fragments for dV/dK.
template <int s>
__device__ __forceinline__ u32x4 dkdv_frag(const uint16_t* stages, const FragOff& fo) {
  if constexpr (s < 32) return frag_row(stages, fo, s & 1, (s % 16) / 2, s / 16);
  else return frag_col(stages, fo, ((s - 32) & 1) ? 0 : 1, (s - 32) / 8, ((s - 32) % 8) / 2);
}

// Is slot `s` the one that issues load instruction i of NI (spread over the tile)?
__host__ __device__ constexpr bool dkdv_dma_at(int i, int ni, int s) { return ((i * 32) / ni) * 2 + 1 == s; }

// One tile: tile A of the stage = Q, tile B = dO.  `nx` issues the loads of the tile two
// ahead.  `ld` points at this stage's lse2 row (64 floats) followed by its Delta row.
// `fo` addresses this tile's stage, `fn` the next tile's (only its first DKDV_LA row
// fragments are read through it).
template <class T, int MASK, int NW, bool MASKED, class Next>
__device__ __forceinline__ void dkdv_compute(DkdvCtx<T, NW>& x, const FragOff& fo, const FragOff& fn,
                                             const uint16_t* stages, const float* ld, float sl2, int qdiff,
                                             int window, uint64_t hbits, const Next& nx) {
  constexpr int NI = Next::COUNT;
  constexpr int LA = DKDV_LA;
  constexpr int KW = 2 * tile_loads_min<NW>();
  f32x16 sacc[2], dacc[2];       // S and dP of blocks 0 and 1
  u32x4* fr = x.fr;              // operand fragments in flight
  u32x4 pa[2][2], da[2][2];      // P^T and dS^T operands: [block][k-step of 16 rows]
  f32x4 Lg[2][2], Dg[2][2];      // lse2 / Delta of row groups: [block][group parity]
  float pk[2], dk2[2];           // first row of a pair, per block

  static_for<0, DKDV_SLOTS>([&](auto sc) {
    constexpr int s = decltype(sc)::value;
    // The MFMA of this slot.
    if constexpr (s < 32) {
      constexpr int mb = s / 16, ks = (s % 16) / 2;
      if constexpr ((s & 1) == 0)
        sacc[mb] = T::mma(fr[s % LA], x.kf[ks], ks ? sacc[mb] : zero16());
      else
        dacc[mb] = T::mma(fr[s % LA], x.vf[ks], ks ? dacc[mb] : zero16());
    } else {
      constexpr int k = s - 32, j = k / 2, t4 = j / 4, nb = j % 4;
      if constexpr ((k & 1) == 0)
        x.dv[nb] = T::mma(pa[t4 / 2][t4 % 2], fr[s % LA], x.dv[nb]);
      else
        x.dk[nb] = T::mma(da[t4 / 2][t4 % 2], fr[s % LA], x.dk[nb]);
    }
    // Next tile's data complete in LDS (every wave's loads), previous readers done.
    if constexpr (s == DKDV_SYNC_SLOT) {
      wait_vmcnt<KW>();
      barrier_keep_reads();
    }
    // Operand read for slot s + LA (of the next tile past the end of this one).
    if constexpr (s + LA < DKDV_SLOTS) fr[(s + LA) % LA] = dkdv_frag<s + LA>(stages, fo);
    else fr[(s + LA) % LA] = dkdv_frag<s + LA - DKDV_SLOTS>(stages, fn);
    // lse2/Delta of a row group whose first row comes DKDV_LD_LEAD slots from now.
    static_for<0, 2>([&](auto mc) {
      constexpr int mb = decltype(mc)::value;
      static_for<0, 4>([&](auto gc) {
        constexpr int g4 = decltype(gc)::value;
        if constexpr (dkdv_row_slot(mb, 4 * g4) - DKDV_LD_LEAD == s) {
          // volatile keeps the reads in this slot (they would otherwise be moved next to
          // their first use and waited for there)
          typedef const volatile __attribute__((address_space(3))) f32x4* lds_f32x4;
          Lg[mb][g4 & 1] = *(lds_f32x4)(ld + mb * 32 + 8 * g4);
          Dg[mb][g4 & 1] = *(lds_f32x4)(ld + 64 + mb * 32 + 8 * g4);
        }
      });
    });
    // Softmax rows of this slot.
    static_for<0, 2>([&](auto mc) {
      constexpr int mb = decltype(mc)::value;
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        if constexpr (dkdv_row_slot(mb, r) == s) {
          constexpr int e = r % 4;
          const float L = Lg[mb][(r / 4) & 1][e];
          const float D = Dg[mb][(r / 4) & 1][e];
          float v = fast_exp2(fmaf(sacc[mb][r], sl2, -L));
          if constexpr (MASKED) {
            constexpr int qo = mb * 32 + 8 * (r / 4) + e;
            bool vis;
            if constexpr (MASK == MASK_WINDOW) vis = (unsigned)(qdiff + qo) < (unsigned)window;
            else vis = (hbits >> qo) & 1ull;
            v = vis ? v : 0.f;
          }
          const float d = v * (dacc[mb][r] - D);
          if constexpr ((r & 1) == 0) {
            pk[mb] = v;
            dk2[mb] = d;
          } else {
            pa[mb][r / 8][(r % 8) / 2] = T::pack2(pk[mb], v);
            da[mb][r / 8][(r % 8) / 2] = T::pack2(dk2[mb], d);
          }
        }
      });
    });
    // Global->LDS loads of the tile two ahead.
    static_for<0, NI>([&](auto ic) {
      if constexpr (dkdv_dma_at(decltype(ic)::value, NI, s)) nx.issue(decltype(ic)::value);
    });
    MA_STEP();
  });
}

// Loads of one dK/dV stage: instruction 0 = the lse2 row (wave 0) and the Delta row
// (wave NW-1), then the Q and dO tiles.
template <int NW>
struct DkdvNext {
  static constexpr int COUNT = 1 + 2 * StageLoads<NW>::J;
  StageLoads<NW> tiles;
  const float* lse2;
  const float* delta;
  uint32_t rows;                 // LDS byte address of this stage's lse2 row (Delta row follows)
  int w, lane;
  __device__ __forceinline__ void issue(int i) const {
    if (i == 0) {
      if (w == 0) row_load_async(rows, lse2, lane);
      if (w == NW - 1) row_load_async(rows + 256, delta, lane);
    } else {
      tiles.issue(i - 1, w);
    }
  }
};

template <class T, int MASK, int NW>
__device__ __forceinline__ void dkdv_tile(const AttnArgs& a, int b, int kvh, int c0, int kv_end, int kb,
                                          uint16_t* stages, float* sld) {
  constexpr int BC = 32 * NW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, h = lane >> 5;
  const size_t kvhead = (size_t)b * a.Hkv + kvh;
  const uint16_t* Kp = (const uint16_t*)a.k + kvhead * a.Skv * HD;
  const uint16_t* Vp = (const uint16_t*)a.v + kvhead * a.Skv * HD;
  const int sq_pad = (a.Sq + 63) & ~63;

  DkdvCtx<T, NW> x;
  // This lane's key row (clamped into the sequence; rows past the end are never stored).
  const int kr = min(c0 + 32 * w + c, a.Skv - 1);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    x.kf[ks] = ld16(Kp + (size_t)kr * HD + ks * 16 + 8 * h);
    x.vf[ks] = ld16(Vp + (size_t)kr * HD + ks * 16 + 8 * h);
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    x.dk[nb] = zero16();
    x.dv[nb] = zero16();
  }

  WindowSource wsrc{};
  BlockSource bsrc{TileWalker(nullptr, 0, 1, 1), 0};
  if constexpr (MASK == MASK_WINDOW) {
    const int qend = min(a.Sq, c0 + BC + a.window - 1);
    const int tlo = c0 >> 6;
    const int thi = (qend + 63) >> 6;
    wsrc = WindowSource::make(kvh * a.group, a.group, tlo, max(0, thi - tlo));
  } else {
    const size_t row = kvhead * a.nkb + kb;
    bsrc = BlockSource{TileWalker(a.sel_k + row * a.nqb, a.cnt_k[row], a.bx, a.Sq), kvh};
  }
  auto next = [&](int& hd, int& t, uint64_t& bits) -> bool {
    if constexpr (MASK == MASK_WINDOW) return wsrc.next(hd, t, bits);
    else return bsrc.next(hd, t, bits);
  };
  // Loads of tile (hd, t) into stage `stg`: Q -> tile A, dO -> tile B, lse2/Delta rows.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t stages_lds = __builtin_amdgcn_readfirstlane(lds_addr(stages));
  const uint32_t sld_lds = __builtin_amdgcn_readfirstlane(lds_addr(sld));
  DkdvNext<NW> nx;
  nx.w = wu;
  nx.lane = lane;
  auto prepare = [&](const TileRef& r, int stg) {
    const size_t qhead = (size_t)b * a.Hq + r.head;
    nx.tiles.prepare((const uint16_t*)a.q + qhead * a.Sq * HD, (const uint16_t*)a.dout + qhead * a.Sq * HD,
                     stages_lds + (uint32_t)(stg * STAGE_BYTES), r.tile * 64, a.Sq, wu, lane);
    nx.lse2 = a.lse2 + qhead * sq_pad + r.tile * 64;
    nx.delta = a.delta + qhead * sq_pad + r.tile * 64;
    nx.rows = sld_lds + (uint32_t)(stg * 512);
  };
  auto issue_all = [&](const TileRef& r, int stg) {
    prepare(r, stg);
#pragma unroll
    for (int i = 0; i < DkdvNext<NW>::COUNT; ++i) nx.issue(i);
  };

  const float sl2 = a.scale_log2;
  const int kj = c0 + 32 * w + c;
  FragOff fo(lane);
  constexpr int KW = 2 * tile_loads_min<NW>();   // Q + dO instructions per tile and wave (at least)
  auto fetch = [&](TileRef& r) -> bool { return next(r.head, r.tile, r.bits); };
  // Tiles i and i + 1 are in flight when tile i is computed; tile i + 2 is issued then.
  TileRef cur{}, nxt{};
  bool vcur = fetch(cur);
  if (vcur) issue_all(cur, gray_stage(0));
  bool vnxt = vcur && fetch(nxt);
  if (vnxt) issue_all(nxt, gray_stage(1));
  if (vcur) {
    // First tile's data complete and visible; its first operands are read here, later
    // tiles' at the end of the tile before them.
    if (vnxt) wait_vmcnt<KW>();
    else wait_vmcnt<0>();
    barrier_keep_reads();
    static_for<0, DKDV_LA>([&](auto sc) { x.fr[decltype(sc)::value] = dkdv_frag<decltype(sc)::value>(stages, fo); });
  }
  int it = 0;
  // Window tiles that need no mask: every (q, kv) of the pair lies inside the window.
  // Rows past the sequence end need none either (lse2 = +inf there), nor do key columns
  // past the end (never stored).
  auto is_full = [&]() -> bool {
    if constexpr (MASK == MASK_WINDOW)
      return (cur.tile * 64 - (c0 + BC - 1) >= 0) && (cur.tile * 64 + 63 - c0 < a.window);
    else
      return cur.bits == ~0ull;
  };
  auto step = [&](auto masked) -> bool {
    constexpr bool MASKED = decltype(masked)::value;
    // Tile `cur` is complete in LDS: the barrier at the sync slot of the previous tile (or
    // the one above for the first tile) ordered it.
    TileRef n2{};
    const bool v2 = vnxt && fetch(n2);
    // Without a tile two ahead the loads repeat the current one into the free stage, which
    // keeps the step free of branches; they are drained before the workgroup moves on.
    prepare(v2 ? n2 : cur, gray_stage(it + 2));
    const int qdiff = cur.tile * 64 + 4 * h - kj;
    const uint64_t hbits = h ? (cur.bits >> 4) : cur.bits;
    FragOff fn = fo;
    fn.advance(it);
    dkdv_compute<T, MASK, NW, MASKED>(x, fo, fn, stages, sld + gray_stage(it) * 128 + 4 * h, sl2, qdiff, a.window,
                                      hbits, nx);
    fo = fn;
    ++it;
    cur = nxt;
    vcur = vnxt;
    nxt = n2;
    vnxt = v2;
    return vcur;
  };
  run_tiles(vcur, step, is_full);
  wait_vmcnt<0>();

  // Epilogue: rows c0 + 32w + 8(r/4) + 4h + r%4, column nb*32 + c.
  uint16_t* dKp = (uint16_t*)a.dk + kvhead * a.Skv * HD;
  uint16_t* dVp = (uint16_t*)a.dv + kvhead * a.Skv * HD;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = c0 + 32 * w + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < kv_end) {
        dKp[(size_t)row * HD + nb * 32 + c] = T::one(x.dk[nb][r] * a.scale);
        dVp[(size_t)row * HD + nb * 32 + c] = T::one(x.dv[nb][r]);
      }
    }
  }
}

template <class T, int MASK, int NW>
__global__ __launch_bounds__(NW * 64) void dkdv_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t stages[NSTAGES * 2 * TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) float sld[NSTAGES * 128];
  const int nbh = a.B * a.Hkv;
  const int wg = blockIdx.x;
  const int bh = wg % nbh, p = wg / nbh;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  if constexpr (MASK == MASK_WINDOW) {
    constexpr int BC = 32 * NW;
    dkdv_tile<T, MASK, NW>(a, b, kvh, p * BC, a.Skv, 0, stages, sld);
    const int p2 = a.n_tiles - 1 - p;
    if (a.pair && p2 != p) {
      __syncthreads();
      dkdv_tile<T, MASK, NW>(a, b, kvh, p2 * BC, a.Skv, 0, stages, sld);
    }
  } else {
    const int c0 = p * a.by;
    dkdv_tile<T, MASK, NW>(a, b, kvh, c0, min(c0 + a.by, a.Skv), p, stages, sld);
  }
}

// --------------------------------------------------------------------------- dQ
// Workgroup = NW waves owning 32*NW consecutive query rows (wave w: rows r0+32w .. +32).
// Per visited key tile of 64 rows, in two 32-row key blocks mb:
//   S^T[kv][q]  = K Q^T       A = K rows (LDS),  B = Q rows (registers)
//   dP^T[kv][q] = V dO^T      A = V rows (LDS),  B = dO rows (registers); the accumulation
//                             starts from -Delta (the lane column is the query row, so
//                             every register of a lane has the same Delta) and therefore
//                             ends holding dP - Delta
//   dQ[q][d] += dS K          A = dS (repacked accumulator), B = K columns (tr read)
// The instruction stream of one tile is a program of 48 slots, one MFMA each:
//   slots  0-15  S/dP of block 0     (slot 2k: S k-step k, slot 2k+1: dP k-step k)
//   slots 16-31  S/dP of block 1
//   slots 32-47  dQ                  (slot 32 + 4 t4 + nb: key rows 16 t4 .. +16, columns 32 nb ..)
// Softmax rows of block 0 run one per slot from slot 17 (its first dQ slot is 32), those of
// block 1 two per slot from slot 33 (its first dQ slot is 40).  Every operand is read from LDS
// DQ_LA slots before its MFMA; at slot DQ_SYNC_SLOT each wave waits for its own loads of the
// next tile and the workgroup meets at a barrier, after which the reads for the last DQ_LA
// slots already fetch the next tile's first operands.  The global->LDS loads of the tile two
// ahead are spread over slots 1..40.
constexpr int DQ_LA = 4;
constexpr int DQ_SLOTS = 48;
constexpr int DQ_SYNC_SLOT = DQ_SLOTS - DQ_LA;

__host__ __device__ constexpr int dq_row_slot(int mb, int r) { return mb == 0 ? 17 + r : 33 + r / 2; }

// Is slot `s` the one that issues load instruction i of NI?
__host__ __device__ constexpr bool dq_dma_at(int i, int ni, int s) { return (i * 40) / ni + 1 == s; }

template <class T>
struct DqCtx {
  u32x4 qf[8], of[8];   // this lane's query row of Q and dO (B operands)
  f32x16 acc[4];        // dQ accumulators, columns 32 nb + c
  f32x16 negd;          // -Delta of this lane's query row in all 16 registers
  u32x4 fr[DQ_LA];      // operand fragments in flight (carried from one tile to the next)
};

// Operand of slot s of a tile: K / V rows for S / dP, K columns for dQ.
template <int s>
__device__ __forceinline__ u32x4 dq_frag(const uint16_t* stages, const FragOff& fo) {
  if constexpr (s < 32) return frag_row(stages, fo, s & 1, (s % 16) / 2, s / 16);
  else return frag_col(stages, fo, 0, (s - 32) / 4, (s - 32) % 4);
}

// One key tile (tile A of the stage = K, tile B = V).  `fo` addresses this tile's stage,
// `fn` the next tile's (only its first DQ_LA row fragments are read through it).
template <class T, int MASK, int NW, bool MASKED>
__device__ __forceinline__ void dq_compute(DqCtx<T>& x, const FragOff& fo, const FragOff& fn,
                                           const uint16_t* stages, float sl2, float l2, int kdiff, int window,
                                           uint64_t hbits, const StageLoads<NW>& nx, int w) {
  constexpr int NI = 2 * StageLoads<NW>::J;
  constexpr int KW = 2 * tile_loads_min<NW>();
  f32x16 sacc[2], dacc[2];    // S^T and dP^T - Delta of blocks 0 and 1
  u32x4 da[2][2];             // dS operands: [block][k-step of 16 key rows]
  float pk[2];                // first row of a pair, per block
  static_for<0, DQ_SLOTS>([&](auto sc) {
    constexpr int s = decltype(sc)::value;
    // The MFMA of this slot.
    if constexpr (s < 32) {
      constexpr int mb = s / 16, ks = (s % 16) / 2;
      if constexpr ((s & 1) == 0)
        sacc[mb] = T::mma(x.fr[s % DQ_LA], x.qf[ks], ks ? sacc[mb] : zero16());
      else
        dacc[mb] = T::mma(x.fr[s % DQ_LA], x.of[ks], ks ? dacc[mb] : x.negd);
    } else {
      constexpr int j = s - 32, t4 = j / 4, nb = j % 4;
      x.acc[nb] = T::mma(da[t4 / 2][t4 % 2], x.fr[s % DQ_LA], x.acc[nb]);
    }
    // Next tile's data complete in LDS (every wave's loads), previous readers done.
    if constexpr (s == DQ_SYNC_SLOT) {
      wait_vmcnt<KW>();
      barrier_keep_reads();
    }
    // Operand read for slot s + DQ_LA (of the next tile past the end of this one).
    if constexpr (s + DQ_LA < DQ_SLOTS) x.fr[(s + DQ_LA) % DQ_LA] = dq_frag<s + DQ_LA>(stages, fo);
    else x.fr[(s + DQ_LA) % DQ_LA] = dq_frag<s + DQ_LA - DQ_SLOTS>(stages, fn);
    // Softmax rows of this slot.
    static_for<0, 2>([&](auto mc) {
      constexpr int mb = decltype(mc)::value;
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        if constexpr (dq_row_slot(mb, r) == s) {
          float v = fast_exp2(fmaf(sacc[mb][r], sl2, -l2));
          if constexpr (MASKED) {
            constexpr int ko = mb * 32 + 8 * (r / 4) + (r % 4);
            bool vis;
            if constexpr (MASK == MASK_WINDOW) vis = (unsigned)(kdiff - ko) < (unsigned)window;
            else vis = (hbits >> ko) & 1ull;
            v = vis ? v : 0.f;
          }
          const float d = v * dacc[mb][r];
          if constexpr ((r & 1) == 0) pk[mb] = d;
          else da[mb][r / 8][(r % 8) / 2] = T::pack2(pk[mb], d);
        }
      });
    });
    // Global->LDS loads of the tile two ahead.
    static_for<0, NI>([&](auto ic) {
      if constexpr (dq_dma_at(decltype(ic)::value, NI, s)) nx.issue(decltype(ic)::value, w);
    });
    MA_STEP();
  });
}

template <class T, int MASK, int NW>
__device__ __forceinline__ void dq_tile(const AttnArgs& a, int b, int hq, int r0, int q_end, int qb,
                                        uint16_t* stages) {
  constexpr int BQ = 32 * NW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, h = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t stages_lds = __builtin_amdgcn_readfirstlane(lds_addr(stages));
  const size_t qhead = (size_t)b * a.Hq + hq;
  const int kvh = hq / a.group;
  const size_t kvhead = (size_t)b * a.Hkv + kvh;
  const uint16_t* Kp = (const uint16_t*)a.k + kvhead * a.Skv * HD;
  const uint16_t* Vp = (const uint16_t*)a.v + kvhead * a.Skv * HD;
  const int sq_pad = (a.Sq + 63) & ~63;

  DqCtx<T> x;
  const int qi = r0 + 32 * w + c;
  const int qr = min(qi, a.Sq - 1);
  const uint16_t* Qp = (const uint16_t*)a.q + (qhead * a.Sq + qr) * HD;
  const uint16_t* Op = (const uint16_t*)a.dout + (qhead * a.Sq + qr) * HD;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    x.qf[ks] = ld16(Qp + ks * 16 + 8 * h);
    x.of[ks] = ld16(Op + ks * 16 + 8 * h);
  }
  const float l2 = a.lse2[qhead * sq_pad + qr];
  const float nd = -a.delta[qhead * sq_pad + qr];
#pragma unroll
  for (int i = 0; i < 16; ++i) x.negd[i] = nd;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) x.acc[nb] = zero16();

  WindowSource wsrc{};
  BlockSource bsrc{TileWalker(nullptr, 0, 1, 1), 0};
  if constexpr (MASK == MASK_WINDOW) {
    const int lo = max(0, r0 - a.window + 1);
    const int hi = min(a.Skv, r0 + BQ);
    const int tlo = lo >> 6, thi = (hi + 63) >> 6;
    wsrc = WindowSource::make(0, 1, tlo, max(0, thi - tlo));
  } else {
    const size_t row = qhead * a.nqb + qb;
    bsrc = BlockSource{TileWalker(a.sel_q + row * a.nkb, a.cnt_q[row], a.by, a.Skv), 0};
  }
  auto next = [&](int& hd, int& t, uint64_t& bits) -> bool {
    if constexpr (MASK == MASK_WINDOW) return wsrc.next(hd, t, bits);
    else return bsrc.next(hd, t, bits);
  };
  StageLoads<NW> nx;
  auto prepare = [&](int t, int stg) {
    nx.prepare(Kp, Vp, stages_lds + (uint32_t)(stg * STAGE_BYTES), t * 64, a.Skv, wu, lane);
  };
  auto issue_all = [&](int t, int stg) {
    prepare(t, stg);
#pragma unroll
    for (int i = 0; i < 2 * StageLoads<NW>::J; ++i) nx.issue(i, wu);
  };

  const float sl2 = a.scale_log2;
  FragOff fo(lane);
  constexpr int KW = 2 * tile_loads_min<NW>();   // K + V instructions per tile and wave (at least)
  auto fetch = [&](TileRef& r) -> bool { return next(r.head, r.tile, r.bits); };
  // Tiles i and i + 1 are in flight when tile i is computed; tile i + 2 is issued then.
  TileRef cur{}, nxt{};
  bool vcur = fetch(cur);
  if (vcur) {
    issue_all(cur.tile, gray_stage(0));
    const bool vn = fetch(nxt);
    if (vn) issue_all(nxt.tile, gray_stage(1));
    if (vn) wait_vmcnt<KW>();
    else wait_vmcnt<0>();
    barrier_keep_reads();
    static_for<0, DQ_LA>([&](auto sc) { x.fr[decltype(sc)::value] = dq_frag<decltype(sc)::value>(stages, fo); });
    bool vnxt = vn;
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
    auto step = [&](auto masked) -> bool {
      constexpr bool MASKED = decltype(masked)::value;
      TileRef n2{};
      const bool v2 = vnxt && fetch(n2);
      // Without a tile two ahead the loads repeat the current one into the free stage, which
      // keeps the step free of branches; they are drained before the workgroup moves on.
      prepare(v2 ? n2.tile : cur.tile, gray_stage(it + 2));
      const int kdiff = qi - cur.tile * 64 - 4 * h;
      const uint64_t hbits = h ? (cur.bits >> 4) : cur.bits;
      FragOff fn = fo;
      fn.advance(it);
      dq_compute<T, MASK, NW, MASKED>(x, fo, fn, stages, sl2, l2, kdiff, a.window, hbits, nx, wu);
      fo = fn;
      ++it;
      cur = nxt;
      const bool vc = vnxt;
      nxt = n2;
      vnxt = v2;
      return vc;
    };
    run_tiles(true, step, is_full);
    wait_vmcnt<0>();
  }

  // Epilogue: rows r0 + 32w + 8(r/4) + 4h + r%4, column nb*32 + c.
  uint16_t* dQp = (uint16_t*)a.dq + qhead * a.Sq * HD;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + 32 * w + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < q_end) dQp[(size_t)row * HD + nb * 32 + c] = T::one(x.acc[nb][r] * a.scale);
    }
  }
}

template <class T, int MASK, int NW>
__global__ __launch_bounds__(NW * 64) void dq_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t stages[NSTAGES * 2 * TILE_ELEMS];
  const int wg = blockIdx.x;
  if constexpr (MASK == MASK_WINDOW) {
    constexpr int BQ = 32 * NW;
    // Work item = (batch, query head, tile pair p).  Consecutive workgroups go to the eight
    // XCDs in turn; when the (batch, kv head) pairs split evenly over them, XCD x serves the
    // kv heads x, x + 8, ..., so the query heads that stream the same K/V tiles share that
    // XCD's L2.  Lower p (heavier tiles) is dispatched first either way.
    int b, hq, p;
    const int nbk = a.B * a.Hkv;
    if ((nbk & 7) == 0) {
      const int xcd = wg & 7, idx = wg >> 3;
      const int per = (nbk >> 3) * a.group;   // query heads served by one XCD
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
    // Heaviest query tiles (most visible keys) first.
    const int t1 = a.n_tiles - 1 - p;
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

// ------------------------------------------------------------- dQ, two workgroups per CU
// The same products as dq_kernel (S^T = K Q^T, dP^T = V dO^T, dQ += dS K per 32-row key
// block), written for two resident workgroups per compute unit: two LDS stages (64 KiB per
// workgroup) and at most 256 registers per lane, so every SIMD holds two waves.  A wave
// issues at most one instruction per issue cycle; with two waves per SIMD the LDS reads,
// scalar work and softmax of one wave issue next to the matrix-core work of the other, and
// each wave's waits are covered by the other one.  Per tile and key block mb: S/dP (16
// MFMA), softmax of the block, dQ of the block (8 MFMA).
// `masked` (uniform) selects the tiles that need the visibility test; it is applied to the
// block's S in place (masked entries become -inf, so exp2 gives exactly 0) behind a scalar
// branch, which keeps one loop body for all tiles.
template <class T, int MASK>
__device__ __forceinline__ void dq2_compute(f32x16* acc, const FragOff& fo, const u32x4* qf, const u32x4* of,
                                            const uint16_t* stages, float sl2, float l2, float dd, int kdiff,
                                            int window, uint64_t hbits, bool masked) {
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
      else d[mb] = T::mma(op, of[ks], ks ? d[mb] : zero16());
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
    const float ds = v * (d[mb][r] - dd);
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

template <class T, int MASK, int NW>
__device__ __forceinline__ void dq2_tile(const AttnArgs& a, int b, int hq, int r0, int q_end, int qb,
                                         uint16_t* stages) {
  constexpr int BQ = 32 * NW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, h = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t stages_lds = __builtin_amdgcn_readfirstlane(lds_addr(stages));
  const size_t qhead = (size_t)b * a.Hq + hq;
  const int kvh = hq / a.group;
  const size_t kvhead = (size_t)b * a.Hkv + kvh;
  const uint16_t* Kp = (const uint16_t*)a.k + kvhead * a.Skv * HD;
  const uint16_t* Vp = (const uint16_t*)a.v + kvhead * a.Skv * HD;
  const int sq_pad = (a.Sq + 63) & ~63;

  const int qi = r0 + 32 * w + c;
  const int qr = min(qi, a.Sq - 1);
  const uint16_t* Qp = (const uint16_t*)a.q + (qhead * a.Sq + qr) * HD;
  const uint16_t* Op = (const uint16_t*)a.dout + (qhead * a.Sq + qr) * HD;
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
    const int hi = min(a.Skv, r0 + BQ);
    const int tlo = lo >> 6, thi = (hi + 63) >> 6;
    wsrc = WindowSource::make(0, 1, tlo, max(0, thi - tlo));
  } else {
    const size_t row = qhead * a.nqb + qb;
    bsrc = BlockSource{TileWalker(a.sel_q + row * a.nkb, a.cnt_q[row], a.by, a.Skv), 0};
  }
  auto fetch = [&](TileRef& r) -> bool {
    if constexpr (MASK == MASK_WINDOW) return wsrc.next(r.head, r.tile, r.bits);
    else return bsrc.next(r.head, r.tile, r.bits);
  };
  auto issue = [&](int t, int stg) {
    const uint32_t dst = stages_lds + (uint32_t)(stg * STAGE_BYTES);
    tile_load_async<NW>(dst, Kp, t * 64, a.Skv, wu, lane);
    tile_load_async<NW>(dst + TILE_BYTES, Vp, t * 64, a.Skv, wu, lane);
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
    if (vn) issue(nx.tile, (it + 1) & 1);
    const int kdiff = qi - cur.tile * 64 - 4 * h;
    const uint64_t hbits = h ? (cur.bits >> 4) : cur.bits;
    dq2_compute<T, MASK>(acc, fo, qf, of, stages, sl2, l2, dd, kdiff, a.window, hbits, masked);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fo.row[i] ^= STAGE_BYTES;
      fo.col[i] ^= STAGE_BYTES;
    }
    ++it;
    cur = nx;
    return vn;
  };
  while (vcur) vcur = step();

  // Epilogue: rows r0 + 32w + 8(r/4) + 4h + r%4, column nb*32 + c.
  uint16_t* dQp = (uint16_t*)a.dq + qhead * a.Sq * HD;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + 32 * w + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < q_end) dQp[(size_t)row * HD + nb * 32 + c] = T::one(acc[nb][r] * a.scale);
    }
  }
}

// Work item decode of the window-path dQ grid (batch, query head, tile pair p): see
// dq_kernel.
__device__ __forceinline__ void dq_window_item(const AttnArgs& a, int wg, int& b, int& hq, int& p) {
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

template <class T, int MASK, int NW>
__global__ __launch_bounds__(NW * 64, 2) void dq2_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t stages[2 * 2 * TILE_ELEMS];
  const int wg = blockIdx.x;
  if constexpr (MASK == MASK_WINDOW) {
    constexpr int BQ = 32 * NW;
    int b, hq, p;
    dq_window_item(a, wg, b, hq, p);
    const int t1 = a.n_tiles - 1 - p;
    dq2_tile<T, MASK, NW>(a, b, hq, t1 * BQ, a.Sq, 0, stages);
    const int t2 = p;
    if (a.pair && t2 != t1) {
      __syncthreads();
      dq2_tile<T, MASK, NW>(a, b, hq, t2 * BQ, a.Sq, 0, stages);
    }
  } else {
    const int nbh = a.B * a.Hq;
    const int bh = wg % nbh, p = wg / nbh;
    const int b = bh / a.Hq, hq = bh % a.Hq;
    const int r0 = p * a.bx;
    dq2_tile<T, MASK, NW>(a, b, hq, r0, min(r0 + a.bx, a.Sq), p, stages);
  }
}

// ------------------------------------------------------- dK / dV, two waves per SIMD
// The same products as dkdv_kernel (S = Q K^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q) for
// the window path, written for two waves per SIMD: a workgroup of 8 waves owns 128 key rows
// whose K and V tiles stay in LDS (64 KiB) instead of registers, next to two Q/dO stages
// (64 KiB), which leaves at most 256 registers per lane.  Wave w works on key block w % 4
// (32 rows) and on query half w / 4 (32 of the 64 rows) of every tile, so waves w and w + 4
// (same SIMD) accumulate partial dK/dV of the same key rows over disjoint query rows; the
// two partial sums are added through LDS at the end (a fixed order: bit-identical results).
// With two waves per SIMD one wave's LDS reads, scalar work and softmax issue next to the
// other's matrix-core work.
constexpr int DKDV8_NW = 8;
constexpr int DKDV8_KV_BYTES = 4 * TILE_BYTES;   // K rows 0-63, K rows 64-127, V rows 0-63, V rows 64-127

template <class T, int MASK>
__device__ __forceinline__ void dkdv8_tile(const AttnArgs& a, int b, int kvh, int c0, uint16_t* smem) {
  constexpr int BC = 128;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, h = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int kb = wu & 3, qh = wu >> 2;
  uint16_t* stages = smem;                                    // 2 stages x (Q tile, dO tile)
  uint16_t* kvs = smem + 2 * 2 * TILE_ELEMS;                  // K, V of the workgroup's key rows
  float* sld = reinterpret_cast<float*>(smem + 2 * 2 * TILE_ELEMS + 4 * TILE_ELEMS);   // 2 x (lse2, Delta)
  const uint32_t stages_lds = __builtin_amdgcn_readfirstlane(lds_addr(stages));
  const uint32_t kvs_lds = __builtin_amdgcn_readfirstlane(lds_addr(kvs));
  const uint32_t sld_lds = __builtin_amdgcn_readfirstlane(lds_addr(sld));
  const size_t kvhead = (size_t)b * a.Hkv + kvh;
  const uint16_t* Kp = (const uint16_t*)a.k + kvhead * a.Skv * HD;
  const uint16_t* Vp = (const uint16_t*)a.v + kvhead * a.Skv * HD;
  const int sq_pad = (a.Sq + 63) & ~63;

  // K and V of rows [c0, c0 + 128) into LDS (rows past the end clamped; never stored).
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    tile_load_async<DKDV8_NW>(kvs_lds + (uint32_t)(t * TILE_BYTES), Kp, c0 + 64 * t, a.Skv, wu, lane);
    tile_load_async<DKDV8_NW>(kvs_lds + (uint32_t)((2 + t) * TILE_BYTES), Vp, c0 + 64 * t, a.Skv, wu, lane);
  }

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    dk[nb] = zero16();
    dv[nb] = zero16();
  }

  WindowSourceDesc wsrc;
  {
    const int qend = min(a.Sq, c0 + BC + a.window - 1);
    const int tlo = c0 >> 6;
    const int thi = (qend + 63) >> 6;
    wsrc = WindowSourceDesc::make(kvh * a.group, a.group, tlo, max(0, thi - tlo));
  }
  auto fetch = [&](TileRef& r) -> bool { return wsrc.next(r.head, r.tile, r.bits); };
  StageLoads<DKDV8_NW> nx;
  auto issue = [&](const TileRef& r, int stg) {
    const size_t qhead = (size_t)b * a.Hq + r.head;
    nx.prepare((const uint16_t*)a.q + qhead * a.Sq * HD, (const uint16_t*)a.dout + qhead * a.Sq * HD,
               stages_lds + (uint32_t)(stg * STAGE_BYTES), r.tile * 64, a.Sq, wu, lane);
#pragma unroll
    for (int i = 0; i < 2 * StageLoads<DKDV8_NW>::J; ++i) nx.issue(i, wu);
    const uint32_t rows = sld_lds + (uint32_t)(stg * 512);
    if (wu == 0) row_load_async(rows, a.lse2 + qhead * sq_pad + r.tile * 64, lane);
    if (wu == DKDV8_NW - 1) row_load_async(rows + 256, a.delta + qhead * sq_pad + r.tile * 64, lane);
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
  // Tiles where every (q, kv) of the workgroup lies inside the window need no mask (rows
  // past the sequence end need none either: lse2 = +inf there; key columns past the end are
  // never stored).
  auto is_full = [&]() -> bool {
    return (cur.tile * 64 - (c0 + BC - 1) >= 0) && (cur.tile * 64 + 63 - c0 < a.window);
  };
  while (vcur) {
    const bool masked = !is_full();
    // This tile's loads (and, first time round, K/V) landed; the other stage is free.
    wait_vmcnt<0>();
    __syncthreads();
    TileRef nxr{};
    const bool vn = fetch(nxr);
    if (vn) issue(nxr, (it + 1) & 1);
    const int stg = it & 1;
    const float* ld = sld + stg * 128 + qh * 32 + 4 * h;   // lse2 row; Delta row at +64

    // S = Q K^T and dP = dO V^T for this wave's 32 query rows x 32 key rows.
    f32x16 s, d;
    u32x4 fq[2], fk[2], fd[2], fv[2];
    fq[0] = frag_row(stages, fo, 0, 0, 0);
    fk[0] = frag_row(kvs, fkv, 0, 0, 0);
    MA_STEP();
    static_for<0, 8>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      fd[ks & 1] = frag_row(stages, fo, 1, ks, 0);
      fv[ks & 1] = frag_row(kvs, fkv, 2, ks, 0);
      s = T::mma(fq[ks & 1], fk[ks & 1], ks ? s : zero16());
      MA_STEP();
      if constexpr (ks + 1 < 8) {
        fq[(ks + 1) & 1] = frag_row(stages, fo, 0, ks + 1, 0);
        fk[(ks + 1) & 1] = frag_row(kvs, fkv, 0, ks + 1, 0);
      }
      d = T::mma(fd[ks & 1], fv[ks & 1], ks ? d : zero16());
      MA_STEP();
    });
    if (masked) {
      const int qdiff = cur.tile * 64 + qh * 32 + 4 * h - kj;
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        constexpr int qo = 8 * (r / 4) + (r % 4);
        s[r] = ((unsigned)(qdiff + qo) < (unsigned)a.window) ? s[r] : -INFINITY;
      });
    }
    MA_STEP();
    // P = exp2(S scale log2e - lse log2e), dS = P (dP - Delta); accumulator rows are query
    // rows 8 (r / 4) + 4 h + r % 4 of this wave's half, the lane column is the key row.
    // Rows 0-7 feed the first four dV/dK k-step pairs and are done up front; rows 8-15 are
    // done one per MFMA between those eight MFMAs, so this wave keeps the matrix core busy
    // while it finishes its softmax.
    u32x4 pa[2], da[2];
    float pk = 0.f, dk2 = 0.f;
    typedef const __attribute__((address_space(3))) f32x4* lds_f32x4;
    f32x4 L[4], D[4];
    L[0] = *(lds_f32x4)(ld);
    D[0] = *(lds_f32x4)(ld + 64);
    L[1] = *(lds_f32x4)(ld + 8);
    D[1] = *(lds_f32x4)(ld + 72);
    L[2] = *(lds_f32x4)(ld + 16);
    D[2] = *(lds_f32x4)(ld + 80);
    L[3] = *(lds_f32x4)(ld + 24);
    D[3] = *(lds_f32x4)(ld + 88);
    auto srow = [&](auto rc) {
      constexpr int r = decltype(rc)::value, g = r / 4, e = r % 4;
      const float v = fast_exp2(fmaf(s[r], sl2, -L[g][e]));
      const float dsv = v * (d[r] - D[g][e]);
      if constexpr ((r & 1) == 0) {
        pk = v;
        dk2 = dsv;
      } else {
        pa[r / 8][(r % 8) / 2] = T::pack2(pk, v);
        da[r / 8][(r % 8) / 2] = T::pack2(dk2, dsv);
      }
    };
    static_for<0, 8>(srow);
    // dV += P^T dO, dK += dS^T Q over this wave's 32 query rows (k-steps 2 qh, 2 qh + 1).
    u32x4 fb[2], fc[2];
    fb[0] = frag_col(stages, fo, 1, 0, 0);
    fc[0] = frag_col(stages, fo, 0, 0, 0);
    MA_STEP();
    static_for<0, 8>([&](auto jc) {
      constexpr int j = decltype(jc)::value, t = j / 4, nb = j % 4;
      if constexpr (j + 1 < 8) {
        fb[(j + 1) & 1] = frag_col(stages, fo, 1, (j + 1) / 4, (j + 1) % 4);
        fc[(j + 1) & 1] = frag_col(stages, fo, 0, (j + 1) / 4, (j + 1) % 4);
      }
      dv[nb] = T::mma(pa[t], fb[j & 1], dv[nb]);
      if constexpr (j < 4) srow(std::integral_constant<int, 8 + 2 * j>{});
      MA_STEP();
      dk[nb] = T::mma(da[t], fc[j & 1], dk[nb]);
      if constexpr (j < 4) srow(std::integral_constant<int, 9 + 2 * j>{});
      MA_STEP();
    });
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fo.row[i] ^= STAGE_BYTES;
      fo.col[i] ^= STAGE_BYTES;
    }
    ++it;
    cur = nxr;
    vcur = vn;
  }
  wait_vmcnt<0>();   // K/V loads when there was no tile at all
  __syncthreads();

  // Partial sums of waves w + 4 into LDS (16-byte chunks, lane-major), added by waves w.
  f32x4* red = reinterpret_cast<f32x4*>(smem) + (size_t)kb * 32 * 64 + lane;
  if (qh == 1) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        red[(nb * 4 + q4) * 64] = (f32x4){dk[nb][4 * q4], dk[nb][4 * q4 + 1], dk[nb][4 * q4 + 2], dk[nb][4 * q4 + 3]};
        red[(16 + nb * 4 + q4) * 64] = (f32x4){dv[nb][4 * q4], dv[nb][4 * q4 + 1], dv[nb][4 * q4 + 2], dv[nb][4 * q4 + 3]};
      }
    }
  }
  __syncthreads();
  if (qh == 0) {
    uint16_t* dKp = (uint16_t*)a.dk + kvhead * a.Skv * HD;
    uint16_t* dVp = (uint16_t*)a.dv + kvhead * a.Skv * HD;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 pk4 = red[(nb * 4 + q4) * 64];
        const f32x4 pv4 = red[(16 + nb * 4 + q4) * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          const int row = c0 + 32 * kb + 8 * q4 + 4 * h + e;
          if (row < a.Skv) {
            dKp[(size_t)row * HD + nb * 32 + c] = T::one((dk[nb][r] + pk4[e]) * a.scale);
            dVp[(size_t)row * HD + nb * 32 + c] = T::one(dv[nb][r] + pv4[e]);
          }
        }
      }
    }
  }
}

template <class T, int MASK>
__global__ __launch_bounds__(DKDV8_NW * 64) void dkdv8_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE_ELEMS + 4 * TILE_ELEMS + 2 * 2 * 64 * 2];
  const int nbh = a.B * a.Hkv;
  const int wg = blockIdx.x;
  const int bh = wg % nbh, p = wg / nbh;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  dkdv8_tile<T, MASK>(a, b, kvh, p * 128, smem);
  const int p2 = a.n_tiles - 1 - p;
  if (a.pair && p2 != p) {
    __syncthreads();
    dkdv8_tile<T, MASK>(a, b, kvh, p2 * 128, smem);
  }
}

template <class T, int MASK, int NW>
inline void launch_dkdv_only(const AttnArgs& a, int grid, hipStream_t st) {
  if constexpr (MASK == MASK_WINDOW)
    hipLaunchKernelGGL((dkdv8_kernel<T, MASK>), dim3(grid), dim3(DKDV8_NW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((dkdv_kernel<T, MASK, NW>), dim3(grid), dim3(NW * 64), 0, st, a);
}

template <class T, int MASK, int NW>
inline void launch_dq_only(const AttnArgs& a, int grid, hipStream_t st) {
  if constexpr (MASK == MASK_WINDOW)
    hipLaunchKernelGGL((dq2_kernel<T, MASK, NW>), dim3(grid), dim3(NW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((dq_kernel<T, MASK, NW>), dim3(grid), dim3(NW * 64), 0, st, a);
}

// Launchers of one (element type, mask kind, waves per workgroup) variant.  Each variant is
// compiled in an object of its own (attn_bwd_variant.hip built once per variant), so the
// build of the large unrolled kernels runs in parallel.
template <class T, int MASK, int NW>
void launch_dkdv_variant(const AttnArgs& a, int grid, hipStream_t st);
template <class T, int MASK, int NW>
void launch_dq_variant(const AttnArgs& a, int grid, hipStream_t st);

}  // namespace ma
