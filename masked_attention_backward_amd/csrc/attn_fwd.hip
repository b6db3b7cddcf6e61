// Attention forward for gfx950 with a sink logit and a sliding causal window, or with a
// block mask: O and the natural-log lse that the backward consumes.  Page "[Example] Add
// GQA Sink Backward BHSD ..." ("Files Added": online softmax with an attention sink and a
// sliding-window mask; commit of the 4->2 revision: forward -> O, lse).
//
// Online softmax per query row, started from the sink: running max m = sink and running
// sum l = 1 (m = -inf, l = 0 without a sink), then every visible key tile rescales and
// accumulates.  lse = m + log(l) therefore includes the sink, and a row that sees
// nothing ends with O = 0, lse = -inf.
//
// Workgroup = NW waves owning 32*NW query rows, two workgroups per compute unit (two LDS
// stages of K/V tiles, 64 KiB; at most 256 registers per lane, so each SIMD holds two waves
// and one wave's softmax issues next to the other's MFMAs); per 64-row key tile:
//   S^T[kv][q] = K Q^T      A = K rows (LDS), B = Q rows (registers); lane column = query
//   O^T[d][q] += V^T P^T    A = V columns (tr read), B = P^T (repacked accumulator)
// Accumulating O transposed keeps each lane's registers on its own query row, so the
// rescale by exp(m_old - m_new) is one multiply per register with no data exchange.
#include "ma_launch.h"
#include "ma_tiles.h"

namespace ma {

template <class T, int MASK, int NW>
__device__ __forceinline__ void fwd_tile(const AttnArgs& a, int b, int hq, int r0, int q_end, int qb,
                                         uint16_t* stages) {
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

  const int qi = r0 + 32 * w + c;
  const int qr = min(qi, sq - 1);
  const uint16_t* Qp = (const uint16_t*)a.q + (qrow0 + qr) * HD;
  u32x4 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = ld16(Qp + ks * 16 + 8 * h);

  float m2 = -INFINITY, l = 0.f;   // running max (log2 domain) and sum
  if constexpr (MASK == MASK_WINDOW) {
    if (a.sink) {
      const float sk = a.sink[hq];
      if (sk > -INFINITY) {
        m2 = sk * LOG2E;
        l = 1.f;
      }
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = zero16();

  int tlo = 0, nt = 0;
  TileWalker walk(nullptr, 0, 1, 1);
  if constexpr (MASK == MASK_WINDOW) {
    const int lo = max(0, r0 - a.window + 1);
    const int hi = min(skv, r0 + BQ);
    tlo = lo >> 6;
    nt = max(0, ((hi + 63) >> 6) - tlo);
  } else {
    const size_t row = qhead * a.nqb + qb;
    walk = TileWalker(a.sel_q + row * a.nkb, ((const_int_ptr)a.cnt_q)[row], a.by, a.Skv);
  }
  int it = 0;
  auto next = [&](int& t, uint64_t& bits) -> bool {
    if constexpr (MASK == MASK_WINDOW) {
      if (it >= nt) return false;
      t = tlo + it++;
      bits = 0;
      return true;
    } else {
      return walk.next(t, bits);
    }
  };
  auto issue = [&](int t, int stg) {
    const uint32_t dst = stages_lds + (uint32_t)(stg * STAGE_BYTES);
    tile_load_async<NW>(dst, Kp, t * 64, skv, wu, lane);
    tile_load_async<NW>(dst + TILE_BYTES, Vp, t * 64, skv, wu, lane);
  };

  const float sl2 = a.scale_log2;
  FragOff fo(lane);
  auto fetch = [&](TileRef& r) -> bool { return next(r.tile, r.bits); };
  TileRef cur{};
  bool vcur = fetch(cur);
  if (vcur) issue(cur.tile, 0);
  int itx = 0;
  auto is_full = [&]() -> bool {
    if constexpr (MASK == MASK_WINDOW)
      return (r0 - (cur.tile * 64 + 63) >= 0) && (r0 + BQ - 1 - cur.tile * 64 < a.window);
    else
      return cur.bits == ~0ull;
  };
  auto step = [&]() -> bool {
    const bool masked = !is_full();
    const int t = cur.tile;
    const uint64_t bits = cur.bits;
    // This tile's loads landed (every wave), and every wave is done with the other stage.
    wait_vmcnt<0>();
    __syncthreads();
    TileRef n2{};
    const bool v2 = fetch(n2);
    if (v2) issue(n2.tile, (itx + 1) & 1);
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = T::mma(frag_row(stages, fo, 0, 0, mb), qf[0], zero16());
#pragma unroll
      for (int ks = 1; ks < 8; ++ks) s[mb] = T::mma(frag_row(stages, fo, 0, ks, mb), qf[ks], s[mb]);
    }
    const int kdiff = qi - t * 64 - 4 * h;
    const uint64_t hbits = h ? (bits >> 4) : bits;
    // Hidden entries become -inf, only on tiles that need the test (a uniform branch, which
    // keeps one loop body for all tiles).
    if (masked) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = mb * 32 + 8 * (r >> 2) + (r & 3);
          bool vis;
          if constexpr (MASK == MASK_WINDOW) vis = (unsigned)(kdiff - ko) < (unsigned)a.window;
          else vis = (hbits >> ko) & 1ull;
          s[mb][r] = vis ? s[mb][r] : -INFINITY;
        }
      }
    }
    // Running max in the log2 domain: the largest raw logit times the (positive) scale, which
    // rounds to the same value as the largest scaled logit.
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
    const float mnew = fmaxf(m2, mx);
    const float alpha = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mnew);
    // P = exp2(s scale - m), one fused multiply-add per logit.  A hidden logit (-inf) gives
    // exp2(-inf) = 0 exactly; a row whose max is still -inf has only hidden logits, and takes 0
    // as its offset so that no -inf - -inf arises.
    const float msub = (mnew == -INFINITY) ? 0.f : mnew;
    float rs = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[mb][r], sl2, -msub));
        s[mb][r] = p;
        rs += p;
      }
    }
    rs += __shfl_xor(rs, 32);
    l = l * alpha + rs;
    // The accumulators are rescaled only when some row's max grew (alpha = 1 exactly
    // otherwise; the test is a ballot, uniform over the wave).
    if (__builtin_amdgcn_ballot_w64(mnew != m2) != 0) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][r] *= alpha;
    }
    m2 = mnew;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const u32x4 pb = pack8<T>(s[t4 >> 1], 8 * (t4 & 1));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[nb] = T::mma(frag_col(stages, fo, 1, t4, nb), pb, acc[nb]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fo.row[i] ^= STAGE_BYTES;
      fo.col[i] ^= STAGE_BYTES;
    }
    ++itx;
    cur = n2;
    return v2;
  };
  while (vcur) vcur = step();

  // Epilogue: lane (c, h) holds O^T[d = nb*32 + 8(r/4) + 4h + r%4][q = qi].
  if (qi < q_end) {
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    uint16_t* Orow = (uint16_t*)a.out_o + (qrow0 + qi) * HD;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 v;
        v[0] = T::pack2(acc[nb][4 * g4 + 0] * inv, acc[nb][4 * g4 + 1] * inv);
        v[1] = T::pack2(acc[nb][4 * g4 + 2] * inv, acc[nb][4 * g4 + 3] * inv);
        st8(Orow + nb * 32 + 8 * g4 + 4 * h, v);
      }
    }
    if (h == 0) a.out_lse[qrow0 + qi] = (l > 0.f) ? (m2 + __log2f(l)) * LN2 : -INFINITY;
  }
}

template <class T, int MASK, int NW>
__global__ __launch_bounds__(NW * 64, 2) void fwd_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t stages[2 * 2 * TILE_ELEMS];
  const int wg = blockIdx.x;
  if constexpr (MASK == MASK_WINDOW) {
    constexpr int BQ = 32 * NW;
    int b, hq, p;
    window_q_item(a, wg, b, hq, p);
    // Heaviest query tiles first; with `pair`, tile p also runs tile n - 1 - p.
    const int t1 = a.n_tiles - 1 - p;
    fwd_tile<T, MASK, NW>(a, b, hq, t1 * BQ, a.Sq, 0, stages);
    const int t2 = p;
    if (a.pair && t2 != t1) {
      __syncthreads();
      fwd_tile<T, MASK, NW>(a, b, hq, t2 * BQ, a.Sq, 0, stages);
    }
  } else {
    const int nbh = a.B * a.Hq;
    const int bh = wg % nbh, p = wg / nbh;
    const int b = bh / a.Hq, hq = bh % a.Hq;
    const int r0 = p * a.bx;
    fwd_tile<T, MASK, NW>(a, b, hq, r0, min(r0 + a.bx, a.Sq), p, stages);
  }
}

template <class T>
static void launch_fwd_t(const AttnArgs& a, int mask, hipStream_t st) {
  if (mask == MASK_WINDOW) {
    // Query tiles of 128 rows; for wide windows tile p is paired with tile n - 1 - p (equal
    // work) whenever that still leaves at least one workgroup per compute unit.
    AttnArgs w = a;
    w.n_tiles = (a.Sq + 127) / 128;
    const bool wide = a.window >= 256 && a.window * 4 >= a.Skv;
    w.pair = (wide && a.B * a.Hq * ((w.n_tiles + 1) / 2) >= 256) ? 1 : 0;
    const int g = a.B * a.Hq * (w.pair ? (w.n_tiles + 1) / 2 : w.n_tiles);
    hipLaunchKernelGGL((fwd_kernel<T, MASK_WINDOW, 4>), dim3(g), dim3(256), 0, st, w);
    return;
  }
  const int g = a.B * a.Hq * a.nqb;
  switch ((a.bx + 31) / 32) {
    case 1: hipLaunchKernelGGL((fwd_kernel<T, MASK_BLOCK, 1>), dim3(g), dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((fwd_kernel<T, MASK_BLOCK, 2>), dim3(g), dim3(128), 0, st, a); break;
    case 3: hipLaunchKernelGGL((fwd_kernel<T, MASK_BLOCK, 3>), dim3(g), dim3(192), 0, st, a); break;
    default: hipLaunchKernelGGL((fwd_kernel<T, MASK_BLOCK, 4>), dim3(g), dim3(256), 0, st, a); break;
  }
}

hipError_t launch_fwd(int dtype, AttnArgs a, int mask, hipStream_t st) {
  if (dtype == 1) launch_fwd_t<BF16>(a, mask, st);
  else launch_fwd_t<F16>(a, mask, st);
  return hipGetLastError();
}

}  // namespace ma
