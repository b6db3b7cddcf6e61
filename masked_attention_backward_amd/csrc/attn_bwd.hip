// Host launchers of the attention backward: preprocess, the chunk reduce, and the dispatch of
// the dK/dV and dQ kernels (their templates are in attn_bwd_kernels.h; each variant is
// instantiated in its own object, see attn_bwd_variant.hip).
#include "attn_bwd_kernels.h"
#include "ma_tables.h"

namespace ma {

// ------------------------------------------------------------------------ preprocess
// Delta[b,h,i] = sum_d dO[b,h,i,d] * O[b,h,i,d]  (fp32) and lse2 = lse * log2(e), one
// 64-row block per workgroup, into per-row buffers padded to a multiple of 64 rows: padding
// rows and rows without any visible key get lse2 = +inf (padding rows also Delta = 0), so
// exp2(s - lse2) is exactly 0 there.
// With a sink: part[b,h,blk] = sum_{i in blk} exp(sink_h - lse_i) * Delta_i, summed in a
// fixed order (tree over the 64 rows).
// o, dout and lse are dense [B, H, S(, D)] when `cu` is null, else packed [H, total(, D)] with
// sequence b at rows cu[b] .. cu[b + 1] (clamped as the attention kernels clamp them); the
// per-row buffers stay [B, H, padded S] either way.
template <class T, bool SINK, bool STREAM>
__device__ __forceinline__ void preprocess_rows(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                const float* __restrict__ lse, const float* __restrict__ sink,
                                                float* __restrict__ delta, float* __restrict__ lse2,
                                                float* __restrict__ part, int H, int S, int nblk,
                                                const int* __restrict__ cu, int total, int blk, int h, int b) {
  const int tid = threadIdx.x, rsub = tid >> 4, ch = tid & 15;
  __shared__ float sd[64];
  size_t head = ((size_t)b * H + h) * (size_t)S;
  int len = S;
  if (cu) {
    const int s0 = min(max(cu[b], 0), total);
    const int s1 = min(max(cu[b + 1], s0), total);
    head = (size_t)h * total + s0;
    len = min(s1 - s0, S);
  }
  const size_t phead = ((size_t)b * H + h) * (size_t)nblk * 64;
  // All eight 16-byte loads of the thread go out before any is used (rows past the end read
  // the last row, in bounds, and are not used): one memory round trip per workgroup.  When O
  // and dO together exceed what the last-level cache could keep for the dK/dV kernel (STREAM)
  // the loads are non-temporal (30 % faster there); otherwise cached, so dO is still near
  // when the dK/dV kernel reads it.
  u32x4 xs[4], ys[4];
  if (len > 0) {
    if constexpr (STREAM) {
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int rr = min(blk * 64 + pass * 16 + rsub, len - 1);
        xs[pass] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o + (head + rr) * HD + ch * 8));
        ys[pass] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dout + (head + rr) * HD + ch * 8));
      }
    } else {
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int rr = min(blk * 64 + pass * 16 + rsub, len - 1);
        xs[pass] = ld16(o + (head + rr) * HD + ch * 8);
        ys[pass] = ld16(dout + (head + rr) * HD + ch * 8);
      }
    }
  }
  if (tid < 64) {
    const int row = blk * 64 + tid;
    // Rows past the end and rows that see no key at all (lse = -inf) get +inf: exp2(s - lse2)
    // is then exactly 0 for every s, including the -inf the kernels put on masked entries.
    const float l = (row < len) ? lse[head + row] : -INFINITY;
    lse2[phead + row] = (l > -INFINITY) ? l * LOG2E : INFINITY;
  }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int row = blk * 64 + pass * 16 + rsub;
    float acc = 0.f;
    if (row < len) {
      const u32x4 x = xs[pass], y = ys[pass];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(T::lo(x[e]), T::lo(y[e]), acc);
        acc = fmaf(T::hi(x[e]), T::hi(y[e]), acc);
      }
    }
    acc += __shfl_xor(acc, 8, 16);
    acc += __shfl_xor(acc, 4, 16);
    acc += __shfl_xor(acc, 2, 16);
    acc += __shfl_xor(acc, 1, 16);
    if (ch == 0) {
      delta[phead + row] = acc;
      sd[pass * 16 + rsub] = acc;
    }
  }
  if constexpr (SINK) {
    __syncthreads();
    if (tid < 64) {
      const int row = blk * 64 + tid;
      float v = 0.f;
      if (row < len) v = expf(sink[h] - lse[head + row]) * sd[tid];
      v += __shfl_xor(v, 32);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 1);
      if (tid == 0) part[((size_t)b * H + h) * nblk + blk] = v;
    }
  }
}

template <class T, bool SINK, bool STREAM>
__global__ __launch_bounds__(256) void preprocess_kernel(const uint16_t* __restrict__ o,
                                                         const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ sink, float* __restrict__ delta,
                                                         float* __restrict__ lse2, float* __restrict__ part, int H,
                                                         int S, int nblk, const int* __restrict__ cu, int total) {
  preprocess_rows<T, SINK, STREAM>(o, dout, lse, sink, delta, lse2, part, H, S, nblk, cu, total, blockIdx.x,
                                   blockIdx.y, blockIdx.z);
}

// Block path: the selection tables and the preprocess are independent, so one launch runs
// both: blocks [0, ntab) build table rows (head bn = i % BN, row group i / BN), the rest take
// one 64-row block of Delta / lse2 each; their latencies overlap and a kernel boundary goes.
template <class T, bool STREAM>
__global__ __launch_bounds__(256) void block_prep_kernel(const uint8_t* __restrict__ mask, int nqb, int nkb,
                                                         uint8_t* __restrict__ mask_t, int* __restrict__ sel_q,
                                                         int* __restrict__ cnt_q, int* __restrict__ sel_k,
                                                         int* __restrict__ cnt_k, int BN, int ntab,
                                                         const uint16_t* __restrict__ o,
                                                         const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ lse, float* __restrict__ delta,
                                                         float* __restrict__ lse2, int H, int S, int nblk) {
  const int i = blockIdx.x;
  if (i < ntab) {
    mask_table_rows(mask, nqb, nkb, mask_t, sel_q, cnt_q, sel_k, cnt_k, i % BN, i / BN);
    return;
  }
  const int j = i - ntab;
  const int blk = j % nblk, h = (j / nblk) % H, b = j / (nblk * H);
  preprocess_rows<T, false, STREAM>(o, dout, lse, nullptr, delta, lse2, nullptr, H, S, nblk, nullptr, 0, blk, h, b);
}

// Key blocks (block path) or key tiles (window path, head split) whose dK/dV sums span several
// workgroups: sum the fp32 partials in chunk order (fixed, so results are bit-identical run to
// run) and cast.  A 256-thread block covers 8 key rows x 128 columns (4 columns per thread) of
// one kv head.
template <class T, int MASK>
__global__ __launch_bounds__(256) void dkv_chunk_reduce_kernel(const AttnArgs a) {
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int row = blockIdx.x * 8 + (threadIdx.x >> 5), col = (threadIdx.x & 31) * 4;
  if (row >= a.Skv) return;
  const int nch = MASK == MASK_WINDOW ? window_chunks(a.Sq, a.window, a.group, a.chunk, row / window_key_rows(a.window))
                                      : block_chunks(a, b, kvh, row / a.by);
  if (nch <= 1) return;   // stored directly by its only workgroup
  const int skv_pad = (a.Skv + 63) & ~63;
  const size_t slot = (size_t)skv_pad * HD;
  const size_t slab = (size_t)a.B * a.Hkv * a.max_chunks * slot;
  const float* pk = a.dkv_part + ((size_t)b * a.Hkv + kvh) * a.max_chunks * slot + (size_t)row * HD + col;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nch; ++c) {
    sk += *reinterpret_cast<const f32x4*>(pk + c * slot);
    sv += *reinterpret_cast<const f32x4*>(pk + slab + c * slot);
  }
  const size_t o = (((size_t)b * a.Hkv + kvh) * a.Skv + row) * HD + col;
  st8((uint16_t*)a.dk + o, (u32x2){T::pack2(sk[0], sk[1]), T::pack2(sk[2], sk[3])});
  st8((uint16_t*)a.dv + o, (u32x2){T::pack2(sv[0], sv[1]), T::pack2(sv[2], sv[3])});
}

// ------------------------------------------------------------------------ launchers
template <class T>
static hipError_t launch_preprocess_t(const void* o, const void* dout, const float* lse, const float* sink,
                                      float* delta, float* lse2, float* part, int B, int H, int S, hipStream_t st,
                                      const int* cu, int total) {
  const int nblk = (S + 63) / 64;   // Delta / lse2 rows are padded to nblk * 64
  dim3 grid(nblk, H, B);
  // O and dO bytes against three quarters of the MI355X's 256 MiB last-level cache.
  const long long rows = cu ? (long long)H * total : (long long)B * H * S;
  const bool stream = rows * HD * 2 * 2 > (192ll << 20);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st, (const uint16_t*)o, (const uint16_t*)dout, lse, sink, delta,
                       lse2, part, H, S, nblk, cu, total);
  };
  if (sink) {
    if (stream) go(preprocess_kernel<T, true, true>);
    else go(preprocess_kernel<T, true, false>);
  } else {
    if (stream) go(preprocess_kernel<T, false, true>);
    else go(preprocess_kernel<T, false, false>);
  }
  return hipGetLastError();
}

hipError_t launch_block_prep(int dtype, const uint8_t* mask, int B, int N, int nqb, int nkb, uint8_t* mask_t,
                             int* sel_q, int* cnt_q, int* sel_k, int* cnt_k, const void* o, const void* dout,
                             const float* lse, float* delta, float* lse2, int S, hipStream_t st) {
  const int BN = B * N, rows = nqb > nkb ? nqb : nkb;
  const int ntab = BN * ((rows + 3) / 4);
  const int nblk = (S + 63) / 64;
  const long long nblocks = (long long)ntab + (long long)nblk * N * B;
  if (nblocks > 0x7fffffffll) return hipErrorInvalidValue;
  const bool stream = (long long)B * N * S * HD * 2 * 2 > (192ll << 20);   // as launch_preprocess_t
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)nblocks), dim3(256), 0, st, mask, nqb, nkb, mask_t, sel_q, cnt_q,
                       sel_k, cnt_k, BN, ntab, (const uint16_t*)o, (const uint16_t*)dout, lse, delta, lse2, N, S,
                       nblk);
  };
  if (dtype == 1) {
    if (stream) go(block_prep_kernel<BF16, true>);
    else go(block_prep_kernel<BF16, false>);
  } else {
    if (stream) go(block_prep_kernel<F16, true>);
    else go(block_prep_kernel<F16, false>);
  }
  return hipGetLastError();
}

hipError_t launch_preprocess(int dtype, const void* o, const void* dout, const float* lse, const float* sink,
                             float* delta, float* lse2, float* part, int B, int H, int S, hipStream_t st,
                             const int* cu, int total) {
  return dtype == 1 ? launch_preprocess_t<BF16>(o, dout, lse, sink, delta, lse2, part, B, H, S, st, cu, total)
                    : launch_preprocess_t<F16>(o, dout, lse, sink, delta, lse2, part, B, H, S, st, cu, total);
}

hipError_t launch_window_bwd(int dtype, AttnArgs a, hipStream_t st, hipEvent_t ev_mid) {
  // Wide windows: key/value tiles of 128 rows (dK/dV, eight waves) and query tiles of 128
  // rows (dQ).  The work per tile grows linearly along the sequence, so a workgroup runs tile
  // p and tile n-1-p (equal total work) whenever that still leaves at least one workgroup per
  // compute unit; dQ from a dS bank takes query tiles of 256 rows, eight waves sharing each
  // staged key tile.  Narrow windows (below 256): dK/dV key tiles of 64 rows (four waves, one
  // LDS stage, two workgroups per CU), whose query range [c0, c0 + 64 + W - 1) wastes less of
  // each 64-row query tile on the band's edges than 128-row key tiles do.  (Measured at S =
  // 8192: equal at W = 256, the wide kernels 3 % faster at 512 and 11 % at 1024.)
  const bool wide = window_wide(a.window);
  const int bc = wide ? 128 : 64;
  const int nt = (a.Skv + bc - 1) / bc;
  AttnArgs ak = a, aq = a;
  aq.dq_nw = (a.ds_bank && wide) ? 8 : 4;
  ak.n_tiles = nt;
  aq.n_tiles = (a.Sq + 32 * aq.dq_nw - 1) / (32 * aq.dq_nw);
  const int pairs_dkdv = a.B * a.Hkv * ((nt + 1) / 2);
  const int pairs_dq = a.B * a.Hq * ((aq.n_tiles + 1) / 2);
  // Head split (planned by the caller for dense sequences with too few key tiles to fill the
  // GPU): max_chunks slots per key tile, the partial sums added by the chunk reduce.
  const bool split = !a.cu && a.max_chunks > 1;
  if (!split) ak.max_chunks = 1;
  ak.pair = (!split && wide && pairs_dkdv >= 256) ? 1 : 0;
  aq.pair = (wide && pairs_dq >= 256) ? 1 : 0;
  const int gk = a.B * a.Hkv * (split ? ak.n_tiles * ak.max_chunks : ak.pair ? (ak.n_tiles + 1) / 2 : ak.n_tiles);
  const int gq = a.B * a.Hq * (aq.pair ? (aq.n_tiles + 1) / 2 : aq.n_tiles);
  if (wide) {
    if (dtype == 1) launch_dkdv_variant<BF16, MASK_WINDOW, 4>(ak, gk, st);
    else launch_dkdv_variant<F16, MASK_WINDOW, 4>(ak, gk, st);
  } else {
    if (dtype == 1) launch_dkdv_variant<BF16, MASK_WINDOW, 2>(ak, gk, st);
    else launch_dkdv_variant<F16, MASK_WINDOW, 2>(ak, gk, st);
  }
  if (split) {
    const dim3 grid((a.Skv + 7) / 8, a.Hkv, a.B);
    if (dtype == 1) hipLaunchKernelGGL((dkv_chunk_reduce_kernel<BF16, MASK_WINDOW>), grid, dim3(256), 0, st, ak);
    else hipLaunchKernelGGL((dkv_chunk_reduce_kernel<F16, MASK_WINDOW>), grid, dim3(256), 0, st, ak);
  }
  if (ev_mid) (void)hipEventRecord(ev_mid, st);
  if (dtype == 1) launch_dq_variant<BF16, MASK_WINDOW, 4>(aq, gq, st);
  else launch_dq_variant<F16, MASK_WINDOW, 4>(aq, gq, st);
  return hipGetLastError();
}

template <class T>
static void launch_block_t(const AttnArgs& a, hipStream_t st, hipEvent_t ev_mid) {
  const int nwk = (a.by + 31) / 32, nwq = (a.bx + 31) / 32;
  const int gk = a.B * a.Hkv * a.nkb * a.max_chunks, gq = a.B * a.Hq * a.nqb;
  switch (nwk) {
    case 1: launch_dkdv_variant<T, MASK_BLOCK, 1>(a, gk, st); break;
    case 2: launch_dkdv_variant<T, MASK_BLOCK, 2>(a, gk, st); break;
    case 3: launch_dkdv_variant<T, MASK_BLOCK, 3>(a, gk, st); break;
    default: launch_dkdv_variant<T, MASK_BLOCK, 4>(a, gk, st); break;
  }
  if (a.max_chunks > 1)
    hipLaunchKernelGGL((dkv_chunk_reduce_kernel<T, MASK_BLOCK>), dim3((a.Skv + 7) / 8, a.Hkv, a.B), dim3(256), 0,
                       st, a);
  if (ev_mid) (void)hipEventRecord(ev_mid, st);
  if (a.ds_bank && (a.bx % 32 != 0 || a.by % 32 != 0)) {
    // dS bank with query halves or key sub-blocks off the 32-row grid: one wave per 32-row
    // query half, DQU_WAVES per workgroup.
    const int per = 32 * DQU_WAVES;
    hipLaunchKernelGGL(dq_ds_blocku_kernel<T>, dim3(a.B * a.Hq * ((a.Sq + per - 1) / per)), dim3(DQU_WAVES * 64), 0,
                       st, a);
    return;
  }
  switch (nwq) {
    case 1: launch_dq_variant<T, MASK_BLOCK, 1>(a, gq, st); break;
    case 2: launch_dq_variant<T, MASK_BLOCK, 2>(a, gq, st); break;
    case 3: launch_dq_variant<T, MASK_BLOCK, 3>(a, gq, st); break;
    default: launch_dq_variant<T, MASK_BLOCK, 4>(a, gq, st); break;
  }
}

hipError_t launch_block_bwd(int dtype, AttnArgs a, hipStream_t st, hipEvent_t ev_mid) {
  if (dtype == 1) launch_block_t<BF16>(a, st, ev_mid);
  else launch_block_t<F16>(a, st, ev_mid);
  return hipGetLastError();
}

}  // namespace ma
