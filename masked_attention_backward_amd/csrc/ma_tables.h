// Device-side block-mask transpose and selection tables (the rows one 256-thread block
// builds), shared by the table kernel and the block path's fused table + preprocess kernel.
//
// Page "knowledge(triton) ... #174" (cannbot-knowledge PR 174), BlockSparseAttentionGrad
// runbook, "optimisation 1" and "optimisation 2": the host only checks shapes, allocates
// and views; the uint8 mask is transposed on the device (result bit-equal to
// mask.permute(0,1,3,2)); each table row lists the kept columns, placed by an exclusive
// prefix count of the kept entries, and a count drives the consumer's loop.
//
// On CDNA4 the prefix count of a 64-column chunk is one wave ballot plus mbcnt (the
// number of set ballot bits below the lane): no dot product, no atomics.  Each wave
// compacts one q-major row (a row of the mask) and one kv-major row (a column of the
// mask, written out as a row of the transposed mask).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ma {

__device__ __forceinline__ int lanes_below(uint64_t ballot) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(ballot >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0u));
}

// Rows 4 rg .. 4 rg + 3 (one per wave of a 256-thread block) of head bn's two tables.
__device__ __forceinline__ void mask_table_rows(const uint8_t* __restrict__ mask, int nqb, int nkb,
                                                uint8_t* __restrict__ mask_t, int* __restrict__ sel_q,
                                                int* __restrict__ cnt_q, int* __restrict__ sel_k,
                                                int* __restrict__ cnt_k, int bn, int rg) {
  const int lane = threadIdx.x & 63;
  const int row = rg * 4 + (threadIdx.x >> 6);
  const uint8_t* m = mask + (size_t)bn * nqb * nkb;
  if (row < nqb) {
    int* out = sel_q + ((size_t)bn * nqb + row) * nkb;
    int base = 0;
    for (int j0 = 0; j0 < nkb; j0 += 64) {
      const int j = j0 + lane;
      const bool keep = (j < nkb) && (m[(size_t)row * nkb + j] != 0);
      const uint64_t bal = __ballot(keep);
      if (keep) out[base + lanes_below(bal)] = j;
      base += __popcll(bal);
    }
    for (int j = base + lane; j < nkb; j += 64) out[j] = -1;
    if (lane == 0) cnt_q[(size_t)bn * nqb + row] = base;
  }
  if (row < nkb) {
    int* out = sel_k + ((size_t)bn * nkb + row) * nqb;
    uint8_t* mt = mask_t + ((size_t)bn * nkb + row) * nqb;
    int base = 0;
    for (int i0 = 0; i0 < nqb; i0 += 64) {
      const int i = i0 + lane;
      const uint8_t v = (i < nqb) ? m[(size_t)i * nkb + row] : (uint8_t)0;
      if (i < nqb) mt[i] = v;
      const bool keep = v != 0;
      const uint64_t bal = __ballot(keep);
      if (keep) out[base + lanes_below(bal)] = i;
      base += __popcll(bal);
    }
    for (int i = base + lane; i < nqb; i += 64) out[i] = -1;
    if (lane == 0) cnt_k[(size_t)bn * nkb + row] = base;
  }
}

}  // namespace ma
