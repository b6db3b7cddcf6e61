// Device-side block-mask transpose and selection tables: the table kernel (the rows it
// builds are defined in ma_tables.h).
#include "ma_launch.h"
#include "ma_tables.h"

namespace ma {

__global__ __launch_bounds__(256) void mask_tables_kernel(const uint8_t* __restrict__ mask, int nqb, int nkb,
                                                          uint8_t* __restrict__ mask_t, int* __restrict__ sel_q,
                                                          int* __restrict__ cnt_q, int* __restrict__ sel_k,
                                                          int* __restrict__ cnt_k) {
  mask_table_rows(mask, nqb, nkb, mask_t, sel_q, cnt_q, sel_k, cnt_k, blockIdx.x, blockIdx.y);
}

hipError_t launch_mask_tables(const uint8_t* mask, int BN, int nqb, int nkb, uint8_t* mask_t, int* sel_q,
                              int* cnt_q, int* sel_k, int* cnt_k, hipStream_t st) {
  const int rows = nqb > nkb ? nqb : nkb;
  dim3 grid(BN, (rows + 3) / 4);
  hipLaunchKernelGGL(mask_tables_kernel, grid, dim3(256), 0, st, mask, nqb, nkb, mask_t, sel_q, cnt_q, sel_k, cnt_k);
  return hipGetLastError();
}

}  // namespace ma
