// One variant of the dK/dV and dQ kernels, selected at compile time:
//   MA_VARIANT_DTYPE  0 = fp16, 1 = bf16
//   MA_VARIANT_MASK   0 = sliding window (+ sink), 1 = block mask
//   MA_VARIANT_NW     waves per workgroup (32 stationary rows each)
// The build compiles this file once per variant the dispatch in attn_bwd.hip uses.
#include "attn_bwd_kernels.h"

#if !defined(MA_VARIANT_DTYPE) || !defined(MA_VARIANT_MASK) || !defined(MA_VARIANT_NW)
#error "MA_VARIANT_DTYPE, MA_VARIANT_MASK and MA_VARIANT_NW must be defined"
#endif

namespace ma {

using VariantT = std::conditional_t<MA_VARIANT_DTYPE == 1, BF16, F16>;

template <class T, int MASK, int NW>
void launch_dkdv_variant(const AttnArgs& a, int grid, hipStream_t st) {
  launch_dkdv_only<T, MASK, NW>(a, grid, st);
}

template <class T, int MASK, int NW>
void launch_dq_variant(const AttnArgs& a, int grid, hipStream_t st) {
  launch_dq_only<T, MASK, NW>(a, grid, st);
}

template void launch_dkdv_variant<VariantT, MA_VARIANT_MASK, MA_VARIANT_NW>(const AttnArgs&, int, hipStream_t);
template void launch_dq_variant<VariantT, MA_VARIANT_MASK, MA_VARIANT_NW>(const AttnArgs&, int, hipStream_t);

}  // namespace ma
