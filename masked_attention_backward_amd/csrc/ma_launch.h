// Host-side launch entry points of the kernels (called by the C ABI in capi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ma_device.h"

namespace ma {

hipError_t launch_preprocess(int dtype, const void* o, const void* dout, const float* lse, const float* sink,
                             float* delta, float* lse2, float* part, int B, int H, int S, hipStream_t st,
                             const int* cu = nullptr, int total = 0);
hipError_t launch_window_bwd(int dtype, AttnArgs a, hipStream_t st, hipEvent_t ev_mid = nullptr);
hipError_t launch_block_bwd(int dtype, AttnArgs a, hipStream_t st, hipEvent_t ev_mid = nullptr);
hipError_t launch_fwd(int dtype, AttnArgs a, int mask, hipStream_t st);
// Block path: selection tables and preprocess (Delta, lse * log2 e) in one launch.
hipError_t launch_block_prep(int dtype, const uint8_t* mask, int B, int N, int nqb, int nkb, uint8_t* mask_t,
                             int* sel_q, int* cnt_q, int* sel_k, int* cnt_k, const void* o, const void* dout,
                             const float* lse, float* delta, float* lse2, int S, hipStream_t st);
hipError_t launch_mask_tables(const uint8_t* mask, int BN, int nqb, int nkb, uint8_t* mask_t, int* sel_q,
                              int* cnt_q, int* sel_k, int* cnt_k, hipStream_t st);

}  // namespace ma
