// Pieces of the mixer backward: the dB / dC placement (mixer_bwd.hip) and the STE backward
// with an accumulated dx (ste.hip).
#pragma once
#include "launch.hpp"

namespace ssm {
hipError_t launch_copy_cols(const float* src, int64_t m, int64_t n, float* dst, int64_t ld_dst, hipStream_t s);
// the straight-through backward (launch_ste_bwd) with dx = add + (its dx); add may equal dx
// (row stride ld_add, fp32 [M, K]) or be NULL (ste.hip)
hipError_t launch_ste_bwd_add(const SteArgs& a, const float* add, int64_t ld_add, void* ws, hipStream_t s);
}  // namespace ssm
