// Element-wise pieces of the mixer backward (mixer_bwd.hip).
#pragma once
#include "launch.hpp"

namespace ssm {
hipError_t launch_add_f32(float* a, const float* b, int64_t n, hipStream_t s);  // a += b (16-byte aligned)
hipError_t launch_copy_cols(const float* src, int64_t m, int64_t n, float* dst, int64_t ld_dst, hipStream_t s);
}  // namespace ssm
