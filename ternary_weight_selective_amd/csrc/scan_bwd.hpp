// Backward of the Mamba-1 kind selective scan (scan_bwd.hip).
#pragma once
#include "launch.hpp"

namespace ssm {

struct ScanBwdArgs {
  int64_t batch, L, H, N;
  int act_bf16, softplus;
  const void* x; int64_t ld_x;
  const void* delta; int64_t ld_delta;   // pre-activation dt
  const float* delta_bias; const float* A;
  const void* Bm; int64_t ld_B;
  const void* Cm; int64_t ld_C;
  const float* D; const float* h0;
  const float* dy; int64_t ld_dy;        // fp32
  float* dx; float* ddelta;              // [B, L, H] each
  float* dA; float* dB; float* dC;       // [H, N], [B, L, N], [B, L, N]
  float* dD; float* dbias; float* dh0;   // [H], [H], [B, H, N]; nullable
};
size_t scan_bwd_workspace(const ScanBwdArgs& a);
hipError_t launch_scan_bwd(const ScanBwdArgs& a, void* ws, hipStream_t s);

}  // namespace ssm
