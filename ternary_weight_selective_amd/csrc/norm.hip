// RMSNorm + per-token absmax int8 quantisation (TriSSM README: an RMSNorm precedes each
// ternary projection, int8 activations; absmax scaling from BitNet b1.58), or RMSNorm to
// bf16 for the W1.58A16 path (Ternary Mamba abstract).  One wave64 per token row.
#include "launch.hpp"

namespace ssm {

// Lane j keeps columns j, j+64, ... of the row in registers.  The sum of squares is the
// fixed-order one: lane j accumulates its columns in ascending order with fused
// multiply-adds from 0, then the butterfly over the wave.  mean = s / k, r = 1 / sqrt(mean
// + eps) with IEEE division and square root; xh = (x * r) * gain.
template <int KPL, typename Tin, int MODE>
__global__ __launch_bounds__(256) void k_norm(const Tin* __restrict__ x, int64_t M, int K, int64_t ldx,
                                              const float* __restrict__ gain, float eps, int ldo,
                                              int8_t* __restrict__ q, float* __restrict__ absmax,
                                              int8_t* __restrict__ q2, bf16_t* __restrict__ xh,
                                              bf16_t* __restrict__ xh_lo) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // uniform per wave
  const Tin* xr = x + row * ldx;
  float v[KPL];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    v[i] = (k < K) ? ld_act(xr + k) : 0.0f;
    s = __builtin_fmaf(v[i], v[i], s);
  }
  s = wave_sum_butterfly(s);
  const float ms = __fdiv_rn(s, (float)K);
  const float r = __fdiv_rn(1.0f, sqrt_rn(ms + eps));
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    float t = v[i] * r;
    if (gain) t = (k < K) ? t * gain[k] : 0.0f;
    v[i] = t;
    m = fmaxf(m, fabsf(t));
  }
  if (MODE == 8) {
    m = wave_absmax(m);
    const float sigma = __fdiv_rn(127.0f, fmaxf(m, 1e-5f));
    int8_t* qr = q + row * ldo;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int k = lane + 64 * i;
      float rr = rintf(v[i] * sigma);
      rr = fminf(fmaxf(rr, -128.0f), 127.0f);
      const int8_t qv = (int8_t)(int)rr;
      if (k < ldo) qr[k] = qv;
      if (q2 && k < K) q2[row * K + k] = qv;
    }
    if (lane == 0) absmax[row] = m;
  } else {
    bf16_t* o = xh + row * ldo;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int k = lane + 64 * i;
      if (k < ldo) {
        const bf16_t hi = f32_to_bf16(v[i]);
        o[k] = hi;
        // second bf16 term: v = hi + lo to about 16 significant bits (for fp32 outputs)
        if (xh_lo) xh_lo[row * ldo + k] = f32_to_bf16(v[i] - bf16_to_f32(hi));
      }
    }
  }
}

template <int KPL, typename Tin>
static void launch_norm_t(const void* x, int64_t m, int k, int64_t ldx, const float* gain, float eps, int mode,
                          int ldo, int8_t* q, float* absmax, int8_t* q2, bf16_t* xh, bf16_t* xh_lo, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(m, 4)), block(256);
  if (mode == 8)
    hipLaunchKernelGGL((k_norm<KPL, Tin, 8>), grid, block, 0, s, (const Tin*)x, m, k, ldx, gain, eps, ldo, q,
                       absmax, q2, xh, xh_lo);
  else
    hipLaunchKernelGGL((k_norm<KPL, Tin, 16>), grid, block, 0, s, (const Tin*)x, m, k, ldx, gain, eps, ldo, q,
                       absmax, q2, xh, xh_lo);
}

template <typename Tin>
static hipError_t launch_norm_k(const void* x, int64_t m, int k, int64_t ldx, const float* gain, float eps,
                                int mode, int ldo, int8_t* q, float* absmax, int8_t* q2, bf16_t* xh,
                                bf16_t* xh_lo, hipStream_t s) {
  if (k <= 64) launch_norm_t<1, Tin>(x, m, k, ldx, gain, eps, mode, ldo, q, absmax, q2, xh, xh_lo, s);
  else if (k <= 128) launch_norm_t<2, Tin>(x, m, k, ldx, gain, eps, mode, ldo, q, absmax, q2, xh, xh_lo, s);
  else if (k <= 256) launch_norm_t<4, Tin>(x, m, k, ldx, gain, eps, mode, ldo, q, absmax, q2, xh, xh_lo, s);
  else if (k <= 512) launch_norm_t<8, Tin>(x, m, k, ldx, gain, eps, mode, ldo, q, absmax, q2, xh, xh_lo, s);
  else if (k <= 1024) launch_norm_t<16, Tin>(x, m, k, ldx, gain, eps, mode, ldo, q, absmax, q2, xh, xh_lo, s);
  else if (k <= 2048) launch_norm_t<32, Tin>(x, m, k, ldx, gain, eps, mode, ldo, q, absmax, q2, xh, xh_lo, s);
  else if (k <= 4096) launch_norm_t<64, Tin>(x, m, k, ldx, gain, eps, mode, ldo, q, absmax, q2, xh, xh_lo, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_norm(const void* x, int x_bf16, int64_t m, int k, int64_t ldx, const float* gain, float eps,
                       int mode, int ldo, int8_t* q, float* absmax, int8_t* q2, bf16_t* xh, bf16_t* xh_lo, hipStream_t s) {
  if (m == 0) return hipSuccess;
  if (x_bf16) return launch_norm_k<bf16_t>(x, m, k, ldx, gain, eps, mode, ldo, q, absmax, q2, xh, xh_lo, s);
  return launch_norm_k<float>(x, m, k, ldx, gain, eps, mode, ldo, q, absmax, q2, xh, xh_lo, s);
}

}  // namespace ssm
