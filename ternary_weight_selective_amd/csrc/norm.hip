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
  // raw elements first (all loads in flight together), then fp32, the gains alongside
  Tin raw[KPL];
  float gn[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    raw[i] = (k < K) ? xr[k] : Tin(0);
    gn[i] = gain ? gain[k < K ? k : 0] : 1.0f;
  }
  float v[KPL];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    v[i] = act_f32(raw[i]);
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
    if (gain) t = (k < K) ? t * gn[i] : 0.0f;
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

// The same computation with the row moved through LDS: 16-byte coalesced loads of x into a
// per-wave LDS row, the per-lane reads in the canonical layout (lane j, columns j + 64 i),
// and the outputs (int8 codes, or the bf16 terms) written back through the same LDS row and
// stored as 16-byte chunks.  Needs 16-byte aligned rows (x, ldx, k and the outputs).
namespace {
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
}  // namespace

template <int KPL, typename Tin, int MODE>
__global__ __launch_bounds__(256) void k_norm_vec(const Tin* __restrict__ x, int64_t M, int K, int64_t ldx,
                                                  const float* __restrict__ gain, float eps, int ldo,
                                                  int8_t* __restrict__ q, float* __restrict__ absmax,
                                                  int8_t* __restrict__ q2, bf16_t* __restrict__ xh,
                                                  bf16_t* __restrict__ xh_lo) {
  constexpr int KMAX = 64 * KPL;
  constexpr int IN_B = KMAX * (int)sizeof(Tin);
  constexpr int OUT_B = MODE == 8 ? KMAX : 4 * KMAX;  // codes, or bf16 hi and lo
  constexpr int RB = IN_B > OUT_B ? IN_B : OUT_B;     // LDS bytes per wave
  __shared__ __align__(16) char s_row[4][RB];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  const bool rv = row < M;  // all waves take part in the barriers
  char* sr = s_row[wv];
  const int nin = K * (int)sizeof(Tin) / 16;
  // the gains first, unconditionally from clamped columns: a load under a lane-dependent
  // condition would be waited for inside it, one memory round trip per load
  float gn[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    gn[i] = gain ? gain[k < K ? k : K - 1] : 1.0f;
  }
  if (rv) {  // every 16-byte chunk of the row in flight at once, then into LDS
    constexpr int CPL = (IN_B / 16 + 63) / 64;
    const v4i* xr = (const v4i*)(x + row * ldx);
    v4i ch[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      ch[j] = c < nin ? xr[c] : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < nin) *(v4i*)(sr + 16 * c) = ch[j];
    }
  }
  lds_sync();
  const Tin* se = (const Tin*)sr;
  float v[KPL];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {  // (every column of the buffer is read; those past K are masked)
    const int k = lane + 64 * i;
    const float e = ld_act(se + k);
    v[i] = (rv && k < K) ? e : 0.0f;
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
    if (gain) t = (k < K) ? t * gn[i] : 0.0f;
    v[i] = t;
    m = fmaxf(m, fabsf(t));
  }
  lds_sync();  // every lane has read its inputs: the row buffer takes the outputs
  const int nout = MODE == 8 ? ldo / 16 : ldo * 2 / 16;
  if (MODE == 8) {
    m = wave_absmax(m);
    const float sigma = __fdiv_rn(127.0f, fmaxf(m, 1e-5f));
    int8_t* so = (int8_t*)sr;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int k = lane + 64 * i;
      float rr = rintf(v[i] * sigma);
      rr = fminf(fmaxf(rr, -128.0f), 127.0f);
      const int8_t qv = (int8_t)(int)rr;
      if (k < ldo) so[k] = qv;
      if (q2 && rv && k < K) q2[row * K + k] = qv;
    }
    if (lane == 0 && rv) absmax[row] = m;
  } else {
    bf16_t* so = (bf16_t*)sr;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int k = lane + 64 * i;
      if (k < ldo) {
        const bf16_t hi = f32_to_bf16(v[i]);
        so[k] = hi;
        if (xh_lo) so[KMAX + k] = f32_to_bf16(v[i] - bf16_to_f32(hi));
      }
    }
  }
  lds_sync();
  if (rv) {
    if (MODE == 8) {
      v4i* qo = (v4i*)(q + row * ldo);
      for (int c = lane; c < nout; c += 64) qo[c] = *(const v4i*)(sr + 16 * c);
    } else {
      v4i* ho = (v4i*)(xh + row * ldo);
      for (int c = lane; c < nout; c += 64) ho[c] = *(const v4i*)(sr + 16 * c);
      if (xh_lo) {
        v4i* lo = (v4i*)(xh_lo + row * ldo);
        for (int c = lane; c < nout; c += 64) lo[c] = *(const v4i*)(sr + 2 * KMAX + 16 * c);
      }
    }
  }
}

template <int KPL, typename Tin>
static void launch_norm_t(const void* x, int64_t m, int k, int64_t ldx, const float* gain, float eps, int mode,
                          int ldo, int8_t* q, float* absmax, int8_t* q2, bf16_t* xh, bf16_t* xh_lo, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(m, 4)), block(256);
  const int es = (int)sizeof(Tin);
  auto al = [](const void* p) { return p == nullptr || ((uintptr_t)p % 16) == 0; };
  const bool vec = KPL >= 8 && (ldx * es) % 16 == 0 && (k * es) % 16 == 0 && al(x) && ldo % 64 == 0 &&
                   ldo <= 64 * KPL && (mode == 8 ? al(q) : al(xh) && al(xh_lo));
  if (vec) {
    if (mode == 8)
      hipLaunchKernelGGL((k_norm_vec<KPL, Tin, 8>), grid, block, 0, s, (const Tin*)x, m, k, ldx, gain, eps, ldo, q,
                         absmax, q2, xh, xh_lo);
    else
      hipLaunchKernelGGL((k_norm_vec<KPL, Tin, 16>), grid, block, 0, s, (const Tin*)x, m, k, ldx, gain, eps, ldo,
                         q, absmax, q2, xh, xh_lo);
    return;
  }
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
