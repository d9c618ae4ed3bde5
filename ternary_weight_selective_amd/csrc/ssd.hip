// Selective scan, SSD kind ("Transformers are SSMs", cited by title in "SSDi8 ...", Builds
// on; the Mamba-2 shape of the Ternary Mamba abstract): scalar A per head, a state of
// headdim x d_state per head, B and C shared by all heads.
//
// Recurrent evaluation: each lane owns 8 states of one (head, channel) pair; the
// d_state / 8 lanes of a channel add their readout partials with xor shuffles.  The decay
// exp(dt A) is one value per (token, head) and is computed once per LDS tile.
#include "launch.hpp"

namespace ssm {

namespace {
__device__ __forceinline__ float softplus_s(float v) { return v > 20.0f ? v : log1pf(expf(v)); }
}  // namespace

template <int NS, typename T>
__global__ __launch_bounds__(256) void k_scan_ssd_rec(ScanArgs a) {
  constexpr int SPL = 8;
  constexpr int LPP = NS / SPL;    // lanes per channel
  constexpr int PPB = 256 / LPP;   // channels per block
  constexpr int TT = 32;
  __shared__ float s_B[TT][NS];
  __shared__ float s_C[TT][NS];
  __shared__ float s_a[TT];
  __shared__ float s_dt[TT];
  __shared__ float s_ux[TT][PPB];
  __shared__ float s_dx[TT][PPB];
  __shared__ float s_y[TT][PPB];

  const int tid = threadIdx.x;
  const int64_t L = a.L, H = a.H, P = a.P;
  const int64_t hd = blockIdx.y, b = blockIdx.z;
  const int pl = tid / LPP, qq = tid % LPP;
  const int64_t p = (int64_t)blockIdx.x * PPB + pl;
  const bool pv = p < P;
  const float A_h = a.A[hd];
  const float bias_h = a.delta_bias ? a.delta_bias[hd] : 0.0f;
  const float D_h = a.D ? a.D[hd] : 0.0f;
  const T* X = (const T*)a.x;
  const T* DT = (const T*)a.delta;
  const T* Bm = (const T*)a.Bm;
  const T* Cm = (const T*)a.Cm;
  T* Y = (T*)a.y;

  float h[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i)
    h[i] = (pv && a.h0) ? a.h0[((b * H + hd) * P + p) * NS + qq * SPL + i] : 0.0f;

  for (int64_t t0 = 0; t0 < L; t0 += TT) {
    for (int e = tid; e < TT * NS; e += 256) {
      const int t = e / NS, n = e % NS;
      const bool valid = t0 + t < L;
      const int64_t tok = b * L + t0 + t;
      s_B[t][n] = valid ? ld_act(Bm + tok * a.ld_B + n) : 0.0f;
      s_C[t][n] = valid ? ld_act(Cm + tok * a.ld_C + n) : 0.0f;
    }
    if (tid < TT) {
      const bool valid = t0 + tid < L;
      float dt = valid ? ld_act(DT + (b * L + t0 + tid) * a.ld_delta + hd) : 0.0f;
      dt += bias_h;
      if (a.softplus) dt = softplus_s(dt);
      s_dt[tid] = dt;
      s_a[tid] = expf(dt * A_h);
    }
    __syncthreads();
    for (int e = tid; e < TT * PPB; e += 256) {
      const int t = e / PPB, pp = e % PPB;
      const int64_t pg = (int64_t)blockIdx.x * PPB + pp;
      const bool valid = (t0 + t < L) && pg < P;
      const float xv = valid ? ld_act(X + (b * L + t0 + t) * a.ld_x + hd * P + pg) : 0.0f;
      s_ux[t][pp] = s_dt[t] * xv;
      s_dx[t][pp] = D_h * xv;
    }
    __syncthreads();
    const int tmax = (int)((L - t0) < TT ? (L - t0) : TT);
    for (int t = 0; t < tmax; ++t) {
      const float ab = s_a[t], ux = s_ux[t][pl];
      float yp = 0.0f;
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int n = qq * SPL + i;
        h[i] = __builtin_fmaf(ab, h[i], ux * s_B[t][n]);
        yp = __builtin_fmaf(s_C[t][n], h[i], yp);
      }
#pragma unroll
      for (int off = LPP / 2; off >= 1; off >>= 1) yp = yp + __shfl_xor(yp, off, 64);
      if (qq == 0) s_y[t][pl] = yp + s_dx[t][pl];
    }
    __syncthreads();
    for (int e = tid; e < TT * PPB; e += 256) {
      const int t = e / PPB, pp = e % PPB;
      const int64_t pg = (int64_t)blockIdx.x * PPB + pp;
      if ((t0 + t < L) && pg < P) st_act(Y + (b * L + t0 + t) * a.ld_y + hd * P + pg, s_y[t][pp]);
    }
  }
  if (a.h_last && pv) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) a.h_last[((b * H + hd) * P + p) * NS + qq * SPL + i] = h[i];
  }
}

template <int NS, typename T>
static void launch_ssd_t(const ScanArgs& a, hipStream_t s) {
  constexpr int PPB = 256 / (NS / 8);
  const dim3 grid((unsigned)cdiv(a.P, PPB), (unsigned)a.H, (unsigned)a.batch), block(256);
  hipLaunchKernelGGL((k_scan_ssd_rec<NS, T>), grid, block, 0, s, a);
}

template <typename T>
static hipError_t launch_ssd_n(const ScanArgs& a, hipStream_t s) {
  switch (a.N) {
    case 16: launch_ssd_t<16, T>(a, s); break;
    case 32: launch_ssd_t<32, T>(a, s); break;
    case 64: launch_ssd_t<64, T>(a, s); break;
    case 128: launch_ssd_t<128, T>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t scan_ssd_workspace(const ScanArgs&) { return 0; }

hipError_t launch_scan_ssd(const ScanArgs& a, void*, size_t, hipStream_t s) {
  if (a.batch == 0 || a.L == 0) return hipSuccess;
  return a.act_bf16 ? launch_ssd_n<bf16_t>(a, s) : launch_ssd_n<float>(a, s);
}

}  // namespace ssm
