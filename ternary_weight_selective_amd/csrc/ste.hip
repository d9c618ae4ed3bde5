// Training side of BitLinear: the backward pass with straight-through estimators and one step
// of quantisation-aware training with learnable scales (TriSSM README: BitLinear trained with
// straight-through estimators; Ternary Mamba abstract: grouped QAT with learnable quantisation
// scales and the zero ratio they can collapse).  The estimator passes gradients through both
// roundings: dx̂ = dy W̃ with W̃ = s q (the ternary codes times their scale), dW = dy^T x̃ with
// x̃ the forward's int8 codes dequantised, then the RMSNorm backward.  The two contractions are
// plain dense fp32 GEMMs (rocBLAS, dense.cpp); the kernels here rebuild the forward's codes,
// the dequantised operands, the RMSNorm backward and the scale gradient.
#include "launch.hpp"

namespace ssm {

// One wave per token row: the forward's RMSNorm and absmax int8 codes in the forward's own
// arithmetic order (so the codes are the forward's), then x̃ = q max(m, 1e-5) / 127 (fp64,
// rounded once) and the row's RMSNorm scale r.
template <int KPL, typename Tin>
__global__ __launch_bounds__(256) void k_ste_act(const Tin* __restrict__ x, int64_t M, int K, int64_t ldx,
                                                 const float* __restrict__ gain, float eps, float* __restrict__ xt,
                                                 float* __restrict__ rs) {
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
  m = wave_absmax(m);
  const float mf = fmaxf(m, 1e-5f);
  const float sigma = __fdiv_rn(127.0f, mf);
  const double step = (double)mf / 127.0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    float q = rintf(v[i] * sigma);
    q = fminf(fmaxf(q, -128.0f), 127.0f);
    if (k < K) xt[row * K + k] = (float)((double)q * step);
  }
  if (lane == 0) rs[row] = r;
}

// W̃[n, k] = s(n, k / group) q[n, k] (one scale when group == 0); thread per packed word.
__global__ __launch_bounds__(256) void k_ste_weights(const uint32_t* __restrict__ W, int64_t N, int64_t K,
                                                     int64_t row_words, const float* __restrict__ scale,
                                                     int64_t group, float* __restrict__ wt) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= N * row_words) return;
  const int64_t n = t / row_words, w = t % row_words;
  const v4i c = unpack16_i8(W[t]);
  const int8_t* cb = (const int8_t*)&c;
  const int64_t ng = group ? K / group : 1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t k = w * 16 + i;
    if (k < K) {
      const float sc = group ? scale[n * ng + k / group] : scale[0];
      wt[n * K + k] = sc * (float)cb[i];
    }
  }
}

// RMSNorm backward, one wave per row: dx = r g dx̂ - x (r^3 / K) sum_j g_j dx̂_j x_j.
template <int KPL, typename Tin>
__global__ __launch_bounds__(256) void k_rms_bwd(const Tin* __restrict__ x, int64_t M, int K, int64_t ldx,
                                                 const float* __restrict__ gain, const float* __restrict__ rs,
                                                 const float* __restrict__ dxh, float* __restrict__ dx,
                                                 int64_t ld_dx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  float xv[KPL], gd[KPL];
  float dot = 0.0f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    const bool ok = k < K;
    xv[i] = ok ? ld_act(x + row * ldx + k) : 0.0f;
    gd[i] = ok ? (gain ? gain[k] : 1.0f) * dxh[row * K + k] : 0.0f;
    dot = __builtin_fmaf(gd[i], xv[i], dot);
  }
  dot = wave_sum_butterfly(dot);
  const float r = rs[row];
  const float c = r * r * r / (float)K * dot;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    if (k < K) dx[row * ld_dx + k] = r * gd[i] - xv[i] * c;
  }
}

// Scale gradient per (row, group) (or per row for one scale, summed afterwards): one wave per
// segment, ds = sum dW (q - v) where |v| <= 1, dW q elsewhere, v = W / s.
__global__ __launch_bounds__(256) void k_scale_grad(const float* __restrict__ dw, const float* __restrict__ wl,
                                                    const float* __restrict__ scale, int64_t N, int64_t K,
                                                    int64_t group, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t G = group ? group : K, ng = K / G;
  if (seg >= N * ng) return;
  const int64_t n = seg / ng, g = seg % ng;
  const float sc = group ? scale[n * ng + g] : scale[0];
  float acc = 0.0f;
  for (int64_t j = lane; j < G; j += 64) {
    const int64_t k = g * G + j;
    const float w = wl[n * K + k];
    const float v = w / sc;
    const float q = fminf(fmaxf(rintf(v), -1.0f), 1.0f);
    const float f = fabsf(v) <= 1.0f ? q - v : q;
    acc = __builtin_fmaf(dw[n * K + k], f, acc);
  }
  acc = wave_sum_butterfly(acc);
  if (lane == 0) out[seg] = acc;
}

// Sum of n per-row partials (one scale per tensor), one wave in a fixed order: lane j adds
// rows j, j + 64, ... in fp64, then the wave's butterfly.
__global__ void k_sum_rows(const float* __restrict__ part, int64_t n, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  double s = 0.0;
  for (int64_t i = lane; i < n; i += 64) s += (double)part[i];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  if (lane == 0) out[0] = (float)s;
}

// dW = sum of the token chunks' partial products, in chunk order.
__global__ __launch_bounds__(256) void k_sum_chunks(const float* __restrict__ part, int64_t count, int64_t chunks,
                                                    float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float s = part[i];
  for (int64_t c = 1; c < chunks; ++c) s += part[c * count + i];
  dw[i] = s;
}

namespace {
// Token chunks for dW = dy^T x̃: the reduction over tokens is split so that the library sees
// several (n x k x tokens / chunks) products (a single long reduction with a small output
// leaves most of the chip idle), their partials kept within 64 MB.
int64_t dw_chunks(int64_t M, int64_t N, int64_t K) {
  int64_t c = 16;
  while (c > 1 && (M % c != 0 || M / c < 512 || c * N * K * 4 > (64ll << 20))) c >>= 1;
  return c;
}
}  // namespace

// W -= lr dW; s -= lr_s ds (fp32 fused multiply-adds).
__global__ __launch_bounds__(256) void k_sgd(float* __restrict__ w, const float* __restrict__ dw, int64_t n,
                                             float lr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) w[i] = __builtin_fmaf(-lr, dw[i], w[i]);
}

namespace {
template <typename Tin>
hipError_t launch_act_k(const SteArgs& a, float* xt, float* rs, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(a.M, 4)), block(256);
  const Tin* x = (const Tin*)a.x;
#define SSM_ACT(KK) hipLaunchKernelGGL((k_ste_act<KK, Tin>), grid, block, 0, s, x, a.M, (int)a.K, a.ldx, a.gain, a.eps, xt, rs)
  if (a.K <= 64) SSM_ACT(1);
  else if (a.K <= 128) SSM_ACT(2);
  else if (a.K <= 256) SSM_ACT(4);
  else if (a.K <= 512) SSM_ACT(8);
  else if (a.K <= 1024) SSM_ACT(16);
  else if (a.K <= 2048) SSM_ACT(32);
  else if (a.K <= 4096) SSM_ACT(64);
  else return hipErrorInvalidValue;
#undef SSM_ACT
  return hipGetLastError();
}

template <typename Tin>
hipError_t launch_rms_bwd_k(const SteArgs& a, const float* rs, const float* dxh, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(a.M, 4)), block(256);
  const Tin* x = (const Tin*)a.x;
#define SSM_RB(KK) hipLaunchKernelGGL((k_rms_bwd<KK, Tin>), grid, block, 0, s, x, a.M, (int)a.K, a.ldx, a.gain, rs, dxh, a.dx, a.ld_dx)
  if (a.K <= 64) SSM_RB(1);
  else if (a.K <= 128) SSM_RB(2);
  else if (a.K <= 256) SSM_RB(4);
  else if (a.K <= 512) SSM_RB(8);
  else if (a.K <= 1024) SSM_RB(16);
  else if (a.K <= 2048) SSM_RB(32);
  else if (a.K <= 4096) SSM_RB(64);
  else return hipErrorInvalidValue;
#undef SSM_RB
  return hipGetLastError();
}
}  // namespace

size_t ste_workspace(const SteArgs& a) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t b = al((size_t)a.M * a.K * 4);       // x̃
  b += al((size_t)a.M * 4);                   // r
  b += al((size_t)a.N * a.K * 4);             // W̃
  b += al((size_t)a.M * a.K * 4);             // dx̂
  b += al((size_t)a.N * 4);                   // per-row scale partials
  const int64_t ch = dw_chunks(a.M, a.N, a.K);
  if (ch > 1) b += al((size_t)ch * a.N * a.K * 4);  // dW partials per token chunk
  return b;
}

hipError_t launch_ste_bwd(const SteArgs& a, void* ws, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  char* p = (char*)ws;
  float* xt = (float*)p; p += al((size_t)a.M * a.K * 4);
  float* rs = (float*)p; p += al((size_t)a.M * 4);
  float* wt = (float*)p; p += al((size_t)a.N * a.K * 4);
  float* dxh = (float*)p; p += al((size_t)a.M * a.K * 4);
  float* part = (float*)p; p += al((size_t)a.N * 4);
  float* dwp = (float*)p;
  hipError_t e = a.x_bf16 ? launch_act_k<bf16_t>(a, xt, rs, s) : launch_act_k<float>(a, xt, rs, s);
  if (e != hipSuccess) return e;
  const int64_t words = a.N * a.w_row_words;
  hipLaunchKernelGGL(k_ste_weights, dim3((unsigned)cdiv(words, 256)), dim3(256), 0, s, a.W, a.N, a.K, a.w_row_words,
                     a.scale, a.group, wt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dx̂ [M, K] = dy [M, N] W̃ [N, K]
  e = sgemm_rm(false, false, a.M, a.K, a.N, a.dy, a.ld_dy, wt, a.K, dxh, a.K, s);
  if (e != hipSuccess) return e;
  e = a.x_bf16 ? launch_rms_bwd_k<bf16_t>(a, rs, dxh, s) : launch_rms_bwd_k<float>(a, rs, dxh, s);
  if (e != hipSuccess) return e;
  if (a.dw) {  // dW [N, K] = dy^T [N, M] x̃ [M, K]
    const int64_t ch = dw_chunks(a.M, a.N, a.K);
    if (ch > 1) {
      const int64_t mc = a.M / ch;
      e = sgemm_rm_batched(true, false, a.N, a.K, mc, a.dy, a.ld_dy, mc * a.ld_dy, xt, a.K, mc * a.K, dwp, a.K,
                           a.N * a.K, ch, s);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_sum_chunks, dim3((unsigned)cdiv(a.N * a.K, 256)), dim3(256), 0, s, dwp, a.N * a.K, ch,
                         a.dw);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
      e = sgemm_rm(true, false, a.N, a.K, a.M, a.dy, a.ld_dy, xt, a.K, a.dw, a.K, s);
      if (e != hipSuccess) return e;
    }
  }
  if (a.dscale) {
    const int64_t segs = a.group ? a.N * (a.K / a.group) : a.N;
    float* dst = a.group ? a.dscale : part;
    hipLaunchKernelGGL(k_scale_grad, dim3((unsigned)cdiv(segs, 4)), dim3(256), 0, s, a.dw, a.w_latent, a.scale, a.N,
                       a.K, a.group, dst);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!a.group) {
      hipLaunchKernelGGL(k_sum_rows, dim3(1), dim3(64), 0, s, part, a.N, a.dscale);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_sgd(float* w, const float* dw, int64_t n, float lr, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_sgd, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, w, dw, n, lr);
  return hipGetLastError();
}

}  // namespace ssm
