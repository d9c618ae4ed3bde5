// Short causal depthwise convolution with SiLU on the SSM input: the block that Mamba
// ("Linear-Time Sequence Modeling with Selective State Spaces", cited under "Builds on")
// wraps around the selective scan, and the gated diagonal-SSM block of "Baseline Shape
// Decides the Verdict ..." (abstract, finding (ii)).
//   a[b, t, c] = bias[c] + sum_{j < K} w[c, j] x[b, t - K + 1 + j, c];   out = a / (1 + exp(-a))
// The output feeds the int8 quantisation of x_proj's input, so it is computed in fp64 (sum in
// the order above, no contraction: this file is compiled with -ffp-contract=off) and rounded
// once to the activation type; the value is then independent of how the work is split.
// HBM-bound: one read and one write of each element (plus K - 1 halo rows per time chunk).
#include "launch.hpp"

namespace ssm {

namespace {
constexpr int kConvT = 16;  // time steps per thread

// thread: channel c (lanes of a wave take consecutive channels: coalesced rows), one chunk of
// time steps of one sequence; the K - 1 inputs before the chunk come from x, or from the
// carried state before t = 0, or are zero
template <typename T, int K>
__global__ __launch_bounds__(256) void k_conv_silu(ConvArgs a, int64_t chunk_len) {
  const int64_t c = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t chunk = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  const int64_t b = blockIdx.z;
  const int64_t t0 = chunk * chunk_len;
  if (c >= a.C || t0 >= a.L) return;
  const int64_t t1 = (t0 + chunk_len < a.L) ? t0 + chunk_len : a.L;
  const T* X = (const T*)a.x;
  T* O = (T*)a.out;
  double wk[K];
#pragma unroll
  for (int j = 0; j < K; ++j) wk[j] = (double)a.w[c * K + j];
  const double bias = a.bias ? (double)a.bias[c] : 0.0;
  // window: win[j] holds the input at time t - K + 1 + j for the current t (j < K - 1)
  float win[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t ts = t0 - (K - 1) + j;
    float v = 0.0f;
    if (ts >= 0) v = ld_act(X + (b * a.L + ts) * a.ldx + c);
    else if (a.state_in) v = a.state_in[(b * (K - 1) + (ts + K - 1)) * a.C + c];
    win[j] = v;
  }
  auto step = [&](float xv, int64_t t) {
    double acc = bias;
#pragma unroll
    for (int j = 0; j < K - 1; ++j) acc = acc + wk[j] * (double)win[j];
    acc = acc + wk[K - 1] * (double)xv;
    const double sv = acc / (1.0 + exp(-acc));
    st_act(O + (b * a.L + t) * a.ldo + c, (float)sv);
#pragma unroll
    for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
    if (K > 1) win[K > 1 ? K - 2 : 0] = xv;
  };
  for (int64_t t = t0; t < t1; ++t) step(ld_act(X + (b * a.L + t) * a.ldx + c), t);
  // the state after the sequence: its last K - 1 inputs (the window after the last step)
  if (a.state_out && t1 == a.L) {
#pragma unroll
    for (int j = 0; j < K - 1; ++j) a.state_out[(b * (K - 1) + j) * a.C + c] = win[j];
  }
}

template <typename T>
void launch_k(const ConvArgs& a, int64_t chunk_len, hipStream_t s) {
  const int64_t nch = cdiv(a.L, chunk_len);
  const dim3 grid((unsigned)cdiv(a.C, 64), (unsigned)cdiv(nch, 4), (unsigned)a.batch), block(256);
  switch (a.K) {
#define SSM_CONV(KK) case KK: hipLaunchKernelGGL((k_conv_silu<T, KK>), grid, block, 0, s, a, chunk_len); break;
    SSM_CONV(1) SSM_CONV(2) SSM_CONV(3) SSM_CONV(4) SSM_CONV(5) SSM_CONV(6) SSM_CONV(7) SSM_CONV(8)
#undef SSM_CONV
    default: break;
  }
}
}  // namespace

hipError_t launch_conv_silu(const ConvArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.L == 0 || a.C == 0) return hipSuccess;
  if (a.K < 1 || a.K > kConvMaxK) return hipErrorInvalidValue;
  // a state updated in place is read (first chunk) and written (last chunk) by one thread
  const bool in_place = a.state_in && a.state_out && (const void*)a.state_in == (const void*)a.state_out;
  const int64_t chunk_len = in_place ? a.L : kConvT;
  if (a.act_bf16) launch_k<bf16_t>(a, chunk_len, s);
  else launch_k<float>(a, chunk_len, s);
  return hipGetLastError();
}

}  // namespace ssm
