// Backward of the Mamba-1 kind selective scan (the training side of the mixer; TriSSM README:
// trained end to end): the exact reverse-mode derivative of the recurrence the forward kernel
// evaluates.  With dt_t = softplus(delta_t + bias), a_t = exp(dt_t A), h_t = a_t h_{t-1} +
// dt_t x_t B_t, y_t = C_t . h_t + D x_t, the state adjoint is g_t = C_t dy_t + a_{t+1} g_{t+1}.
// Pass 1 re-runs the forward and stores every state; pass 2 walks time backwards; pass 3 sums,
// in a fixed order, the partial gradients of parameters that several blocks share (A, D and the
// delta bias over sequences; B and C over channel tiles).  Thread layout as in the forward: a
// block owns 64 channels of one sequence (lane = channel), wave w the states w NS/4 ...
#include "scan_bwd.hpp"

namespace ssm {

namespace {
constexpr float kLog2eB = 1.4426950408889634f;
constexpr int kCPBb = 64;

// the forward's softplus (the same operations)
__device__ __forceinline__ float softplus_b(float v) {
  const float z = __builtin_amdgcn_exp2f(v * kLog2eB);
  const float u = 1.0f + z;
  const float um1 = u - 1.0f;
  const float big = (0.69314718055994531f * __builtin_amdgcn_logf(u)) * (z * __builtin_amdgcn_rcpf(um1));
  const float small = z * __builtin_fmaf(-0.5f, z, 1.0f);
  const float r = z < 1e-4f ? small : big;
  return v > 20.0f ? v : r;
}

// steps per register tile of the two passes (the loads of the next tile are in flight while the
// current one is computed)
template <int SPL> constexpr int bwd_tile() { return SPL >= 16 ? 1 : (SPL >= 8 ? 2 : (SPL >= 4 ? 4 : 8)); }

// pass 1: the forward recurrence, storing h_t for every step: hs[b][t][d][n]
template <int NS, typename T>
__global__ __launch_bounds__(256) void k_scan_save(ScanBwdArgs a, float* __restrict__ hs) {
  constexpr int SPL = NS / 4, TT = bwd_tile<SPL>();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t b = blockIdx.x, d = (int64_t)blockIdx.y * kCPBb + lane, H = a.H, L = a.L;
  if (d >= H) return;  // no barriers in this kernel
  const float bias = a.delta_bias ? a.delta_bias[d] : 0.0f;
  float h[SPL], Al[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int n = w * SPL + i;
    Al[i] = a.A[d * NS + n] * kLog2eB;
    h[i] = a.h0 ? a.h0[(b * H + d) * NS + n] : 0.0f;
  }
  float rd[TT], rx[TT], rb[TT][SPL];
  auto load = [&](int64_t t0) {
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      const int64_t t = t0 + u;
      const bool ok = t < L;
      const int64_t tok = b * L + (ok ? t : 0);
      rd[u] = ok ? ld_act((const T*)a.delta + tok * a.ld_delta + d) : 0.0f;
      rx[u] = ok ? ld_act((const T*)a.x + tok * a.ld_x + d) : 0.0f;
#pragma unroll
      for (int i = 0; i < SPL; ++i) rb[u][i] = ok ? ld_act((const T*)a.Bm + tok * a.ld_B + w * SPL + i) : 0.0f;
    }
  };
  load(0);
  for (int64_t t0 = 0; t0 < L; t0 += TT) {
    float cd[TT], cx[TT], cb[TT][SPL];
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      cd[u] = rd[u];
      cx[u] = rx[u];
#pragma unroll
      for (int i = 0; i < SPL; ++i) cb[u][i] = rb[u][i];
    }
    if (t0 + TT < L) load(t0 + TT);
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      const int64_t t = t0 + u;
      if (t >= L) break;
      const float pre = cd[u] + bias;
      const float dt = a.softplus ? softplus_b(pre) : pre;
      const float dx = dt * cx[u];
      float* hr = hs + ((b * L + t) * H + d) * NS + w * SPL;
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const float ab = __builtin_amdgcn_exp2f(dt * Al[i]);
        h[i] = __builtin_fmaf(ab, h[i], dx * cb[u][i]);
        hr[i] = h[i];
      }
    }
  }
}

// pass 2: reverse time, TT steps per register tile (TT <= 2: the reverse step holds more)
template <int NS, typename T>
__global__ __launch_bounds__(256) void k_scan_rev(ScanBwdArgs a, const float* __restrict__ hs,
                                                  float* __restrict__ pB, float* __restrict__ pC,
                                                  float* __restrict__ pA, float* __restrict__ pD,
                                                  float* __restrict__ pbias) {
  constexpr int SPL = NS / 4, TT = bwd_tile<SPL>() > 2 ? 2 : bwd_tile<SPL>();
  __shared__ float s_red[2][2][4][kCPBb];  // [step parity][d dt, sum g B][wave][channel]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t b = blockIdx.x, tile = blockIdx.y, d = tile * kCPBb + lane, H = a.H, L = a.L;
  const int64_t ntile = gridDim.y;
  const bool dv = d < H;
  const int64_t dc = dv ? d : H - 1;  // lanes past the last channel run on zeros
  const float bias = a.delta_bias ? a.delta_bias[dc] : 0.0f;
  const float Dd = a.D ? a.D[dc] : 0.0f;
  float Av[SPL], Al[SPL], g[SPL], dA[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    Av[i] = a.A[dc * NS + w * SPL + i];
    Al[i] = Av[i] * kLog2eB;
    g[i] = 0.0f;  // a_{t+1} g_{t+1}
    dA[i] = 0.0f;
  }
  float dD = 0.0f, dbias = 0.0f;
  // per step: pre-activation dt, x, dy, B, C and h_{t-1}; h_t is the previous step's h_{t-1}
  float rd[TT], rx[TT], ry[TT], rB[TT][SPL], rC[TT][SPL], rh[TT][SPL];
  auto load = [&](int64_t t1) {  // steps t1, t1 - 1, ..., t1 - TT + 1
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      const int64_t t = t1 - u;
      const bool ok = t >= 0;
      const int64_t tok = b * L + (ok ? t : 0);
      rd[u] = ok ? ld_act((const T*)a.delta + tok * a.ld_delta + dc) : 0.0f;
      rx[u] = (ok && dv) ? ld_act((const T*)a.x + tok * a.ld_x + dc) : 0.0f;
      ry[u] = (ok && dv) ? a.dy[tok * a.ld_dy + dc] : 0.0f;
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int n = w * SPL + i;
        rB[u][i] = ok ? ld_act((const T*)a.Bm + tok * a.ld_B + n) : 0.0f;
        rC[u][i] = ok ? ld_act((const T*)a.Cm + tok * a.ld_C + n) : 0.0f;
        rh[u][i] = t > 0 ? hs[((tok - 1) * H + dc) * NS + n]
                         : ((ok && a.h0) ? a.h0[(b * H + dc) * NS + n] : 0.0f);
      }
    }
  };
  float ht[SPL];  // h_t of the current step
#pragma unroll
  for (int i = 0; i < SPL; ++i) ht[i] = hs[((b * L + L - 1) * H + dc) * NS + w * SPL + i];
  load(L - 1);
  for (int64_t t1 = L - 1; t1 >= 0; t1 -= TT) {
    float cd[TT], cx[TT], cy[TT], cB[TT][SPL], cC[TT][SPL], ch[TT][SPL];
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      cd[u] = rd[u]; cx[u] = rx[u]; cy[u] = ry[u];
#pragma unroll
      for (int i = 0; i < SPL; ++i) { cB[u][i] = rB[u][i]; cC[u][i] = rC[u][i]; ch[u][i] = rh[u][i]; }
    }
    if (t1 - TT >= 0) load(t1 - TT);
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      const int64_t t = t1 - u;
      if (t < 0) break;
      const int64_t tok = b * L + t;
      const float pre = cd[u] + bias;
      float dt, sig;
      if (a.softplus) {
        sig = pre > 20.0f ? 1.0f : 1.0f / (1.0f + __builtin_amdgcn_exp2f(-pre * kLog2eB));
        dt = softplus_b(pre);
      } else {
        sig = 1.0f;
        dt = pre;
      }
      const float xv = cx[u], dyv = cy[u];
      float pddt = 0.0f, pgb = 0.0f;
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int n = w * SPL + i;
        const float Bn = cB[u][i], Cn = cC[u][i];
        const float hprev = ch[u][i];
        const float ab = __builtin_amdgcn_exp2f(dt * Al[i]);
        const float gi = dv ? __builtin_fmaf(Cn, dyv, g[i]) : 0.0f;
        const float gha = gi * hprev * ab;
        pddt = __builtin_fmaf(gha, Av[i], __builtin_fmaf(gi * xv, Bn, pddt));
        pgb = __builtin_fmaf(gi, Bn, pgb);
        dA[i] = __builtin_fmaf(gha, dt, dA[i]);
        const float cb = wave_sum_butterfly(gi * dt * xv);            // dB over the block's channels
        const float cc = wave_sum_butterfly(dv ? dyv * ht[i] : 0.0f);  // dC
        if (lane == 0) {
          pB[(tok * ntile + tile) * NS + n] = cb;
          pC[(tok * ntile + tile) * NS + n] = cc;
        }
        g[i] = ab * gi;
        ht[i] = hprev;
      }
      const int par = (int)(t & 1);
      s_red[par][0][w][lane] = pddt;
      s_red[par][1][w][lane] = pgb;
      __syncthreads();  // one barrier per step: the other parity's buffer is free
      if (w == 0 && dv) {
        const float ddt = ((s_red[par][0][0][lane] + s_red[par][0][1][lane]) + s_red[par][0][2][lane]) +
                          s_red[par][0][3][lane];
        const float sgb = ((s_red[par][1][0][lane] + s_red[par][1][1][lane]) + s_red[par][1][2][lane]) +
                          s_red[par][1][3][lane];
        const float ddl = ddt * sig;
        a.ddelta[tok * H + dc] = ddl;
        a.dx[tok * H + dc] = __builtin_fmaf(Dd, dyv, dt * sgb);
        dbias += ddl;
        dD = __builtin_fmaf(dyv, xv, dD);
      }
    }
  }
  if (dv) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int n = w * SPL + i;
      pA[(b * H + dc) * NS + n] = dA[i];
      if (a.dh0) a.dh0[(b * H + dc) * NS + n] = g[i];
    }
    if (w == 0) {
      pD[b * H + dc] = dD;
      pbias[b * H + dc] = dbias;
    }
  }
}

// out[o, i] = sum over m of in[o, m, i], m ascending
__global__ __launch_bounds__(256) void k_sum_mid(const float* __restrict__ in, int64_t outer, int64_t mid,
                                                 int64_t inner, float* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= outer * inner) return;
  const int64_t o = e / inner, i = e % inner;
  float s = 0.0f;
  for (int64_t m = 0; m < mid; ++m) s += in[(o * mid + m) * inner + i];
  out[e] = s;
}

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

struct BwdPlan {
  size_t off_hs, off_pB, off_pC, off_pA, off_pD, off_pbias, total;
  int64_t ntile;
};
BwdPlan plan_bwd(const ScanBwdArgs& a) {
  BwdPlan p{};
  p.ntile = cdiv(a.H, kCPBb);
  const int64_t M = a.batch * a.L;
  size_t off = 0;
  p.off_hs = off; off += al256((size_t)M * a.H * a.N * 4);
  p.off_pB = off; off += al256((size_t)M * p.ntile * a.N * 4);
  p.off_pC = off; off += al256((size_t)M * p.ntile * a.N * 4);
  p.off_pA = off; off += al256((size_t)a.batch * a.H * a.N * 4);
  p.off_pD = off; off += al256((size_t)a.batch * a.H * 4);
  p.off_pbias = off; off += al256((size_t)a.batch * a.H * 4);
  p.total = off;
  return p;
}

template <int NS, typename T>
hipError_t launch_bwd_t(const ScanBwdArgs& a, void* ws, hipStream_t s) {
  const BwdPlan p = plan_bwd(a);
  char* base = (char*)ws;
  float* hs = (float*)(base + p.off_hs);
  float* pB = (float*)(base + p.off_pB);
  float* pC = (float*)(base + p.off_pC);
  float* pA = (float*)(base + p.off_pA);
  float* pD = (float*)(base + p.off_pD);
  float* pb = (float*)(base + p.off_pbias);
  const dim3 grid((unsigned)a.batch, (unsigned)p.ntile), block(256);
  hipLaunchKernelGGL((k_scan_save<NS, T>), grid, block, 0, s, a, hs);
  hipLaunchKernelGGL((k_scan_rev<NS, T>), grid, block, 0, s, a, hs, pB, pC, pA, pD, pb);
  const int64_t M = a.batch * a.L;
  auto sum = [&](const float* in, int64_t outer, int64_t mid, int64_t inner, float* out) {
    if (!out) return;
    hipLaunchKernelGGL(k_sum_mid, dim3((unsigned)cdiv(outer * inner, 256)), dim3(256), 0, s, in, outer, mid, inner,
                       out);
  };
  sum(pB, M, p.ntile, NS, a.dB);
  sum(pC, M, p.ntile, NS, a.dC);
  sum(pA, 1, a.batch, a.H * NS, a.dA);
  sum(pD, 1, a.batch, a.H, a.dD);
  sum(pb, 1, a.batch, a.H, a.dbias);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_n(const ScanBwdArgs& a, void* ws, hipStream_t s) {
  switch (a.N) {
    case 4: return launch_bwd_t<4, T>(a, ws, s);
    case 8: return launch_bwd_t<8, T>(a, ws, s);
    case 16: return launch_bwd_t<16, T>(a, ws, s);
    case 32: return launch_bwd_t<32, T>(a, ws, s);
    case 64: return launch_bwd_t<64, T>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

size_t scan_bwd_workspace(const ScanBwdArgs& a) { return plan_bwd(a).total; }

hipError_t launch_scan_bwd(const ScanBwdArgs& a, void* ws, hipStream_t s) {
  if (a.batch == 0 || a.L == 0) return hipSuccess;
  return a.act_bf16 ? launch_bwd_n<bf16_t>(a, ws, s) : launch_bwd_n<float>(a, ws, s);
}

}  // namespace ssm
