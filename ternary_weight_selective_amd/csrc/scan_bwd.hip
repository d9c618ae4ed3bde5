// Backward of the Mamba-1 kind selective scan (the training side of the mixer; TriSSM README:
// trained end to end): the exact reverse-mode derivative of the recurrence the forward kernel
// evaluates.  With dt_t = softplus(delta_t + bias), a_t = exp(dt_t A), h_t = a_t h_{t-1} +
// dt_t x_t B_t, y_t = C_t . h_t + D x_t, the state adjoint is g_t = C_t dy_t + a_{t+1} g_{t+1}.
//
// Time is cut into chunks of LC steps and every chunk of every (sequence, channel tile) is a
// block of its own, so the work is spread over B x tiles x chunks blocks.  Both recurrences are
// linear in their carried value, so each chunk's contribution can be formed from a zero carry
// and the chunks joined afterwards (the forward scan's chunking, applied to both directions):
//   1. local: per chunk, the state reached from a zero state (S), the sum of dt (the chunk's
//      decay is exp(A sum dt)) and the adjoint carry leaving the chunk at its start from a zero
//      carry at its end (GL);
//   2. combine: per (sequence, channel, state), in chunk order, S becomes the state at the end
//      of each chunk (starting from h0), then in reverse order GL becomes the carry entering
//      each chunk at its end; what leaves chunk 0 is dh0;
//   3. chunk: per chunk, the states are re-run from the state entering it (kept in registers,
//      one per step and state) and time walked backwards with the true carry, giving dx, d
//      delta and the partial sums of dA, dD, d bias (per chunk) and of dB, dC (per channel tile);
//   4. sums of those partials in a fixed order (results do not depend on timing).
// Thread layout as in the forward: a block owns 64 channels (lane = channel), wave w the states
// w NS/4 .. w NS/4 + NS/4 - 1.  A chunk's inputs are staged once into LDS.
#include "scan_bwd.hpp"

namespace ssm {

namespace {
constexpr float kLog2eB = 1.4426950408889634f;
constexpr int kCPBb = 64;

// the forward's softplus (the same operations)
__device__ __forceinline__ float softplus_b(float v) {
  const float z = __builtin_amdgcn_exp2f(v * kLog2eB);
  const float u = 1.0f + z;
  const float c = u < 2.0f ? (u - 1.0f) - z : 0.0f;  // the rounding of u below 2, subtracted from log(u)
  const float big = 0.69314718055994531f * __builtin_amdgcn_logf(u) - c;
  const float small = z * __builtin_fmaf(-0.5f, z, 1.0f);
  const float r = z < 1e-4f ? small : big;
  return v > 20.0f ? v : r;
}

// lane value exchanged with lane ^ MASK
template <int MASK> __device__ __forceinline__ float xchg(float v) {
  const int i = __float_as_int(v);
  if constexpr (MASK == 32) return __int_as_float(__shfl_xor(i, 32, 64));
  else if constexpr (MASK == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, false));
  else if constexpr (MASK == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, false));
  else return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x1F | (MASK << 10)));  // bit-mask mode: lane ^ MASK
}

// one round of a transposed wave sum over the values a[0 .. W): lanes whose bit MASK is clear
// keep the first half, the others the second, each adding its partner's copy of what it keeps
template <int MASK, int W, int V>
__device__ __forceinline__ void xsum_round(float (&a)[V], int lane) {
  if constexpr (W > 1) {
    const bool hi = (lane & MASK) != 0;
#pragma unroll
    for (int j = 0; j < W / 2; ++j) {
      const float keep = hi ? a[W / 2 + j] : a[j];
      const float send = hi ? a[j] : a[W / 2 + j];
      a[j] = keep + xchg<MASK>(send);
    }
  } else {
    a[0] = a[0] + xchg<MASK>(a[0]);
  }
}

// V sums over the 64 lanes at once (V a power of two up to 32): afterwards lane l holds the
// sum of value l >> (6 - log2 V).  Each value is added up in a fixed tree, the same on every run.
template <int V> __device__ __forceinline__ float wave_sum_transposed(float (&a)[V], int lane) {
  xsum_round<32, V, V>(a, lane);
  xsum_round<16, (V >= 2 ? V / 2 : 1), V>(a, lane);
  xsum_round<8, (V >= 4 ? V / 4 : 1), V>(a, lane);
  xsum_round<4, (V >= 8 ? V / 8 : 1), V>(a, lane);
  xsum_round<2, (V >= 16 ? V / 16 : 1), V>(a, lane);
  xsum_round<1, (V >= 32 ? V / 32 : 1), V>(a, lane);
  return a[0];
}
template <int V> constexpr int log2c() { return V <= 1 ? 0 : 1 + log2c<V / 2>(); }

// steps per chunk: the chunk's states (LC x NS/4 per lane) stay in registers in pass 3
template <int NS> constexpr int bwd_chunk() {
  return NS >= 64 ? 4 : (NS >= 32 ? 8 : (NS >= 16 ? 16 : (NS >= 8 ? 32 : 64)));
}

// A chunk's inputs in LDS: per (step, channel) dt (0 past the end), softplus'(pre), x and dy
// (0 for channels past the last), per (step, state) B and C.
template <int NS, int LC> struct ChunkLds {
  float dt[LC][kCPBb], sig[LC][kCPBb], x[LC][kCPBb], dy[LC][kCPBb];
  float B[LC][NS], C[LC][NS];
};

template <int NS, int LC, typename T>
__device__ __forceinline__ void stage_chunk(const ScanBwdArgs& a, ChunkLds<NS, LC>& s, int64_t b, int64_t dc, bool dv,
                                            int64_t t0, int64_t t1, float bias) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t L = a.L;
#pragma unroll
  for (int j = 0; j < (LC + 3) / 4; ++j) {
    const int u = w + 4 * j;
    if (u >= LC) break;
    const int64_t t = t0 + u;
    const bool ok = t < t1;
    const int64_t tok = b * L + (ok ? t : t0);  // past the end: a valid row, zeroed below
    const float pre = ld_act((const T*)a.delta + tok * a.ld_delta + dc) + bias;
    float dt, sg;
    if (a.softplus) {
      sg = pre > 20.0f ? 1.0f : 1.0f / (1.0f + __builtin_amdgcn_exp2f(-pre * kLog2eB));
      dt = softplus_b(pre);
    } else {
      sg = 1.0f;
      dt = pre;
    }
    const float xv = ld_act((const T*)a.x + tok * a.ld_x + dc);
    const float dyv = a.dy[tok * a.ld_dy + dc];
    s.dt[u][lane] = ok ? dt : 0.0f;
    s.sig[u][lane] = sg;
    s.x[u][lane] = (ok && dv) ? xv : 0.0f;
    s.dy[u][lane] = (ok && dv) ? dyv : 0.0f;
  }
  for (int e = threadIdx.x; e < LC * NS; e += 256) {
    const int u = e / NS, n = e % NS;
    const int64_t t = t0 + u;
    const int64_t tok = b * L + (t < t1 ? t : t0);
    s.B[u][n] = ld_act((const T*)a.Bm + tok * a.ld_B + n);
    s.C[u][n] = ld_act((const T*)a.Cm + tok * a.ld_C + n);
  }
}

struct ChunkBufs {
  float *S, *SD, *GL;      // [B][NC][H][NS], [B][NC][H], [B][NC][H][NS]
  float *pB, *pC;          // [B L][tiles][NS]
  float *pA, *pD, *pbias;  // [B][NC][H][NS], [B][NC][H], [B][NC][H]
  int64_t nc;
};

// pass 1: per chunk, the state from a zero state, sum dt, and the adjoint carry from a zero carry
template <int NS, typename T>
__global__ __launch_bounds__(256) void k_bwd_local(ScanBwdArgs a, ChunkBufs cb) {
  constexpr int SPL = NS / 4, LC = bwd_chunk<NS>();
  __shared__ ChunkLds<NS, LC> s;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t b = blockIdx.x, c = blockIdx.z, H = a.H, L = a.L;
  const int64_t d = (int64_t)blockIdx.y * kCPBb + lane;
  const bool dv = d < H;
  const int64_t dc = dv ? d : H - 1;
  const int64_t t0 = c * LC, t1 = (t0 + LC < L) ? t0 + LC : L;
  const float bias = a.delta_bias ? a.delta_bias[dc] : 0.0f;
  float Al[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) Al[i] = a.A[dc * NS + w * SPL + i] * kLog2eB;
  stage_chunk<NS, LC, T>(a, s, b, dc, dv, t0, t1, bias);
  __syncthreads();
  float h[SPL], g[SPL], sdt = 0.0f;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    h[i] = 0.0f;
    g[i] = 0.0f;
  }
  float ra[LC][SPL];  // a_t of the chunk's steps, for the reverse loop
#pragma unroll
  for (int u = 0; u < LC; ++u) {  // steps past the end have dt = 0: a = 1, nothing added
    const float dt = s.dt[u][lane], dx = dt * s.x[u][lane];
    sdt += dt;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      ra[u][i] = __builtin_amdgcn_exp2f(dt * Al[i]);
      h[i] = __builtin_fmaf(ra[u][i], h[i], dx * s.B[u][w * SPL + i]);
    }
  }
#pragma unroll
  for (int u = LC - 1; u >= 0; --u) {  // past the end: dy = 0 and a = 1, the carry passes through
    const float dyv = s.dy[u][lane];
#pragma unroll
    for (int i = 0; i < SPL; ++i) g[i] = ra[u][i] * __builtin_fmaf(s.C[u][w * SPL + i], dyv, g[i]);
  }
  if (dv) {
    const int64_t si = ((b * cb.nc + c) * H + d) * NS + w * SPL;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      cb.S[si + i] = h[i];
      cb.GL[si + i] = g[i];
    }
    if (w == 0) cb.SD[(b * cb.nc + c) * H + d] = sdt;
  }
}

// pass 2: per (sequence, channel, state), the chunks joined in order: S[c] becomes the state at
// the end of chunk c, GL[c] the adjoint carry entering chunk c at its end; dh0 what leaves chunk 0
__global__ __launch_bounds__(256) void k_bwd_combine(const float* __restrict__ A, const float* __restrict__ h0,
                                                     ChunkBufs cb, int64_t B, int64_t H, int NS,
                                                     float* __restrict__ dh0) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * H * NS) return;
  const int64_t b = i / (H * NS), dn = i % (H * NS), d = dn / NS;
  const float a2 = A[dn] * kLog2eB;
  const int64_t sb = b * cb.nc * H * NS + dn, db = b * cb.nc * H + d;  // chunk 0 of this element
  constexpr int G = 8;  // chunks whose loads are in flight together
  float h = h0 ? h0[i] : 0.0f;
  for (int64_t c0 = 0; c0 < cb.nc; c0 += G) {
    float sv[G], P[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int64_t c = c0 + u < cb.nc ? c0 + u : cb.nc - 1;
      sv[u] = cb.S[sb + c * H * NS];
      P[u] = cb.SD[db + c * H];
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (c0 + u >= cb.nc) break;
      h = __builtin_fmaf(__builtin_amdgcn_exp2f(a2 * P[u]), h, sv[u]);
      cb.S[sb + (c0 + u) * H * NS] = h;
    }
  }
  float gam = 0.0f;
  for (int64_t c1 = cb.nc - 1; c1 >= 0; c1 -= G) {  // chunks c1, c1 - 1, ..., c1 - G + 1
    float gv[G], P[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int64_t c = c1 - u >= 0 ? c1 - u : 0;
      gv[u] = cb.GL[sb + c * H * NS];
      P[u] = cb.SD[db + c * H];
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (c1 - u < 0) break;
      cb.GL[sb + (c1 - u) * H * NS] = gam;
      gam = __builtin_fmaf(__builtin_amdgcn_exp2f(a2 * P[u]), gam, gv[u]);
    }
  }
  if (dh0) dh0[i] = gam;
}

// pass 3: per chunk, states re-run from the state entering it, then time walked backwards
template <int NS, typename T>
__global__ __launch_bounds__(256) void k_bwd_chunk(ScanBwdArgs a, ChunkBufs cb) {
  constexpr int SPL = NS / 4, LC = bwd_chunk<NS>();
  __shared__ ChunkLds<NS, LC> s;
  __shared__ float s_red[2][2][4][kCPBb];  // [step parity][d dt, sum g B][wave][channel]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t b = blockIdx.x, tile = blockIdx.y, c = blockIdx.z, H = a.H, L = a.L;
  const int64_t ntile = gridDim.y;
  const int64_t d = tile * kCPBb + lane;
  const bool dv = d < H;
  const int64_t dc = dv ? d : H - 1;  // lanes past the last channel run on zeros
  const int64_t t0 = c * LC, t1 = (t0 + LC < L) ? t0 + LC : L;
  const float bias = a.delta_bias ? a.delta_bias[dc] : 0.0f;
  const float Dd = a.D ? a.D[dc] : 0.0f;
  float Av[SPL], Al[SPL], h[SPL], g[SPL], dA[SPL];
  const int64_t si = ((b * cb.nc + c) * H + dc) * NS + w * SPL;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int n = w * SPL + i;
    Av[i] = a.A[dc * NS + n];
    Al[i] = Av[i] * kLog2eB;
    h[i] = c > 0 ? cb.S[si - H * NS + i] : (a.h0 ? a.h0[(b * H + dc) * NS + n] : 0.0f);
    g[i] = dv ? cb.GL[si + i] : 0.0f;  // a_{t+1} g_{t+1} entering the chunk's last step
    dA[i] = 0.0f;
  }
  stage_chunk<NS, LC, T>(a, s, b, dc, dv, t0, t1, bias);
  __syncthreads();
  // the chunk's states: hp[u] = h_{t0 + u - 1} (a_t is recomputed in the reverse loop: kept
  // here it costs more in occupancy than the exponentials it saves)
  float hp[LC][SPL];
#pragma unroll
  for (int u = 0; u < LC; ++u) {
    const float dt = s.dt[u][lane], dx = dt * s.x[u][lane];
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      hp[u][i] = h[i];
      h[i] = __builtin_fmaf(__builtin_amdgcn_exp2f(dt * Al[i]), h[i], dx * s.B[u][w * SPL + i]);
    }
  }
  float dD = 0.0f, dbias = 0.0f;
  // h holds h_t of the step being processed (steps past the end left it unchanged)
#pragma unroll
  for (int u = LC - 1; u >= 0; --u) {
    const int64_t t = t0 + u;
    if (t >= t1) continue;  // the same for the whole block
    const int64_t tok = b * L + t;
    const float dt = s.dt[u][lane], sig = s.sig[u][lane];
    const float xv = s.x[u][lane], dyv = s.dy[u][lane];
    float pddt = 0.0f, pgb = 0.0f;
    float red[2 * SPL];  // this lane's dB (first SPL) and dC terms of the wave's states
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int n = w * SPL + i;
      const float Bn = s.B[u][n], Cn = s.C[u][n];
      const float hprev = hp[u][i];
      const float ab = __builtin_amdgcn_exp2f(dt * Al[i]);
      const float gi = dv ? __builtin_fmaf(Cn, dyv, g[i]) : 0.0f;
      const float gha = gi * hprev * ab;
      pddt = __builtin_fmaf(gha, Av[i], __builtin_fmaf(gi * xv, Bn, pddt));
      pgb = __builtin_fmaf(gi, Bn, pgb);
      dA[i] = __builtin_fmaf(gha, dt, dA[i]);
      red[i] = gi * dt * xv;
      red[SPL + i] = dyv * h[i];  // dy is 0 past the last channel
      g[i] = ab * gi;
      h[i] = hprev;
    }
    {  // dB and dC over the block's channels: one lane per value stores it
      constexpr int K = log2c<2 * SPL>();
      const float r = wave_sum_transposed<2 * SPL>(red, lane);
      const int j = lane >> (6 - K);
      if ((lane & ((64 >> K) - 1)) == 0) {
        float* dst = j < SPL ? cb.pB : cb.pC;
        dst[(tok * ntile + tile) * NS + w * SPL + (j < SPL ? j : j - SPL)] = r;
      }
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
  if (dv) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) cb.pA[si + i] = dA[i];
    if (w == 0) {
      cb.pD[(b * cb.nc + c) * H + dc] = dD;
      cb.pbias[(b * cb.nc + c) * H + dc] = dbias;
    }
  }
}

// sum of in[(base + m) * inner + i] over m in [m0, m1), m ascending, eight loads in flight
__device__ __forceinline__ float sum_rows(const float* __restrict__ in, int64_t base, int64_t m0, int64_t m1,
                                          int64_t inner, int64_t i) {
  float s = 0.0f;
  int64_t m = m0;
  for (; m + 8 <= m1; m += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = in[(base + m + u) * inner + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; m < m1; ++m) s += in[(base + m) * inner + i];
  return s;
}

// out[o, i] = sum over m of in[o, m, i], m ascending
__global__ __launch_bounds__(256) void k_sum_mid(const float* __restrict__ in, int64_t outer, int64_t mid,
                                                 int64_t inner, float* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= outer * inner) return;
  const int64_t o = e / inner, i = e % inner;
  out[e] = sum_rows(in, o * mid, 0, mid, inner, i);
}

// first level of a long sum: part[g, i] = sum over m in segment g (seg rows) of in[m, i]
__global__ __launch_bounds__(256) void k_sum_seg(const float* __restrict__ in, int64_t mid, int64_t inner, int64_t seg,
                                                 float* __restrict__ part) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x, g = blockIdx.y;
  if (i >= inner) return;
  const int64_t m0 = g * seg, m1 = (m0 + seg < mid) ? m0 + seg : mid;
  part[g * inner + i] = sum_rows(in, 0, m0, m1, inner, i);
}

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

int chunk_len(int64_t N) {
  switch (N) {
    case 4: return bwd_chunk<4>();
    case 8: return bwd_chunk<8>();
    case 16: return bwd_chunk<16>();
    case 32: return bwd_chunk<32>();
    default: return bwd_chunk<64>();
  }
}

struct BwdPlan {
  size_t off_S, off_SD, off_GL, off_pB, off_pC, off_pA, off_pD, off_pbias, total;
  int64_t ntile, nc;
};
BwdPlan plan_bwd(const ScanBwdArgs& a) {
  BwdPlan p{};
  p.ntile = cdiv(a.H, kCPBb);
  p.nc = cdiv(a.L, chunk_len(a.N));
  const int64_t M = a.batch * a.L, BC = a.batch * p.nc;
  size_t off = 0;
  p.off_S = off; off += al256((size_t)BC * a.H * a.N * 4);
  p.off_SD = off; off += al256((size_t)BC * a.H * 4);
  p.off_GL = off; off += al256((size_t)BC * a.H * a.N * 4);
  p.off_pB = off; off += al256((size_t)M * p.ntile * a.N * 4);
  p.off_pC = off; off += al256((size_t)M * p.ntile * a.N * 4);
  p.off_pA = off; off += al256((size_t)BC * a.H * a.N * 4);
  p.off_pD = off; off += al256((size_t)BC * a.H * 4);
  p.off_pbias = off; off += al256((size_t)BC * a.H * 4);
  p.total = off;
  return p;
}

template <int NS, typename T>
hipError_t launch_bwd_t(const ScanBwdArgs& a, void* ws, hipStream_t s) {
  const BwdPlan p = plan_bwd(a);
  char* base = (char*)ws;
  ChunkBufs cb{};
  cb.S = (float*)(base + p.off_S);
  cb.SD = (float*)(base + p.off_SD);
  cb.GL = (float*)(base + p.off_GL);
  cb.pB = (float*)(base + p.off_pB);
  cb.pC = (float*)(base + p.off_pC);
  cb.pA = (float*)(base + p.off_pA);
  cb.pD = (float*)(base + p.off_pD);
  cb.pbias = (float*)(base + p.off_pbias);
  cb.nc = p.nc;
  const dim3 grid((unsigned)a.batch, (unsigned)p.ntile, (unsigned)p.nc), block(256);
  hipLaunchKernelGGL((k_bwd_local<NS, T>), grid, block, 0, s, a, cb);
  const int64_t ne = a.batch * a.H * NS;
  hipLaunchKernelGGL(k_bwd_combine, dim3((unsigned)cdiv(ne, 256)), dim3(256), 0, s, a.A, a.h0, cb, a.batch, a.H, NS,
                     a.dh0);
  hipLaunchKernelGGL((k_bwd_chunk<NS, T>), grid, block, 0, s, a, cb);
  const int64_t M = a.batch * a.L;
  // fixed-order sums; a long one (over sequences x chunks) in segments of 32 first, the
  // segment sums going to the chunk states' region, which is free once pass 3 has run
  auto sum = [&](const float* in, int64_t outer, int64_t mid, int64_t inner, float* out) {
    if (!out) return;
    if (outer == 1 && mid > 64) {
      const int64_t seg = 32, ns = cdiv(mid, seg);
      hipLaunchKernelGGL(k_sum_seg, dim3((unsigned)cdiv(inner, 256), (unsigned)ns), dim3(256), 0, s, in, mid, inner,
                         seg, cb.S);
      in = cb.S;
      mid = ns;
    }
    hipLaunchKernelGGL(k_sum_mid, dim3((unsigned)cdiv(outer * inner, 256)), dim3(256), 0, s, in, outer, mid, inner,
                       out);
  };
  sum(cb.pB, M, p.ntile, NS, a.dB);
  sum(cb.pC, M, p.ntile, NS, a.dC);
  sum(cb.pA, 1, a.batch * p.nc, a.H * NS, a.dA);
  sum(cb.pD, 1, a.batch * p.nc, a.H, a.dD);
  sum(cb.pbias, 1, a.batch * p.nc, a.H, a.dbias);
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
