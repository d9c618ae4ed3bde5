// Selective scan, Mamba-1 kind (Mamba, cited by title in "Baseline Shape Decides the
// Verdict ...", Builds on; TriSSM README: input-dependent Delta, B, C, and the recurrence
// evaluated with a parallel associative scan).  A is per (channel, state); one channel per
// head.
//
// Work split.  A block owns 64 channels (the lanes) of one sequence and one time chunk; its
// 4 waves split the NS states into 4 groups, so that B and C of a step are the same for a
// whole wave: they are read from LDS at wave-uniform addresses (a broadcast), for a group of
// steps at a time with one wait.  Each lane runs the recurrence of NS / 4 states over time in
// registers: per state and step one exp2 (A is pre-scaled by log2 e), two multiplies and two
// fused multiply-adds; the kernel is bound by VALU issue.  The waves' readout partials meet
// in LDS and are added in wave order.
//
// Time is staged through LDS in tiles of 32 steps: the next tile's x, B, C (and dt input
// codes) are loaded into registers, coalesced, while the current tile runs.
//
// Chunks (the carried inter-chunk state).  When batch x channel tiles give too few blocks
// to fill the chip, the sequence is cut into T chunks: pass 1 runs every chunk but the last
// from a zero state and keeps its end state h_loc and sum(dt); pass 2 composes the chunks
// in order with the associative operator (P, h_loc) o h = P * h + h_loc, P = exp(A sum dt);
// pass 3 reruns every chunk from its true incoming state and writes y.
//
// Optionally (the mixer path) dt is the A8 BitLinear of a low-rank input dr (k = R <= 64
// columns), computed here: a pre-kernel RMS-normalises and absmax-quantises each token's
// row once, with a group of 16..64 lanes in the same fixed order as the standalone
// BitLinear (for k <= 64 the 64-lane butterfly reduces to the group's butterfly plus exact
// zero additions); in the scan each channel's int32 dot product with its ternary weight
// row is v_dot4 instructions, and the dequantisation is the BitLinear epilogue's fp64
// expression.
#include <type_traits>

#include "launch.hpp"

namespace ssm {

namespace {
constexpr float LOG2E = 1.4426950408889634f;
constexpr int RMAX = 64;

// softplus(v) = log(1 + e^v), the identity above 20.  With z = e^v and u = fl(1 + z), the
// rounding of u is c = (u - 1) - z (exact while u < 2, and below an ulp of the result above),
// and log1p(z) = log(u) - c / u + O(c^2); taking c for c / u changes the result by at most
// |c| z / (1 + z) <= 2^-24 min(z, 1), below its own rounding.  Below z = 1e-4 the series
// z - z^2 / 2 is used.  Branch-free, on the hardware exp2 and log2 (no reciprocal).
__device__ __forceinline__ float softplus_f(float v) {
  const float z = __builtin_amdgcn_exp2f(v * LOG2E);
  const float u = 1.0f + z;
  const float c = (u - 1.0f) - z;
  const float big = 0.69314718055994531f * __builtin_amdgcn_logf(u) - c;
  const float small = z * __builtin_fmaf(-0.5f, z, 1.0f);
  const float r = z < 1e-4f ? small : big;
  return v > 20.0f ? v : r;
}

struct ChunkArgs {
  int64_t chunk_len;  // time steps per chunk (a multiple of the tile length)
  int nchunks;
  float* st;          // [B, nchunks, Di, NS]: pass 1 end states, then (pass 2) incoming states
  float* sdt;         // [B, nchunks, Di]: sum of dt over each chunk
};

}  // namespace

// dt-input quantisation, once per token: int8 codes [M, 16 * RW] (zero past R) and the fp64
// dequantisation factor max(m, 1e-5) / 127 [M].  A group of G = 16, 32 or 64 lanes per token.
__global__ __launch_bounds__(256) void k_dt_codes(const void* __restrict__ dr, int bf16, int64_t M, int64_t ld,
                                                  int R, const float* __restrict__ g, float eps,
                                                  int8_t* __restrict__ codes, int cw, double* __restrict__ deq) {
  const int lane = threadIdx.x & 63;
  const int G = R <= 16 ? 16 : (R <= 32 ? 32 : 64);
  const int gl = lane & (G - 1);
  const int64_t tok = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / G) + lane / G;
  const bool ok = tok < M;
  const float gv = g ? g[gl < R ? gl : 0] : 1.0f;  // in flight with the row's load
  float v = 0.0f;
  if (ok && gl < R)
    v = bf16 ? bf16_to_f32(((const bf16_t*)dr)[tok * ld + gl]) : ((const float*)dr)[tok * ld + gl];
  float s = __builtin_fmaf(v, v, 0.0f);
  for (int dd = G / 2; dd >= 1; dd >>= 1) s = s + __shfl_xor(s, dd, 64);
  const float ms = __fdiv_rn(s, (float)R);
  const float r = __fdiv_rn(1.0f, sqrt_rn(ms + eps));
  float xh = v * r;
  if (g) xh = gl < R ? xh * gv : 0.0f;
  float m = fabsf(xh);
  for (int dd = G / 2; dd >= 1; dd >>= 1) m = fmaxf(m, __shfl_xor(m, dd, 64));
  const float sigma = __fdiv_rn(127.0f, fmaxf(m, 1e-5f));
  float q = rintf(xh * sigma);
  q = fminf(fmaxf(q, -128.0f), 127.0f);
  if (ok && gl < cw) codes[tok * cw + gl] = (int8_t)(int)q;
  if (ok && gl == 0) deq[tok] = (double)fmaxf(m, 1e-5f) / 127.0;
}

namespace {
struct DtCodes {
  const int8_t* codes;  // [M, 16 * RW]
  const double* deq;    // [M]
};
}  // namespace

// Lanes are 64 channels; the 4 waves of a block are 4 groups of NS / 4 states, so B and C of
// a step are the same for a whole wave and are read from LDS at wave-uniform addresses.  Each
// wave writes its readout partial per (step, channel) to LDS; the partials are added in wave
// order, plus D x, one tile later.
//
// One barrier per tile of TT = 16 steps, with double-buffered LDS: per tile i a thread
//   1. stages tile i: B, C into LDS, and for its (step, channel) items the step's dt (dot
//      product of the step's dt codes, held in registers since the previous tile, with the
//      channel's ternary row; fp64 dequantisation; bias; softplus) and dt x;
//   2. requests tile i + 1 (x, B, C, codes) into registers;
//   3. barrier;
//   4. adds the four waves' readout partials of tile i - 1, plus D x, and stores y;
//   5. runs the recurrence over tile i, writing its partials.
// A buffer of tile i is rewritten at tile i + 2, after the barrier of tile i + 1 that every
// wave reaches only once it has finished with tile i.
// MODE 1 (LOCAL): pass 1 (zero start, no readout; writes the chunk's end state and sum(dt)).
// MODE 2 (GATE): the readout is multiplied by SiLU of the gate input before it is stored.
template <int NS, typename T, int RW, int MODE>
__global__ __launch_bounds__(256, 2) void k_scan_m1(ScanArgs a, ChunkArgs ch, DtCodes dc) {
  constexpr bool LOCAL = MODE == 1;
  constexpr bool GATE = MODE == 2;
  constexpr bool FUSED = RW > 0;  // dt from the low-rank input: RW 16-byte code words per token
  constexpr int SPL = NS / 4;     // states per lane
  constexpr int CPB = 64;         // channels per block
  constexpr int TT = 16;          // time steps per tile
  constexpr int XPT = TT * CPB / 256;                    // (step, channel) items per thread
  constexpr int BPT = (TT * NS + 255) / 256;             // B (and C) elements per thread per tile
  constexpr int RWQ = FUSED ? RW : 1;
  __shared__ float2 s_dd[2][TT][CPB];  // (dt, dt * x)
  __shared__ __align__(16) float s_B[2][TT][NS];
  __shared__ __align__(16) float s_C[LOCAL ? 1 : 2][LOCAL ? 1 : TT][NS];
  __shared__ float s_yp[LOCAL ? 1 : 2][LOCAL ? 1 : 4][LOCAL ? 1 : TT][CPB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t Di = a.H, L = a.L;
  const int64_t b = blockIdx.x;   // sequence fastest: the channel tiles of a sequence share an XCD
  const int chunk = blockIdx.z;
  const int64_t tb = (int64_t)chunk * ch.chunk_len;
  const int64_t te = (tb + ch.chunk_len < L) ? tb + ch.chunk_len : L;
  const int64_t d0 = (int64_t)blockIdx.y * CPB;
  const int64_t d = d0 + lane;
  const bool dv = d < Di;
  // staging role: thread -> (channel lane, steps w, w + 4, ...).  Lanes past the last channel
  // take the per-channel parameters of the last channel (their results are never stored), so
  // the loads below have no lane-dependent branches and are all in flight together.
  const int64_t dcl = dv ? d : Di - 1;
  const float bias_s = a.delta_bias ? a.delta_bias[dcl] : 0.0f;
  const float D_s = a.D ? a.D[dcl] : 0.0f;
  constexpr int cw = 16 * RW;  // code bytes per token

  const T* X = (const T*)a.x;
  const T* DL = (const T*)a.delta;

  v4i wdt[4];
  double s_dt = 0.0;
  if (FUSED) {
    s_dt = (double)a.s_dt[0];
#pragma unroll
    for (int q = 0; q < 4; ++q) wdt[q] = unpack16_i8(q < RW ? a.w_dt[dcl * a.w_dt_row_words + q] : 0u);
  }

  // the initial state: h0 for the first chunk, the carry of the previous chunk otherwise
  const float* hsrc = nullptr;
  int64_t hoff = 0;
  if (!LOCAL) {
    if (chunk == 0) {
      hsrc = a.h0;
      hoff = (b * Di + dcl) * NS;
    } else {
      hsrc = ch.st;
      hoff = ((b * ch.nchunks + chunk - 1) * Di + dcl) * NS;
    }
  }
  float Al[SPL], h[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int n = w * SPL + i;
    Al[i] = a.A[dcl * NS + n] * LOG2E;
    h[i] = hsrc ? hsrc[hoff + n] : 0.0f;
  }
  float sum_dt = 0.0f;

  // prefetch registers for the next tile: x (and delta) of the thread's items, B, C, the
  // items' dt codes (a whole wave reads the same token row) and dequantisation factors
  // (raw activation elements: a conditional load that is converted at once makes the compiler
  // wait for it inside the condition, one round trip per load)
  T rx[XPT], rd[FUSED ? 1 : XPT], rb[BPT], rc[BPT], rz[GATE ? XPT : 1];
  v4i rq[FUSED ? XPT : 1][RWQ];
  double rf[FUSED ? XPT : 1];
  auto load_tile = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int t = w + 4 * i;
      const bool okt = t0 + t < te;
      const bool ok = okt && dv;
      const int64_t tok = b * L + t0 + t;
      rx[i] = ok ? X[tok * a.ld_x + d] : T(0);
      if (GATE) rz[GATE ? i : 0] = ok ? ((const T*)a.gate)[tok * a.ld_gate + d] : T(0);
      if (!FUSED) rd[FUSED ? 0 : i] = ok ? DL[tok * a.ld_delta + d] : T(0);
      if (FUSED) {
#pragma unroll
        for (int q = 0; q < RWQ; ++q)
          rq[FUSED ? i : 0][q] = okt ? ((const v4i*)(dc.codes + tok * cw))[q] : v4i{0, 0, 0, 0};
        rf[FUSED ? i : 0] = okt ? dc.deq[tok] : 0.0;
      }
    }
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int e = tid + 256 * i, t = e / NS, n = e % NS;
      const bool ok = (e < TT * NS) && (t0 + t < te);
      const int64_t tok = b * L + t0 + t;
      rb[i] = ok ? ((const T*)a.Bm)[tok * a.ld_B + n] : T(0);
      rc[i] = (ok && !LOCAL) ? ((const T*)a.Cm)[tok * a.ld_C + n] : T(0);
    }
  };

  float xprev[XPT];  // x of the previous tile's items, for D x
  float zprev[GATE ? XPT : 1];  // and their gate inputs
  int64_t tprev = -1;  // first step of the tile whose readout is pending
  auto store_y = [&](int buf, int64_t t0p) {
    T* Y = (T*)a.y;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int t = w + 4 * i;
      if ((t0p + t < te) && dv) {
        const float y = ((s_yp[LOCAL ? 0 : buf][0][t][lane] + s_yp[LOCAL ? 0 : buf][LOCAL ? 0 : 1][t][lane]) +
                         s_yp[LOCAL ? 0 : buf][LOCAL ? 0 : 2][t][lane]) + s_yp[LOCAL ? 0 : buf][LOCAL ? 0 : 3][t][lane];
        float yo = y + D_s * xprev[i];
        if (GATE) yo = yo * silu_gate(zprev[GATE ? i : 0]);
        st_act(Y + (b * L + t0p + t) * a.ld_y + d, yo);
      }
    }
  };

  load_tile(tb);
  int buf = 0;
  for (int64_t t0 = tb; t0 < te; t0 += TT, buf ^= 1) {
    // 1. stage this tile: B, C; per item dt, softplus, dt * x
    float xcur[XPT], zcur[GATE ? XPT : 1];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int t = w + 4 * i;
      const float xv = act_f32(rx[i]);
      xcur[i] = xv;
      if (GATE) zcur[GATE ? i : 0] = act_f32(rz[GATE ? i : 0]);
      float dtv;
      if (FUSED) {
        int acc = 0;
#pragma unroll
        for (int q = 0; q < RW; ++q)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_sdot4(rq[FUSED ? i : 0][q][j], wdt[q][j], acc, false);
        dtv = (float)((s_dt * (double)acc) * rf[FUSED ? i : 0]);
      } else {
        dtv = act_f32(rd[FUSED ? 0 : i]);
      }
      dtv += bias_s;
      if (a.softplus) dtv = softplus_f(dtv);
      s_dd[buf][t][lane] = make_float2(dtv, dtv * xv);
    }
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int e = tid + 256 * i;
      if (e < TT * NS) {
        s_B[buf][e / NS][e % NS] = act_f32(rb[i]);
        if (!LOCAL) s_C[LOCAL ? 0 : buf][LOCAL ? 0 : e / NS][e % NS] = act_f32(rc[i]);
      }
    }
    // 2. next tile in flight
    if (t0 + TT < te) load_tile(t0 + TT);
    // 3.
    __syncthreads();
    // 4. readout of the previous tile
    if (!LOCAL && tprev >= 0) store_y(buf ^ 1, tprev);
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      xprev[i] = xcur[i];
      if (GATE) zprev[GATE ? i : 0] = zcur[GATE ? i : 0];
    }
    tprev = t0;
    // 5. recurrence.  B and C of a step are the same for the whole wave (broadcast LDS reads);
    //    groups of GQ steps, software-pipelined: the LDS reads of group g + 1 are issued before
    //    the arithmetic of group g
    const int tmax = (int)((te - t0) < TT ? (te - t0) : TT);
    if (tmax == TT) {
      constexpr int GQ = 4, NG = TT / GQ;
      float bq[2][GQ][SPL], cq[2][GQ][SPL];
      float2 dd[2][GQ];
      auto ld = [&](int tt, int sl) {
#pragma unroll
        for (int u = 0; u < GQ; ++u) {
          const int t = tt + u;
#pragma unroll
          for (int i = 0; i < SPL; ++i) {
            bq[sl][u][i] = s_B[buf][t][w * SPL + i];
            if (!LOCAL) cq[sl][u][i] = s_C[LOCAL ? 0 : buf][LOCAL ? 0 : t][w * SPL + i];
          }
          dd[sl][u] = s_dd[buf][t][lane];
        }
      };
      ld(0, 0);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int sl = g & 1;
        if (g + 1 < NG) ld((g + 1) * GQ, sl ^ 1);
#pragma unroll
        for (int u = 0; u < GQ; ++u) {
          float yp = 0.0f;
#pragma unroll
          for (int i = 0; i < SPL; ++i) {
            const float ab = __builtin_amdgcn_exp2f(dd[sl][u].x * Al[i]);
            h[i] = __builtin_fmaf(ab, h[i], dd[sl][u].y * bq[sl][u][i]);
            if (!LOCAL) yp = i == 0 ? cq[sl][u][0] * h[0] : __builtin_fmaf(cq[sl][u][i], h[i], yp);
          }
          if (LOCAL) sum_dt += dd[sl][u].x;
          else s_yp[LOCAL ? 0 : buf][LOCAL ? 0 : w][LOCAL ? 0 : g * GQ + u][lane] = yp;
        }
      }
    } else {
      for (int t = 0; t < tmax; ++t) {
        const float2 ddt = s_dd[buf][t][lane];
        float yp = 0.0f;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
          const float ab = __builtin_amdgcn_exp2f(ddt.x * Al[i]);
          h[i] = __builtin_fmaf(ab, h[i], ddt.y * s_B[buf][t][w * SPL + i]);
          if (!LOCAL) yp = i == 0 ? s_C[LOCAL ? 0 : buf][LOCAL ? 0 : t][w * SPL] * h[0]
                                  : __builtin_fmaf(s_C[LOCAL ? 0 : buf][LOCAL ? 0 : t][w * SPL + i], h[i], yp);
        }
        if (LOCAL) sum_dt += ddt.x;
        else s_yp[LOCAL ? 0 : buf][LOCAL ? 0 : w][LOCAL ? 0 : t][lane] = yp;
      }
    }
  }
  if (!LOCAL && tprev >= 0) {
    __syncthreads();
    store_y(buf ^ 1, tprev);
  }
  if (LOCAL) {
    if (dv) {
#pragma unroll
      for (int i = 0; i < SPL; ++i) ch.st[((b * ch.nchunks + chunk) * Di + d) * NS + w * SPL + i] = h[i];
      if (w == 0) ch.sdt[(b * ch.nchunks + chunk) * Di + d] = sum_dt;
    }
  } else if (a.h_last && dv && chunk == ch.nchunks - 1) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) a.h_last[(b * Di + d) * NS + w * SPL + i] = h[i];
  }
}

// Pass 2: for every (sequence, channel, state), compose the chunks in order.  Afterwards
// st[b, c] holds the state entering chunk c + 1.
__global__ __launch_bounds__(256) void k_scan_m1_combine(const float* __restrict__ A, const float* __restrict__ h0,
                                                         float* __restrict__ st, const float* __restrict__ sdt,
                                                         int64_t B, int64_t Di, int NS, int T) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * Di * NS) return;
  const int64_t b = i / (Di * NS), dn = i % (Di * NS), d = dn / NS;
  float h = h0 ? h0[i] : 0.0f;
  const float a2 = A[dn] * LOG2E;
  for (int c = 0; c + 1 < T; ++c) {
    const int64_t si = ((b * T + c) * Di) * NS + dn;
    const float P = __builtin_amdgcn_exp2f(a2 * sdt[(b * T + c) * Di + d]);
    h = __builtin_fmaf(P, h, st[si]);
    st[si] = h;
  }
}

namespace {
constexpr int kCPB = 64;  // channels per block of k_scan_m1
constexpr int kTT = 16;   // time steps per tile of k_scan_m1

struct ScanPlan {
  int T = 1;
  int64_t chunk_len = 0;
  int cw = 0;             // dt code bytes per token (fused dt projection)
  size_t off_deq = 0, off_st = 0, ws = 0;
};

// Chunk count: a pure function of the shape (so results do not depend on the device).
// Blocks of batch x channel tiles below 512 (two per MI355X compute unit) are multiplied
// by time chunks of at least 128 steps.
ScanPlan plan_scan(const ScanArgs& a) {
  ScanPlan p;
  const int64_t blocks = cdiv(a.H, kCPB) * a.batch;
  int64_t T = 1;
  if (blocks < 512) {
    T = cdiv(512, blocks);
    const int64_t tmax = a.L / 128;
    if (T > tmax) T = tmax;
    if (T < 1) T = 1;
  }
  p.chunk_len = round_up(cdiv(a.L, T), kTT);
  p.T = (int)cdiv(a.L, p.chunk_len);
  const int64_t M = a.batch * a.L;
  size_t off = 0;
  if (a.R > 0) {  // the dt input's codes and dequantisation factors (dt_proj fused into the scan)
    p.cw = 16 * (int)cdiv(a.R, 16);
    off = round_up((int64_t)M * p.cw, 256);
    p.off_deq = off;
    off = round_up(off + (size_t)M * sizeof(double), 256);
  }
  p.off_st = off;
  if (p.T > 1) off += (size_t)a.batch * p.T * a.H * (a.N + 1) * sizeof(float);
  p.ws = off;
  return p;
}

template <int NS, typename T>
hipError_t launch_m1_t(const ScanArgs& a, void* ws, hipStream_t s) {
  const ScanPlan p = plan_scan(a);
  ChunkArgs ch{};
  ch.chunk_len = p.chunk_len;
  ch.nchunks = p.T;
  if (p.T > 1) {
    ch.st = (float*)((char*)ws + p.off_st);
    ch.sdt = ch.st + (size_t)a.batch * p.T * a.H * NS;
  }
  DtCodes dc{};
  const bool fused = a.dr != nullptr;
  if (fused) {
    const int64_t M = a.batch * a.L;
    int8_t* codes = (int8_t*)ws;
    double* deq = (double*)((char*)ws + p.off_deq);
    if (!a.dt_codes_ready) {
      const int G = a.R <= 16 ? 16 : (a.R <= 32 ? 32 : 64);
      const int64_t tok_per_block = 4 * (64 / G);
      hipLaunchKernelGGL(k_dt_codes, dim3((unsigned)cdiv(M, tok_per_block)), dim3(256), 0, s, a.dr, a.act_bf16, M,
                         a.ld_dr, a.R, a.g_dt, a.eps, codes, p.cw, deq);
    }
    dc.codes = codes;
    dc.deq = deq;
  }
  // grid (sequence, channel tile, chunk): blocks are dealt to the 8 XCDs round-robin by linear
  // index, so with the sequence fastest the channel tiles of sequence b all run on XCD b mod 8
  // and share its L2 for B, C and the dt codes
  const unsigned gx = (unsigned)a.batch, gy = (unsigned)cdiv(a.H, kCPB);
  const int rw = fused ? p.cw / 16 : 0;
  auto run = [&](auto rwc, bool local, unsigned gz) {
    constexpr int RWc = decltype(rwc)::value;
    if (local) hipLaunchKernelGGL((k_scan_m1<NS, T, RWc, 1>), dim3(gx, gy, gz), dim3(256), 0, s, a, ch, dc);
    else if (a.gate) hipLaunchKernelGGL((k_scan_m1<NS, T, RWc, 2>), dim3(gx, gy, gz), dim3(256), 0, s, a, ch, dc);
    else hipLaunchKernelGGL((k_scan_m1<NS, T, RWc, 0>), dim3(gx, gy, gz), dim3(256), 0, s, a, ch, dc);
  };
  auto run_rw = [&](bool local, unsigned gz) {
    switch (rw) {
      case 0: run(std::integral_constant<int, 0>{}, local, gz); break;
      case 1: run(std::integral_constant<int, 1>{}, local, gz); break;
      case 2: run(std::integral_constant<int, 2>{}, local, gz); break;
      case 3: run(std::integral_constant<int, 3>{}, local, gz); break;
      default: run(std::integral_constant<int, 4>{}, local, gz); break;
    }
  };
  if (p.T > 1) {
    run_rw(true, (unsigned)(p.T - 1));
    const int64_t n = a.batch * a.H * NS;
    hipLaunchKernelGGL(k_scan_m1_combine, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, a.A, a.h0, ch.st, ch.sdt,
                       a.batch, a.H, NS, p.T);
  }
  run_rw(false, (unsigned)p.T);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_m1_n(const ScanArgs& a, void* ws, hipStream_t s) {
  switch (a.N) {
    case 4: return launch_m1_t<4, T>(a, ws, s);
    case 8: return launch_m1_t<8, T>(a, ws, s);
    case 16: return launch_m1_t<16, T>(a, ws, s);
    case 32: return launch_m1_t<32, T>(a, ws, s);
    case 64: return launch_m1_t<64, T>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

void scan_m1_code_layout(const ScanArgs& a, int* cw, size_t* off_deq) {
  const ScanPlan p = plan_scan(a);
  *cw = p.cw;
  *off_deq = p.off_deq;
}

size_t scan_m1_workspace(const ScanArgs& a) {
  if (a.batch == 0 || a.L == 0) return 0;
  return plan_scan(a).ws;
}

hipError_t launch_scan_m1(const ScanArgs& a, void* ws, hipStream_t s) {
  if (a.batch == 0 || a.L == 0) return hipSuccess;
  return a.act_bf16 ? launch_m1_n<bf16_t>(a, ws, s) : launch_m1_n<float>(a, ws, s);
}

}  // namespace ssm
