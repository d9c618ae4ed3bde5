// Selective scan, Mamba-1 kind (Mamba, cited by title in "Baseline Shape Decides the
// Verdict ...", Builds on; TriSSM README: input-dependent Delta, B, C, and the recurrence
// evaluated with a parallel associative scan).  A is per (channel, state); one channel per
// head.
//
// Two kernels.  d_state 16 (k_scan_m1_g8): a channel's states are split over lanes, 8
// channels x 8 state pairs per wave, independent waves; the readout sum over the pairs is
// reduced inside the wave (kernel comment below).  Other d_state (k_scan_m1): a block owns 64
// channels (the lanes) of one sequence and one time chunk; its 4 waves split the NS states
// into 4 groups, so that B and C of a step are the same for a whole wave: they are read from
// LDS at wave-uniform addresses (a broadcast); the waves' readout partials meet in LDS and are
// added in wave order.  In both, each lane runs the recurrence of its states over time in
// registers: per state and step one exp2 (A is pre-scaled by log2 e), two multiplies and two
// fused multiply-adds.  Time is staged through LDS in tiles (16 and 8 steps): the next tiles'
// x, B, C (and dt input codes) are loaded into registers through buffer resources over the
// block's sequence while the current tile runs.
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
// row is v_dot4 instructions, and the dequantisation s_dt acc max(m, 1e-5) / 127 is fp32
// (the value never reaches memory: two roundings where a stored BitLinear output has one).
#include <mutex>
#include <type_traits>

#include "launch.hpp"

namespace ssm {

namespace {
constexpr int RMAX = 64;

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
  int32_t* dbg_acc;     // nullable [M, Di]: the int32 sums, stored for stage-wise checks
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
//      channel's ternary row; fp32 dequantisation; bias; softplus) and dt x;
//   2. requests tile i + 1 (x, B, C, codes) into registers;
//   3. barrier;
//   4. adds the four waves' readout partials of tile i - 1, plus D x, and stores y;
//   5. runs the recurrence over tile i, writing its partials.
// A buffer of tile i is rewritten at tile i + 2, after the barrier of tile i + 1 that every
// wave reaches only once it has finished with tile i.
// Memory is reached through buffer resources over the block's sequence: a wave-uniform row
// offset plus a per-lane column offset, no per-item address arithmetic or branches; rows past
// the sequence end read zeros and their stores are dropped.  A tile that ends past the
// sequence runs its missing steps with dt = 0 (the state is left unchanged).  Lanes past the
// last channel take the last channel's parameters and store nothing.
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
  constexpr uint32_t S = sizeof(T);
  __shared__ float2 s_dd[2][TT][CPB];  // (dt, dt * x)
  __shared__ __align__(16) float s_B[2][TT][NS];
  __shared__ __align__(16) float s_C[LOCAL ? 1 : 2][LOCAL ? 1 : TT][NS];
  __shared__ float s_yp[LOCAL ? 1 : 2][LOCAL ? 1 : 4][LOCAL ? 1 : TT][CPB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t Di = a.H, L = a.L;
  const int64_t b = blockIdx.x;   // sequence fastest: the channel tiles of a sequence share an XCD
  const int chunk = blockIdx.z;
  // step indices within the sequence are 32-bit (a sequence spans less than 2^31 bytes)
  const int tb = __builtin_amdgcn_readfirstlane((int)(chunk * ch.chunk_len));
  const int te = __builtin_amdgcn_readfirstlane((int)((chunk * ch.chunk_len + ch.chunk_len < L) ? chunk * ch.chunk_len + ch.chunk_len : L));
  const int64_t d0 = (int64_t)blockIdx.y * CPB;
  const int64_t d = d0 + lane;
  const bool dv = d < Di;
  // per-channel parameters: lanes past the last channel take the last channel's (their results
  // are never stored), so these loads have no lane-dependent branches
  const int64_t dcl = dv ? d : Di - 1;
  const float bias_s = a.delta_bias ? a.delta_bias[dcl] : 0.0f;
  const float D_s = a.D ? a.D[dcl] : 0.0f;
  constexpr int cw = 16 * RW;  // code bytes per token

  // buffer resources over sequence b (rows 0 .. L - 1; activation tensors from channel d0)
  const int64_t row0 = b * L;
  const int64_t nch = Di - d0;
  auto act_rsrc = [&](const void* p, int64_t ld) {
    return buf_rsrc((const T*)p + row0 * ld + d0, (uint32_t)(((L - 1) * ld + nch) * S));
  };
  const auto rX = act_rsrc(a.x, a.ld_x);
  const auto rDL = act_rsrc(FUSED ? a.x : a.delta, FUSED ? a.ld_x : a.ld_delta);
  const auto rZ = act_rsrc(GATE ? a.gate : a.x, GATE ? a.ld_gate : a.ld_x);
  const auto rY = act_rsrc(a.y, a.ld_y);
  const auto rB = buf_rsrc((const T*)a.Bm + row0 * a.ld_B, (uint32_t)(((L - 1) * a.ld_B + NS) * S));
  const auto rC = buf_rsrc((const T*)a.Cm + row0 * a.ld_C, (uint32_t)(((L - 1) * a.ld_C + NS) * S));
  const auto rQ = buf_rsrc(FUSED ? dc.codes + row0 * cw : nullptr, FUSED ? (uint32_t)(L * cw) : 0u);
  const auto rF = buf_rsrc(FUSED ? dc.deq + row0 : nullptr, FUSED ? (uint32_t)(L * 8) : 0u);
  const auto rG = buf_rsrc(dc.dbg_acc ? dc.dbg_acc + row0 * Di + d0 : nullptr,
                           dc.dbg_acc ? (uint32_t)(((L - 1) * Di + nch) * 4) : 0u);
  const uint32_t vlane = (uint32_t)lane * S;
  // row strides in bytes (wave-uniform)
  const uint32_t sx = (uint32_t)a.ld_x * S, sdl = (uint32_t)(FUSED ? a.ld_x : a.ld_delta) * S;
  const uint32_t sz = (uint32_t)(GATE ? a.ld_gate : a.ld_x) * S, sy = (uint32_t)a.ld_y * S;
  const uint32_t sb = (uint32_t)a.ld_B * S, sc = (uint32_t)a.ld_C * S;
  // B and C: thread -> elements (t, n) = divmod(tid + 256 i, NS) of a tile
  uint32_t vb[BPT], vc[BPT];
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int e = tid + 256 * i, t = e / NS, n = e % NS;
    vb[i] = e < TT * NS ? (uint32_t)t * sb + (uint32_t)n * S : kOutside;
    vc[i] = e < TT * NS ? (uint32_t)t * sc + (uint32_t)n * S : kOutside;
  }

  v4i wdt[4];
  float s_dt = 0.0f;
  if (FUSED) {
    s_dt = a.s_dt[0];
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
  T rx[XPT], rd[FUSED ? 1 : XPT], rb[BPT], rc[BPT], rz[GATE ? XPT : 1];
  v4i rq[FUSED ? XPT : 1][RWQ];
  double rf[FUSED ? XPT : 1];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const uint32_t row = (uint32_t)(t0 + w + 4 * i);
      rx[i] = buf_ld_act<T>(rX, vlane, row * sx);
      if (GATE) rz[GATE ? i : 0] = buf_ld_act<T>(rZ, vlane, row * sz);
      if (!FUSED) rd[FUSED ? 0 : i] = buf_ld_act<T>(rDL, vlane, row * sdl);
      if (FUSED) {
#pragma unroll
        for (int q = 0; q < RWQ; ++q)
          rq[FUSED ? i : 0][q] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rQ, 16u * q, row * cw, 0));
        rf[FUSED ? i : 0] = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(rF, 0u, row * 8u, 0));
      }
    }
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      rb[i] = buf_ld_act<T>(rB, vb[i], (uint32_t)t0 * sb);
      if (!LOCAL) rc[i] = buf_ld_act<T>(rC, vc[i], (uint32_t)t0 * sc);
    }
  };

  float xprev[XPT];  // x of the previous tile's items, for D x
  float zprev[GATE ? XPT : 1];  // and their gate inputs
  int tprev = -1;  // first step of the tile whose readout is pending
  auto store_y = [&](int buf, int t0p) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int t = w + 4 * i;
      const float y = ((s_yp[LOCAL ? 0 : buf][0][t][lane] + s_yp[LOCAL ? 0 : buf][LOCAL ? 0 : 1][t][lane]) +
                       s_yp[LOCAL ? 0 : buf][LOCAL ? 0 : 2][t][lane]) + s_yp[LOCAL ? 0 : buf][LOCAL ? 0 : 3][t][lane];
      float yo = y + D_s * xprev[i];
      if (GATE) yo = yo * silu_gate(zprev[GATE ? i : 0]);
      if (dv) buf_st_act<T>(yo, rY, vlane, (uint32_t)(t0p + t) * sy);
    }
  };

  load_tile(tb);
  int buf = 0;
  for (int t0 = tb; t0 < te; t0 += TT, buf ^= 1) {
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
        if (!LOCAL && dc.dbg_acc && dv)
          __builtin_amdgcn_raw_buffer_store_b32((uint32_t)acc, rG, (uint32_t)lane * 4u, (uint32_t)(t0 + t) * (uint32_t)Di * 4u, 0);
        dtv = (s_dt * (float)acc) * (float)rf[FUSED ? i : 0];
      } else {
        dtv = act_f32(rd[FUSED ? 0 : i]);
      }
      dtv += bias_s;
      if (a.softplus) dtv = softplus_f(dtv);
      if (t0 + t >= te) dtv = 0.0f;  // past the sequence end: the state stays as it is
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

// d_state 16: the states of a channel are split over lanes instead of waves.  Lane l of a wave
// holds channel c = l mod 8 of the wave's 8 channels and the state pair (2g, 2g + 1), g = l / 8;
// a block is 4 waves (32 channels).  A layer at the TriSSM shape is then 4096 waves, four per
// SIMD (measured: the VALU issues the recurrence ~1.25x faster than with two), and the readout
// sum over the 8 pairs stays inside the wave: the 8 steps of a tile are reduced and scattered
// at once (lanes 32 apart, then 16 with the permlane swaps, then 8 with a row rotation), after
// which lane (g, c) holds the whole readout of step bitrev3(g) of channel c.  Each pairwise sum
// adds the same two operands on both lanes, so y = ((p0 + p4) + (p2 + p6)) + ((p1 + p5) +
// (p3 + p7)) for the pair partials p (each an fma chain over its two states), then + D x.
// The same lane stages that (step, channel) item: its dt (dot product of the step's dt codes
// with the channel's ternary row, fp32 dequantisation, bias, softplus) and dt x into a
// per-wave LDS area, and keeps x for D x; each wave stages the tile's B and C for itself, so
// the waves never wait for one another (no block barrier).  Tiles of TT = 8 steps,
// double-buffered LDS: per tile stage, request the tile after next into registers,
// recurrence, readout.
// MODE 1 (LOCAL): pass 1 of the chunked scan; MODE 2 (GATE): readout times SiLU(gate).
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// value of lane l ^ 8 (rotation of each 16-lane row by 8)
__device__ __forceinline__ float xor8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

template <typename T, int RW, int MODE>
__global__ __launch_bounds__(256, RW >= 3 ? 2 : 4) void k_scan_m1_g8(ScanArgs a, ChunkArgs ch, DtCodes dc) {
  constexpr bool LOCAL = MODE == 1;
  constexpr bool GATE = MODE == 2;
  constexpr bool FUSED = RW > 0;
  constexpr int NS = 16, SPL = 2, CPW = 8, NW = 4, CPB = CPW * NW, TT = 8;
  constexpr int RWQ = FUSED ? RW : 1;
  constexpr uint32_t S = sizeof(T);
  constexpr int cw = 16 * RW;
  // rows padded to TT + 2 steps: the 8 distinct 16-byte reads of a wave fall in distinct banks
  __shared__ __align__(16) float s_B[2][NW][NS / SPL][TT + 2][SPL];  // [buf][wave][pair][step][state of the pair]
  __shared__ __align__(16) float s_C[LOCAL ? 1 : 2][NW][NS / SPL][TT + 2][SPL];
  __shared__ __align__(16) float2 s_dd[2][NW][CPW][TT + 2];      // [buf][wave][channel][step]: (dt, dt x)

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 3, c = lane & 7;
  const int si = ((g & 1) << 2) | (g & 2) | (g >> 2);  // the step this lane stages and reads out
  const int64_t Di = a.H, L = a.L;
  const int64_t b = blockIdx.x;
  const int chunk = blockIdx.z;
  const int tb = __builtin_amdgcn_readfirstlane((int)(chunk * ch.chunk_len));
  const int te = __builtin_amdgcn_readfirstlane((int)((chunk * ch.chunk_len + ch.chunk_len < L) ? chunk * ch.chunk_len + ch.chunk_len : L));
  const int64_t d0 = (int64_t)blockIdx.y * CPB + w * CPW;  // the wave's first channel
  const int64_t d = d0 + c;
  const bool dv = d < Di;
  const int64_t dcl = dv ? d : Di - 1;
  const float bias_s = a.delta_bias ? a.delta_bias[dcl] : 0.0f;
  const float D_s = a.D ? a.D[dcl] : 0.0f;

  // buffer resources over sequence b (activation tensors from channel d0)
  const int64_t row0 = b * L;
  const int64_t nch = Di - d0;
  auto act_rsrc = [&](const void* p, int64_t ld) {
    const int64_t n = (L - 1) * ld + nch;
    return buf_rsrc((const T*)p + row0 * ld + d0, n > 0 ? (uint32_t)(n * S) : 0u);
  };
  const auto rX = act_rsrc(a.x, a.ld_x);
  const auto rDL = act_rsrc(FUSED ? a.x : a.delta, FUSED ? a.ld_x : a.ld_delta);
  const auto rZ = act_rsrc(GATE ? a.gate : a.x, GATE ? a.ld_gate : a.ld_x);
  const auto rY = act_rsrc(a.y, a.ld_y);
  // B and C of a tile, staged by each wave for itself (no barrier between waves): lane ->
  // step bt = l / 8, state pair bp = l mod 8, elements (bt, 2 bp) and (bt, 2 bp + 1)
  const int bt = lane >> 3, bp = lane & 7;
  const auto rB = buf_rsrc((const T*)a.Bm + row0 * a.ld_B, (uint32_t)(((L - 1) * a.ld_B + NS) * S));
  const auto rC = buf_rsrc((const T*)a.Cm + row0 * a.ld_C, (uint32_t)(((L - 1) * a.ld_C + NS) * S));
  const uint32_t vb = ((uint32_t)bt * (uint32_t)a.ld_B + 2u * bp) * S, sb = (uint32_t)a.ld_B * S;
  const uint32_t vc = ((uint32_t)bt * (uint32_t)a.ld_C + 2u * bp) * S, sc = (uint32_t)a.ld_C * S;
  const auto rQ = buf_rsrc(FUSED ? dc.codes + row0 * cw : nullptr, FUSED ? (uint32_t)(L * cw) : 0u);
  const auto rF = buf_rsrc(FUSED ? dc.deq + row0 : nullptr, FUSED ? (uint32_t)(L * 8) : 0u);
  const auto rG = buf_rsrc(dc.dbg_acc ? dc.dbg_acc + row0 * Di + d0 : nullptr,
                           (dc.dbg_acc && nch > 0) ? (uint32_t)(((L - 1) * Di + nch) * 4) : 0u);
  const uint32_t sx = (uint32_t)a.ld_x * S, sdl = (uint32_t)(FUSED ? a.ld_x : a.ld_delta) * S;
  const uint32_t sz = (uint32_t)(GATE ? a.ld_gate : a.ld_x) * S, sy = (uint32_t)a.ld_y * S;
  // per-lane offsets of the lane's item (step si, channel c)
  const uint32_t vx = (uint32_t)si * sx + (uint32_t)c * S, vdl = (uint32_t)si * sdl + (uint32_t)c * S;
  const uint32_t vz = (uint32_t)si * sz + (uint32_t)c * S;
  // stores: lanes past the last channel write outside their resource (dropped), so every store
  // is issued unconditionally and the waits for loads stay exact counts
  const uint32_t vy = dv ? (uint32_t)si * sy + (uint32_t)c * S : kOutside;
  const uint32_t vg = dv ? ((uint32_t)si * (uint32_t)Di + (uint32_t)c) * 4u : kOutside;

  v4i wdt[4];
  float s_dt = 0.0f;
  if (FUSED) {
    s_dt = a.s_dt[0];
#pragma unroll
    for (int q = 0; q < 4; ++q) wdt[q] = unpack16_i8(q < RW ? a.w_dt[dcl * a.w_dt_row_words + q] : 0u);
  }
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
    Al[i] = a.A[dcl * NS + SPL * g + i] * LOG2E;
    h[i] = hsrc ? hsrc[hoff + SPL * g + i] : 0.0f;
  }
  float sum_dt = 0.0f;

  // Register sets for two tiles: the loads of tile i + 2 are issued as tile i is staged, so a
  // tile's data has two tiles of work to arrive.  Every load is unconditional (rows past the
  // sequence read zeros), so the waits are exact counts, and tiles run in pairs: a tile wholly
  // past the sequence end (odd tile count) runs with dt = 0 and stores nothing.
  struct Regs {
    T rx, rd, rz, rb0, rb1, rc0, rc1;
    v4i rq[RWQ];
    double rf;
  };
  Regs R0, R1;
  auto load_tile = [&](Regs& r, int t0) {
    const uint32_t tr = (uint32_t)t0;
    r.rx = buf_ld_act<T>(rX, vx, tr * sx);
    if (GATE) r.rz = buf_ld_act<T>(rZ, vz, tr * sz);
    if (!FUSED) r.rd = buf_ld_act<T>(rDL, vdl, tr * sdl);
    if (FUSED) {
#pragma unroll
      for (int q = 0; q < RWQ; ++q)
        r.rq[q] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rQ, (uint32_t)si * cw + 16u * q, tr * cw, 0));
      r.rf = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(rF, (uint32_t)si * 8u, tr * 8u, 0));
    }
    r.rb0 = buf_ld_act<T>(rB, vb, tr * sb);
    r.rb1 = buf_ld_act<T>(rB, vb + S, tr * sb);
    if (!LOCAL) {
      r.rc0 = buf_ld_act<T>(rC, vc, tr * sc);
      r.rc1 = buf_ld_act<T>(rC, vc + S, tr * sc);
    }
  };

  auto run_tile = [&](Regs& r, int t0, int buf) {
    // 1. stage: this lane's item, and the block's B and C.  x and the gate input are kept for
    //    the readout in registers of their own (a copy), so that the loads of the tile after
    //    next can refill r in place (otherwise the compiler rotates the register sets across
    //    iterations and waits for those loads at the end of each pair)
    float xv, zv = 0.0f;
    asm("v_mov_b32 %0, %1" : "=v"(xv) : "v"(act_f32(r.rx)));
    if (GATE) asm("v_mov_b32 %0, %1" : "=v"(zv) : "v"(act_f32(r.rz)));
    float dtv;
    if (FUSED) {
      int acc = 0;
#pragma unroll
      for (int q = 0; q < RW; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_sdot4(r.rq[q][j], wdt[q][j], acc, false);
      if (!LOCAL)  // dropped unless the sums are asked for (rG is then empty) and the lane holds a channel
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)acc, rG, vg, (uint32_t)t0 * (uint32_t)Di * 4u, 0);
      dtv = (s_dt * (float)acc) * (float)r.rf;
    } else {
      dtv = act_f32(r.rd);
    }
    dtv += bias_s;
    if (a.softplus) dtv = softplus_f(dtv);
    if (t0 + si >= te) dtv = 0.0f;  // past the sequence end: the state stays as it is
    s_dd[buf][w][c][si] = make_float2(dtv, dtv * xv);
    *(float2*)&s_B[buf][w][bp][bt][0] = make_float2(act_f32(r.rb0), act_f32(r.rb1));
    if (!LOCAL) *(float2*)&s_C[LOCAL ? 0 : buf][w][bp][bt][0] = make_float2(act_f32(r.rc0), act_f32(r.rc1));
    // 2. the tile after next in flight
    load_tile(r, t0 + 2 * TT);
    // 3. this wave's LDS writes before its reads (LDS executes a wave's operations in order;
    //    the fences keep the compiler from reordering them)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 4. recurrence over the tile, two steps per LDS read; the reads of the next two steps are
    //    issued before the arithmetic of the current two (kept in place by scheduling fences),
    //    so a wave's LDS traffic is spread over its recurrence
    float yp[TT];
    float4 dd = *(const float4*)&s_dd[buf][w][c][0];
    float4 bb = *(const float4*)&s_B[buf][w][g][0][0];
    float4 cc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (!LOCAL) cc = *(const float4*)&s_C[LOCAL ? 0 : buf][w][LOCAL ? 0 : g][0][0];
#pragma unroll
    for (int t = 0; t < TT; t += 2) {
      float4 ddn = dd, bbn = bb, ccn = cc;
      if (t + 2 < TT) {
        ddn = *(const float4*)&s_dd[buf][w][c][t + 2];
        bbn = *(const float4*)&s_B[buf][w][g][t + 2][0];
        if (!LOCAL) ccn = *(const float4*)&s_C[LOCAL ? 0 : buf][w][LOCAL ? 0 : g][t + 2][0];
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        const float ab0 = __builtin_amdgcn_exp2f(dd.x * Al[0]);
        const float ab1 = __builtin_amdgcn_exp2f(dd.x * Al[1]);
        h[0] = __builtin_fmaf(ab0, h[0], dd.y * bb.x);
        h[1] = __builtin_fmaf(ab1, h[1], dd.y * bb.y);
        yp[t] = __builtin_fmaf(cc.y, h[1], cc.x * h[0]);
      }
      {
        const float ab0 = __builtin_amdgcn_exp2f(dd.z * Al[0]);
        const float ab1 = __builtin_amdgcn_exp2f(dd.z * Al[1]);
        h[0] = __builtin_fmaf(ab0, h[0], dd.w * bb.z);
        h[1] = __builtin_fmaf(ab1, h[1], dd.w * bb.w);
        yp[t + 1] = __builtin_fmaf(cc.w, h[1], cc.z * h[0]);
      }
      if (LOCAL) sum_dt += dd.x + dd.z;
      __builtin_amdgcn_sched_barrier(0);
      dd = ddn;
      bb = bbn;
      cc = ccn;
    }
    if (!LOCAL) {
      // 5. readout: reduce the 8 pair partials of each step and scatter the steps over the lanes
#pragma unroll
      for (int j = 0; j < 4; ++j) swap32(yp[2 * j], yp[2 * j + 1]);
      float r1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) r1[j] = yp[2 * j] + yp[2 * j + 1];
      swap16(r1[0], r1[1]);
      swap16(r1[2], r1[3]);
      const float r20 = r1[0] + r1[1], r21 = r1[2] + r1[3];
      const bool hi8 = (lane & 8) != 0;
      const float keep = hi8 ? r21 : r20, give = hi8 ? r20 : r21;
      const float y = keep + xor8(give);
      float yo = y + D_s * xv;
      if (GATE) yo = yo * silu_gate(zv);
      buf_st_act<T>(yo, rY, vy, (uint32_t)t0 * sy);  // lanes past the last channel: outside rY
    }
  };

  load_tile(R0, tb);
  __builtin_amdgcn_sched_barrier(0);  // tile 0's loads stay ahead of tile 1's (exact wait counts)
  load_tile(R1, tb + TT);
  // Wave priority by progress: the arbiter favours the oldest wave, so the four waves of a SIMD
  // would otherwise finish one after another, the last ones alone on the SIMD; a wave drops its
  // priority a step per quarter of its tiles done, so the waves advance together (measured: the
  // layer's span 46 -> 43 us at the TriSSM shape).
  const int npairs = (te - tb + 2 * TT - 1) / (2 * TT);
  for (int t0 = tb; t0 < te; t0 += 2 * TT) {
    const int q = (4 * ((t0 - tb) / (2 * TT))) / npairs;  // quarters done (uniform)
    if (q == 0) __builtin_amdgcn_s_setprio(3);
    else if (q == 1) __builtin_amdgcn_s_setprio(2);
    else if (q == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    run_tile(R0, t0, 0);
    run_tile(R1, t0 + TT, 1);
  }
  if (LOCAL) {
    if (dv) {
#pragma unroll
      for (int i = 0; i < SPL; ++i) ch.st[((b * ch.nchunks + chunk) * Di + d) * NS + SPL * g + i] = h[i];
      if (g == 0) ch.sdt[(b * ch.nchunks + chunk) * Di + d] = sum_dt;
    }
  } else if (a.h_last && dv && chunk == ch.nchunks - 1) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) a.h_last[(b * Di + d) * NS + SPL * g + i] = h[i];
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

// d_state 16 runs k_scan_m1_g8: 32 channels and pairs of 8-step tiles per block, four blocks
// per compute unit.
constexpr int kCPB16 = 32, kTT16 = 16;  // chunks hold whole pairs of 8-step tiles

// Chunk count: a pure function of the shape (so results do not depend on the device).
// Fewer than 512 blocks of batch x channel tiles (two waves per SIMD) are multiplied by time
// chunks of at least 128 steps, up to a full chip: 512 blocks of k_scan_m1 (two per MI355X
// compute unit), 1024 of k_scan_m1_g8 (four).  From 512 blocks on k_scan_m1_g8 runs unchunked:
// going from two to four waves per SIMD does not pay for pass 1 (measured at the TernarySSM
// shape, 16 x 1024 tokens x 1024 channels: 149 us chunked in two, 107 us unchunked; the
// long-sequence shape, 8 x 8192 x 512, takes 273 us in 8 chunks, 330 us in 4).
ScanPlan plan_scan(const ScanArgs& a) {
  ScanPlan p;
  const bool g8 = a.N == 16;
  const int64_t full = g8 ? 1024 : 512;
  const int64_t blocks = cdiv(a.H, g8 ? kCPB16 : kCPB) * a.batch;
  int64_t T = 1;
  if (blocks < 512) {
    T = cdiv(full, blocks);
    const int64_t tmax = a.L / 128;
    if (T > tmax) T = tmax;
    if (T < 1) T = 1;
  }
  p.chunk_len = round_up(cdiv(a.L, T), g8 ? kTT16 : kTT);
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
    if (a.ext_codes) {
      codes = (int8_t*)a.ext_codes;
      deq = (double*)a.ext_deq;
    } else if (!a.dt_codes_ready) {
      launch_dt_codes(a.dr, a.act_bf16, M, a.ld_dr, a.R, a.g_dt, a.eps, codes, deq, s);
    }
    dc.codes = codes;
    dc.deq = deq;
    dc.dbg_acc = a.dbg_dt_acc;
  }
  // grid (sequence, channel tile, chunk): blocks are dealt to the 8 XCDs round-robin by linear
  // index, so with the sequence fastest the channel tiles of sequence b all run on XCD b mod 8
  // and share its L2 for B, C and the dt codes
  const unsigned gx = (unsigned)a.batch, gy = (unsigned)cdiv(a.H, NS == 16 ? kCPB16 : kCPB);
  const int rw = fused ? p.cw / 16 : 0;
  auto run = [&](auto rwc, bool local, unsigned gz) {
    constexpr int RWc = decltype(rwc)::value;
    if (NS == 16) {
      if (local) hipLaunchKernelGGL((k_scan_m1_g8<T, RWc, 1>), dim3(gx, gy, gz), dim3(256), 0, s, a, ch, dc);
      else if (a.gate) hipLaunchKernelGGL((k_scan_m1_g8<T, RWc, 2>), dim3(gx, gy, gz), dim3(256), 0, s, a, ch, dc);
      else hipLaunchKernelGGL((k_scan_m1_g8<T, RWc, 0>), dim3(gx, gy, gz), dim3(256), 0, s, a, ch, dc);
    } else if (local) hipLaunchKernelGGL((k_scan_m1<NS, T, RWc, 1>), dim3(gx, gy, gz), dim3(256), 0, s, a, ch, dc);
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

hipError_t launch_dt_codes(const void* dr, int bf16, int64_t M, int64_t ld, int R, const float* g, float eps,
                           int8_t* codes, double* deq, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int G = R <= 16 ? 16 : (R <= 32 ? 32 : 64);
  const int64_t tok_per_block = 4 * (64 / G);
  hipLaunchKernelGGL(k_dt_codes, dim3((unsigned)cdiv(M, tok_per_block)), dim3(256), 0, s, dr, bf16, M, ld, R, g, eps,
                     codes, 16 * (int)cdiv(R, 16), deq);
  return hipGetLastError();
}

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

// ---- the library's own scratch memory, for callers that cannot allocate (static_scratch)
// One array per GPU, held until the process ends.  Its name is a host-side stand-in in host
// code: the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int d = 0;
  hipError_t e = hipGetDevice(&d);
  if (e != hipSuccess) return e;
  if (d < 0 || d >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[d]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[d] = p;
  }
  *ptr = g_scratch_ptr[d];
  return hipSuccess;
}

}  // namespace ssm
