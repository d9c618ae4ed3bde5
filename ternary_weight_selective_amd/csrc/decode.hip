// One decoding step of the Mamba-1 kind mixer (one token per sequence, the recurrent state
// carried between calls; Mamba, cited by title in "Baseline Shape Decides the Verdict ...",
// Builds on: the recurrence evaluated step by step at inference; TriSSM README: ternary
// BitLinear projections with int8 activations for Delta, B, C).  At one token per sequence
// the whole-sequence kernels run on a handful of compute units (one row block), so the step
// has a kernel of its own: one block per sequence runs the whole layer for its token
// (sequences are independent while decoding), in phases separated by block barriers:
//   in_proj (each wave a quarter-share of the 16-wide output tiles, int8 MFMA with the one
//   token as the B operand), x's norm and codes, x_proj, the dt input's codes, every
//   channel's dt and its NS states advanced one step (a thread per channel), y's norm and
//   codes, out_proj with the residual.  Every global load (weights, state, A, the residual) is
//   issued at the start, so the block waits for memory once.
// Every value is computed as the whole-sequence path computes it: the same fixed-order norms
// and absmax quantisation, the same int32 sums, the same fp64 epilogues rounded once to the
// activation type, the same in-scan dt dequantisation in fp32, softplus, exp2 recurrence and
// readout order (d_state 16: eight state pairs, each an fma chain, summed in the scan's
// in-wave tree; otherwise four groups of NS / 4 states, each accumulated by fused
// multiply-adds, the groups added in order; then D x).
#include "launch.hpp"

namespace ssm {

namespace {

// One 64-lane wave: RMSNorm + absmax codes of the single row held in LDS (K = 64 KPL
// values), the canonical lane layout, codes into sq and the factor into *sdeq.
template <int KPL>
__device__ __forceinline__ void norm_quant_one(const float* src, const float (&gn)[KPL], int K, float eps, int8_t* sq,
                                               double* sdeq, int lane) {
  float v[1][KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) v[0][i] = src[lane + 64 * i];
  norm_quant_rows<1, KPL>(v, gn, K, eps, sq, 0, sdeq, lane);
}

// The block's one token as the B operand of a contraction over K = 64 KPL: lane group 0
// (lanes with lm == 0) holds the codes of k step ks, the other lanes zeros.  Read once per
// phase and shared by the phase's tiles.
template <int KPL>
__device__ __forceinline__ void dec_codes(v4i (&bq)[KPL], const int8_t* sq, int lane) {
  const int kq = lane >> 4, lm = lane & 15;
#pragma unroll
  for (int ks = 0; ks < KPL; ++ks)
    bq[ks] = lm == 0 ? *(const v4i*)(sq + (kq * KPL + ks) * 16) : v4i{0, 0, 0, 0};
}

// in_proj / x_proj / out_proj of the block's one token: 16-wide output tiles t of W [n_out,
// 64 KPL] (packed) against the token's codes.  Returns the int32 sums of outputs 16 t + 4 kq
// .. + 3 in lanes with lm == 0.
template <int KPL>
__device__ __forceinline__ v4i dec_tile(const uint32_t (&w)[KPL], const v4i (&bq)[KPL]) {
  v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < KPL; ++ks) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16_i8(w[ks]), bq[ks], acc, 0, 0, 0);
  return acc;
}

// Lane (n, kq) of tile t: packed words kq KPL .. kq KPL + KPL - 1 of row 16 t + n (rows of
// 4 KPL words; 16-byte loads when KPL is a multiple of 4, the rows then being 16-byte aligned
// whenever W is).  Rows past n_out read row n_out - 1: their sums are never stored (and the
// loaded words are used as they are, so that no wait for them comes before their use).
template <int KPL>
__device__ __forceinline__ void dec_load_w(uint32_t (&w)[KPL], const uint32_t* W, int n_out, int t, int lane) {
  const int kq = lane >> 4, lm = lane & 15;
  const int n = t * 16 + lm;
  const uint32_t* wr = W + (int64_t)(n < n_out ? n : n_out - 1) * (4 * KPL) + kq * KPL;
  if constexpr (KPL % 4 == 0) {
#pragma unroll
    for (int v = 0; v < KPL / 4; ++v) {
      const uint4 u4 = ((const uint4*)wr)[v];
      w[4 * v] = u4.x; w[4 * v + 1] = u4.y; w[4 * v + 2] = u4.z; w[4 * v + 3] = u4.w;
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KPL; ++ks) w[ks] = wr[ks];
  }
}

// What the block copies to LDS ahead of a layer, in 16-byte chunks: its in_proj and x_proj
// weights (x_proj padded to 64 rows), then the RMSNorm gains of u, x and y and of the dt input
// (64 values), padded to a multiple of 1 KB.
// (The widest shape, d_model 512 and d_inner 1024, leaves no room for the gains: it reads
// them from global memory.)
constexpr bool dec_stage_gains(int Dm, int Di) { return Di * Dm <= 256 * 1024; }
constexpr int dec_gain_bytes(int Dm, int Di) {
  return dec_stage_gains(Dm, Di) ? (4 * Dm + 8 * Di + 256 + 1023) / 1024 * 1024 : 0;
}
constexpr int dec_stage_bytes(int Dm, int Di) { return Di * Dm / 4 + 64 * Di / 4 + dec_gain_bytes(Dm, Di); }

// One block of 512 threads per sequence; Dm = 64 KPM, Di = 64 KPL, NS states; the layers
// a.layer[0 .. nl - 1] in order, the activations between them kept in LDS.  A layer's in_proj
// and x_proj weights, gains and scales (what it needs first) are in LDS when it starts, fetched
// behind the previous layer's work; its other loads (out_proj, the channels' state and dt
// parameters) are issued as it starts and waited for where used.
template <typename T, int KPM, int KPL, int NS>
__global__ __launch_bounds__(512) void k_dec_stack(DecodeArgs a) {
  constexpr int DM = 64 * KPM, DI = 64 * KPL, SPL = NS / 4;
  constexpr int IT = DI / 16 / 8;           // in_proj tiles per wave
  // out_proj tiles per wave and round: registers for 32 packed words, no more than the rows need
  constexpr int OT = (32 + KPL - 1) / KPL < (DM / 16 + 7) / 8 ? (32 + KPL - 1) / KPL : (DM / 16 + 7) / 8;
  constexpr int WIN_B = DI * DM / 4, WX_B = 64 * DI / 4, STG_B = dec_stage_bytes(DM, DI);
  constexpr int NCH = STG_B / 16, NRND = (NCH + 511) / 512;  // 16-byte chunks, copy rounds
  // chunk ranges: W_in, W_x, then the gains g_in [DM], g_x [DI], g_out [DI], g_dt [64]
  constexpr bool SG = dec_stage_gains(DM, DI);
  constexpr int C_WX = WIN_B / 16, C_GI = C_WX + WX_B / 16, C_GX = C_GI + DM / 4, C_GO = C_GX + DI / 4,
                C_GD = C_GO + DI / 4, C_END = SG ? C_GD + 16 : C_GI;
  static_assert(STG_B % 1024 == 0 && WIN_B % 16 == 0 && C_END <= NCH, "whole waves of 16-byte chunks");
  __shared__ __align__(16) uint32_t s_w[STG_B / 4];  // W_in [Di][Dm / 16 words], W_x, gains
  __shared__ __align__(16) float s_sc[64];           // the four scales (s_in, s_x, s_dt, s_out)
  __shared__ __align__(16) int8_t s_q[DI];
  __shared__ __align__(16) float s_v[DI];   // x, then y
  __shared__ __align__(16) float s_u[DM];   // the layer's input (a value of the activation type)
  __shared__ float s_p[64];                 // dr | B | C (rounded to the activation type)
  __shared__ __align__(16) int8_t s_qd[64];
  __shared__ double s_deq[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = lane >> 4, lm = lane & 15;
  const int64_t b = blockIdx.x;
  const int nl = a.nl;
  // copy of layer l's weights and gains into s_w, 16-byte chunk i = tid + 512 r from thread
  // tid; a chunk with nothing to copy (W_x's padding rows, the dt gains past dt_rank, a gain
  // vector not given, the padding) loads the first chunk of W_in and is stored as well; the
  // four scales are loaded alike and stored by threads 0 .. 3.  Where the
  // chunks take at most 8 rounds (32 registers) and the layer's registers allow, the next
  // layer's are fetched into registers behind the current layer's work (plain loads, no wait
  // until their store at the next layer's start; the last layer issues as many loads, of one
  // chunk, so that every layer issues the same loads and the waits for earlier ones count them
  // exactly);
  // otherwise a layer's copy is made as it starts.
  constexpr bool PREF = NRND <= 8 && KPL <= 8;
  const int nwx = a.PW * DI / 64;    // W_x chunks
  const int ngd = (a.R + 3) / 4;     // g_dt chunks
  v4i pf[PREF ? NRND : 1];
  float pfs[4];
  auto chunk_src = [&](const DecodeLayer& Ls, int i) -> const v4i* {
    const uint8_t* win = (const uint8_t*)Ls.w_in;
    const uint8_t* src = win;
    if (i < C_WX) src = win + 16 * (int64_t)i;
    else if (i < C_GI) { if (i - C_WX < nwx) src = (const uint8_t*)Ls.w_x + 16 * (int64_t)(i - C_WX); }
    else if (!SG) {}
    else if (i < C_GX) { if (Ls.g_in) src = (const uint8_t*)Ls.g_in + 16 * (i - C_GI); }
    else if (i < C_GO) { if (Ls.g_x) src = (const uint8_t*)Ls.g_x + 16 * (i - C_GX); }
    else if (i < C_GD) { if (Ls.g_out) src = (const uint8_t*)Ls.g_out + 16 * (i - C_GO); }
    else if (i < C_END) { if (Ls.g_dt && i - C_GD < ngd) src = (const uint8_t*)Ls.g_dt + 16 * (i - C_GD); }
    return (const v4i*)src;
  };
  // (a gain vector not given is stored as ones)
  const v4i ones = v4i{0x3F800000, 0x3F800000, 0x3F800000, 0x3F800000};
  auto put_chunk = [&](int gm, int i, const v4i& v) {
    const bool one = SG && ((i >= C_GI && i < C_GX && !(gm & 1)) || (i >= C_GX && i < C_GO && !(gm & 2)) ||
                            (i >= C_GO && i < C_GD && !(gm & 4)) || (i >= C_GD && i < C_END && !(gm & 8)));
    if (i < NCH) *(v4i*)((uint8_t*)s_w + 16 * i) = one ? ones : v;
  };
  auto put_scales = [&]() {
    if (tid < 4) s_sc[tid] = tid == 0 ? pfs[0] : tid == 1 ? pfs[1] : tid == 2 ? pfs[2] : pfs[3];
  };
  auto fetch = [&](int l, bool real) {
    const DecodeLayer& Ls = a.layer[l];
#pragma unroll
    for (int r = 0; r < NRND; ++r) pf[r] = *(real ? chunk_src(Ls, tid + 512 * r) : (const v4i*)Ls.w_in);
    pfs[0] = Ls.s_in[0]; pfs[1] = Ls.s_x[0]; pfs[2] = Ls.s_dt[0]; pfs[3] = Ls.s_out[0];
  };
  auto put = [&](int l) {
    const int gm = a.layer[l].gains;
#pragma unroll
    for (int r = 0; r < NRND; ++r) put_chunk(gm, tid + 512 * r, pf[r]);
    put_scales();
  };
  // the copy made at once, four rounds at a time (for the shapes that do not prefetch)
  auto copy_now = [&](int l) {
    const DecodeLayer& Ls = a.layer[l];
    const int gm = Ls.gains;
#pragma unroll
    for (int r0 = 0; r0 < NRND; r0 += 4) {
      v4i v[4];
#pragma unroll
      for (int r = r0; r < r0 + 4 && r < NRND; ++r) v[r - r0] = *chunk_src(Ls, tid + 512 * r);
#pragma unroll
      for (int r = r0; r < r0 + 4 && r < NRND; ++r) put_chunk(gm, tid + 512 * r, v[r - r0]);
    }
    pfs[0] = Ls.s_in[0]; pfs[1] = Ls.s_x[0]; pfs[2] = Ls.s_dt[0]; pfs[3] = Ls.s_out[0];
    put_scales();
  };
  if constexpr (PREF) {
    fetch(0, true);
    put(0);
  } else {
    copy_now(0);
  }
  // the first layer's input
  const T* Ug = (const T*)a.u + b * a.Dm;
  for (int i = tid; i < DM; i += 512) s_u[i] = ld_act(Ug + i);
  const int Rr = a.R;
  const int Gl = Rr <= 16 ? 16 : (Rr <= 32 ? 32 : 64);
  const int gl = lane & (Gl - 1);
  const int ntx = (a.PW + 15) / 16;
  const int nto = (a.Dm + 15) / 16;
  constexpr int CPT = (DI + 511) / 512;
  const int RW = (a.R + 15) / 16;
  for (int l = 0; l < nl; ++l) {
    const DecodeLayer& Lw = a.layer[l];
    // layer l's copy into LDS (fetched during layer l - 1, or now); the barrier: everyone's
    // copy, and the previous layer's output in s_u
    if (l > 0) {
      if constexpr (PREF) put(l);
      else copy_now(l);
    }
    bar_lds();
    // gains (wave 0 normalises u, x, y and the dt input) and scales, from the copy in LDS
    const float* sg = (const float*)(s_w + C_GI * 4);
    const float* gi = SG ? sg : Lw.g_in;
    const float* gxp = SG ? sg + DM : Lw.g_x;
    const float* gop = SG ? sg + DM + DI : Lw.g_out;
    const float* gdp = SG ? sg + DM + 2 * DI : Lw.g_dt;
    // (in LDS a gain vector not given reads as ones: no test needed there)
    float gu[KPM], gx[KPL], gy[KPL], gdt = 1.0f;
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < KPM; ++i) gu[i] = (SG || Lw.g_in) ? gi[lane + 64 * i] : 1.0f;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        gx[i] = (SG || Lw.g_x) ? gxp[lane + 64 * i] : 1.0f;
        gy[i] = (SG || Lw.g_out) ? gop[lane + 64 * i] : 1.0f;
      }
      gdt = (SG || Lw.g_dt) ? gdp[gl < Rr ? gl : 0] : 1.0f;
    }
    const float sc_in = s_sc[0], sc_x = s_sc[1], sc_dt = s_sc[2], sc_out = s_sc[3];
    // u: norm and codes (wave 0, before its loads below: the other waves issue theirs meanwhile)
    if (wave == 0) norm_quant_one<KPM>(s_u, gu, DM, a.eps, s_q, &s_deq[0], lane);
    // the layer's loads from global memory: the first out_proj tiles (where registers allow,
    // else with the others), then the channels' state and parameters
    // (unconditional, tiles past the last repeating it, so that later waits count them exactly)
    constexpr bool kEarlyWo = KPL <= 8;
    uint32_t wo[OT][KPL];
    if (kEarlyWo) {
#pragma unroll
      for (int j = 0; j < OT; ++j)
        dec_load_w<KPL>(wo[j], Lw.w_out, a.Dm, wave + 8 * j < nto ? wave + 8 * j : nto - 1, lane);
    }
    // (two channels per thread at d_inner 1024: loaded after x_proj, where registers allow;
    // dt weight words past dt_rank repeat the last and are not used)
    float h[CPT][NS], Al[CPT][NS], bias[CPT], Dc[CPT];
    uint32_t wdw[CPT][4];
    auto load_ch = [&]() {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = tid + 512 * j < DI ? tid + 512 * j : DI - 1;
        const float4* st = (const float4*)(Lw.state + (b * a.Di + c) * NS);
        const float4* ar = (const float4*)(Lw.A + (int64_t)c * NS);
#pragma unroll
        for (int n4 = 0; n4 < NS / 4; ++n4) {
          const float4 hv = st[n4], av = ar[n4];
          h[j][4 * n4] = hv.x; h[j][4 * n4 + 1] = hv.y; h[j][4 * n4 + 2] = hv.z; h[j][4 * n4 + 3] = hv.w;
          Al[j][4 * n4] = av.x; Al[j][4 * n4 + 1] = av.y; Al[j][4 * n4 + 2] = av.z; Al[j][4 * n4 + 3] = av.w;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) wdw[j][q] = Lw.w_dt[(int64_t)c * a.w_dt_row_words + (q < RW ? q : RW - 1)];
        bias[j] = Lw.dt_bias ? Lw.dt_bias[c] : 0.0f;
        Dc[j] = Lw.D ? Lw.D[c] : 0.0f;
      }
    };
    constexpr bool kEarlyCh = CPT == 1;
    if (kEarlyCh) load_ch();
    bar_lds();
    // in_proj; x rounded to the activation type into LDS
    {
      const double sw = (double)sc_in, deq = s_deq[0];
      v4i bq[KPM];
      dec_codes<KPM>(bq, s_q, lane);
#pragma unroll
      for (int j = 0; j < IT; ++j) {
        uint32_t wi[KPM];
        dec_load_w<KPM>(wi, s_w, a.Di, wave + 8 * j, lane);
        const v4i acc = dec_tile<KPM>(wi, bq);
        if (lm == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = (wave + 8 * j) * 16 + kq * 4 + q;
            T r;
            st_act(&r, (float)((sw * (double)acc[q]) * deq));
            s_v[n] = act_f32(r);
          }
        }
      }
    }
    bar_lds();
    // x: norm and codes (wave 0); x_proj (waves 0 .. 3)
    if (wave == 0) norm_quant_one<KPL>(s_v, gx, DI, a.eps, s_q, &s_deq[0], lane);
    bar_lds();
    if (wave < ntx) {
      uint32_t wx[KPL];
      dec_load_w<KPL>(wx, s_w + WIN_B / 4, a.PW, wave, lane);
      v4i bq[KPL];
      dec_codes<KPL>(bq, s_q, lane);
      const v4i acc = dec_tile<KPL>(wx, bq);
      if (lm == 0) {
        const double sw = (double)sc_x, deq = s_deq[0];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = wave * 16 + kq * 4 + q;
          if (n < a.PW) {
            T r;
            st_act(&r, (float)((sw * (double)acc[q]) * deq));
            s_p[n] = act_f32(r);
          }
        }
      }
    }
    bar_lds();
    if (!kEarlyCh) load_ch();
    // the next layer's copy, in registers until that layer starts
    if constexpr (PREF) fetch(l + 1 < nl ? l + 1 : l, l + 1 < nl);
    // the dt input's codes: a group of G lanes (the standalone quantiser's order), wave 0
    if (wave == 0) {
      const int R = Rr, G = Gl;
      const float v = gl < R ? s_p[gl] : 0.0f;
      float sq = __builtin_fmaf(v, v, 0.0f);
      for (int dd = G / 2; dd >= 1; dd >>= 1) sq = sq + __shfl_xor(sq, dd, 64);
      const float ms = __fdiv_rn(sq, (float)R);
      const float r = __fdiv_rn(1.0f, sqrt_rn(ms + a.eps));
      float xh = v * r;
      if (SG || Lw.g_dt) xh = gl < R ? xh * gdt : 0.0f;  // (times 1 where no gains are given)
      float m = fabsf(xh);
      for (int dd = G / 2; dd >= 1; dd >>= 1) m = fmaxf(m, __shfl_xor(m, dd, 64));
      const float sigma = __fdiv_rn(127.0f, fmaxf(m, 1e-5f));
      float q = rintf(xh * sigma);
      q = fminf(fmaxf(q, -128.0f), 127.0f);
      s_qd[lane] = lane < R ? (int8_t)(int)q : (int8_t)0;
      if (lane == 0) s_deq[1] = (double)fmaxf(m, 1e-5f) / 127.0;
    }
    bar_lds();
    // every channel's dt and its states, one step; y rounded to the activation type
    {
      const float dq = (float)s_deq[1];
      const float* Bv = s_p + a.R;
      const float* Cv = s_p + a.R + NS;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = tid + 512 * j;
        if (c >= DI) continue;
        int acc = 0;
#pragma unroll
        for (int qw = 0; qw < 4; ++qw) {
          if (qw >= RW) continue;
          const v4i wd = unpack16_i8(wdw[j][qw]);
          const v4i cd = *(const v4i*)(s_qd + 16 * qw);
#pragma unroll
          for (int k = 0; k < 4; ++k) acc = __builtin_amdgcn_sdot4(cd[k], wd[k], acc, false);
        }
        float dtv = (sc_dt * (float)acc) * dq;
        dtv += bias[j];
        dtv = softplus_f(dtv);
        const float xv = s_v[c];
        const float ddy = dtv * xv;
        float y = 0.0f;
        if constexpr (NS == 16) {  // eight state pairs, summed in the scan's in-wave tree
          float pp[8];
#pragma unroll
          for (int g = 0; g < 8; ++g) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const int n = 2 * g + i;
              const float ab = __builtin_amdgcn_exp2f(dtv * (Al[j][n] * LOG2E));
              h[j][n] = __builtin_fmaf(ab, h[j][n], ddy * Bv[n]);
            }
            pp[g] = __builtin_fmaf(Cv[2 * g + 1], h[j][2 * g + 1], Cv[2 * g] * h[j][2 * g]);
          }
          y = ((pp[0] + pp[4]) + (pp[2] + pp[6])) + ((pp[1] + pp[5]) + (pp[3] + pp[7]));
        } else {  // four groups of NS / 4 states, added in order
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float yp = 0.0f;
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
              const int n = g * SPL + i;
              const float ab = __builtin_amdgcn_exp2f(dtv * (Al[j][n] * LOG2E));
              h[j][n] = __builtin_fmaf(ab, h[j][n], ddy * Bv[n]);
              yp = i == 0 ? Cv[n] * h[j][n] : __builtin_fmaf(Cv[n], h[j][n], yp);
            }
            y = g == 0 ? yp : y + yp;
          }
        }
        const float yo = y + Dc[j] * xv;
        T r;
        st_act(&r, yo);
        s_v[c] = act_f32(r);  // x of channel c is no longer needed
        float4* st = (float4*)(Lw.state + (b * a.Di + c) * NS);
#pragma unroll
        for (int n4 = 0; n4 < NS / 4; ++n4)
          st[n4] = make_float4(h[j][4 * n4], h[j][4 * n4 + 1], h[j][4 * n4 + 2], h[j][4 * n4 + 3]);
      }
    }
    bar_lds();
    // out_proj: y's norm and codes (wave 0), then the tiles, residual added in fp64; the
    // output rounded to the activation type goes to s_u (the next layer's input) or, after the
    // last layer, to out
    if (wave == 0) norm_quant_one<KPL>(s_v, gy, DI, a.eps, s_q, &s_deq[0], lane);
    bar_lds();
    const double sw = (double)sc_out, deq = s_deq[0];
    v4i bqy[KPL];
    dec_codes<KPL>(bqy, s_q, lane);
    T* Og = (T*)a.out + b * a.Dm;
    for (int t0 = 0; t0 < nto; t0 += 8 * OT) {
      if (t0 > 0 || !kEarlyWo) {
#pragma unroll
        for (int j = 0; j < OT; ++j)
          if (t0 + wave + 8 * j < nto) dec_load_w<KPL>(wo[j], Lw.w_out, a.Dm, t0 + wave + 8 * j, lane);
      }
#pragma unroll
      for (int j = 0; j < OT; ++j) {
        const int t = t0 + wave + 8 * j;
        if (t >= nto) continue;
        const v4i acc = dec_tile<KPL>(wo[j], bqy);
        if (lm == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = t * 16 + kq * 4 + q;
            if (n >= a.Dm) continue;
            double v = (sw * (double)acc[q]) * deq;
            if (a.add_residual) v += (double)s_u[n];
            T r;
            st_act(&r, (float)v);
            if (l + 1 < nl) s_u[n] = act_f32(r);
            else Og[n] = r;
          }
        }
      }
    }
  }
}

template <typename T, int KPM, int KPL>
hipError_t launch_dec_t(const DecodeArgs& a, hipStream_t s) {
  if (a.NS != 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_dec_stack<T, KPM, KPL, 16>), dim3((unsigned)a.B), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <typename T, int KPM>
hipError_t launch_dec_di(const DecodeArgs& a, hipStream_t s) {
  switch (a.Di) {
    case 128: return launch_dec_t<T, KPM, 2>(a, s);
    case 256: return launch_dec_t<T, KPM, 4>(a, s);
    case 512: return launch_dec_t<T, KPM, 8>(a, s);
    case 1024: return launch_dec_t<T, KPM, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  switch (a.Dm) {
    case 64: return launch_dec_di<T, 1>(a, s);
    case 128: return launch_dec_di<T, 2>(a, s);
    case 256: return launch_dec_di<T, 4>(a, s);
    case 512: return launch_dec_di<T, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

bool decode_supported(int Dm, int Di, int NS, int R, int PW) {
  const bool dm = Dm == 64 || Dm == 128 || Dm == 256 || Dm == 512;
  const bool di = Di == 128 || Di == 256 || Di == 512 || Di == 1024;
  return dm && di && NS == 16 && R >= 1 && R <= 64 && R % 4 == 0 && PW == R + 2 * NS && PW <= 64;
}

hipError_t launch_decode_m1(const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (!decode_supported(a.Dm, a.Di, a.NS, a.R, a.PW)) return hipErrorInvalidValue;
  return a.act_bf16 ? launch_decode_t<bf16_t>(a, s) : launch_decode_t<float>(a, s);
}

}  // namespace ssm
