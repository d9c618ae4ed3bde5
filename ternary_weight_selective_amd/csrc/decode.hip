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
// readout order (four groups of NS / 4 states, each accumulated by fused multiply-adds, the
// groups added in order, then D x).
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

// x_proj / out_proj of the block's one token: 16-wide output tiles t of W [n_out, 64 KPL]
// (packed), the token's codes (LDS, 64 KPL bytes) as lane group 0 of the B operand.  Returns
// the int32 sums of outputs 16 t + 4 kq .. + 3 in lanes with lm == 0.
template <int KPL>
__device__ __forceinline__ v4i dec_tile(const uint32_t (&w)[KPL], const int8_t* sq, int lane) {
  const int kq = lane >> 4, lm = lane & 15;
  v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < KPL; ++ks) {
    const v4i b = lm == 0 ? *(const v4i*)(sq + (kq * KPL + ks) * 16) : v4i{0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16_i8(w[ks]), b, acc, 0, 0, 0);
  }
  return acc;
}

// Lane (n, kq) of tile t: packed words kq KPL .. kq KPL + KPL - 1 of row 16 t + n (rows of
// 4 KPL words; 16-byte loads when KPL is a multiple of 4, the rows then being 16-byte aligned
// whenever W is).  Rows past n_out read row n_out - 1 and are zeroed.
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
  if (n >= n_out) {
#pragma unroll
    for (int ks = 0; ks < KPL; ++ks) w[ks] = 0u;
  }
}

// One block of 512 threads per sequence; Dm = 64 KPM, Di = 64 KPL, NS states.
template <typename T, int KPM, int KPL, int NS>
__global__ __launch_bounds__(512) void k_dec_layer(DecodeArgs a) {
  constexpr int DM = 64 * KPM, DI = 64 * KPL, SPL = NS / 4;
  constexpr int IT = DI / 16 / 8;           // in_proj tiles per wave
  constexpr int OT = (32 + KPL - 1) / KPL;  // out_proj tiles per wave and round
  __shared__ __align__(16) int8_t s_q[DI];
  __shared__ __align__(16) float s_v[DI];   // x, then y
  __shared__ float s_p[64];                 // dr | B | C (rounded to the activation type)
  __shared__ __align__(16) int8_t s_qd[64];
  __shared__ double s_deq[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = lane >> 4, lm = lane & 15;
  const int64_t b = blockIdx.x;
  const T* Ug = (const T*)a.u + b * a.Dm;
  // loads first: u, the in_proj tiles, the x_proj tile of waves 0 .. 3, the first round of
  // out_proj tiles, the channels' state and parameters, the residual
  float uv[1][KPM], gu[KPM];
#pragma unroll
  for (int i = 0; i < KPM; ++i) {
    uv[0][i] = ld_act(Ug + lane + 64 * i);
    gu[i] = a.g_in ? a.g_in[lane + 64 * i] : 1.0f;
  }
  uint32_t wi[IT][KPM];
#pragma unroll
  for (int j = 0; j < IT; ++j) dec_load_w<KPM>(wi[j], a.w_in, a.Di, wave + 8 * j, lane);
  // gains (x, y: wave 0 normalises both; the dt input's, per lane) and the four scales
  float gx[KPL], gy[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    gx[i] = a.g_x ? a.g_x[lane + 64 * i] : 1.0f;
    gy[i] = a.g_out ? a.g_out[lane + 64 * i] : 1.0f;
  }
  const int Rr = a.R;
  const int Gl = Rr <= 16 ? 16 : (Rr <= 32 ? 32 : 64);
  const int gl = lane & (Gl - 1);
  const float gdt = a.g_dt ? a.g_dt[gl < Rr ? gl : 0] : 1.0f;
  const float sc_in = a.s_in[0], sc_x = a.s_x[0], sc_dt = a.s_dt[0], sc_out = a.s_out[0];
  // u: norm and codes (wave 0, as soon as u has arrived); the other loads go out behind it
  if (wave == 0) norm_quant_rows<1, KPM>(uv, gu, DM, a.eps, s_q, 0, &s_deq[0], lane);
  const int ntx = (a.PW + 15) / 16;
  uint32_t wx[KPL];
  if (wave < ntx) dec_load_w<KPL>(wx, a.w_x, a.PW, wave, lane);
  const int nto = (a.Dm + 15) / 16;
  uint32_t wo[OT][KPL];
#pragma unroll
  for (int j = 0; j < OT; ++j)
    if (wave + 8 * j < nto) dec_load_w<KPL>(wo[j], a.w_out, a.Dm, wave + 8 * j, lane);
  // the thread's channels c = tid + 512 j: state, A, dt weights, bias, D
  constexpr int CPT = (DI + 511) / 512;
  const int RW = (a.R + 15) / 16;
  float h[CPT][NS], Al[CPT][NS], bias[CPT], Dc[CPT];
  uint32_t wdw[CPT][4];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = tid + 512 * j < DI ? tid + 512 * j : DI - 1;
    const float4* st = (const float4*)(a.state + (b * a.Di + c) * NS);
    const float4* ar = (const float4*)(a.A + (int64_t)c * NS);
#pragma unroll
    for (int n4 = 0; n4 < NS / 4; ++n4) {
      const float4 hv = st[n4], av = ar[n4];
      h[j][4 * n4] = hv.x; h[j][4 * n4 + 1] = hv.y; h[j][4 * n4 + 2] = hv.z; h[j][4 * n4 + 3] = hv.w;
      Al[j][4 * n4] = av.x; Al[j][4 * n4 + 1] = av.y; Al[j][4 * n4 + 2] = av.z; Al[j][4 * n4 + 3] = av.w;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) wdw[j][q] = q < RW ? a.w_dt[(int64_t)c * a.w_dt_row_words + q] : 0u;
    bias[j] = a.dt_bias ? a.dt_bias[c] : 0.0f;
    Dc[j] = a.D ? a.D[c] : 0.0f;
  }
  // the residual of the out_proj outputs this lane writes (first round of tiles)
  float res[OT][4];
#pragma unroll
  for (int j = 0; j < OT; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = (wave + 8 * j) * 16 + kq * 4 + q;
      res[j][q] = (a.add_residual && n < a.Dm) ? ld_act(Ug + n) : 0.0f;
    }
  bar_lds();
  // in_proj; x rounded to the activation type into LDS
  {
    const double sw = (double)sc_in, deq = s_deq[0];
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      const v4i acc = dec_tile<KPM>(wi[j], s_q, lane);
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
    const v4i acc = dec_tile<KPL>(wx, s_q, lane);
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
  // the dt input's codes: a group of G lanes (the standalone quantiser's order), wave 0
  if (wave == 0) {
    const int R = Rr, G = Gl;
    const float gv = gdt;
    const float v = gl < R ? s_p[gl] : 0.0f;
    float s = __builtin_fmaf(v, v, 0.0f);
    for (int dd = G / 2; dd >= 1; dd >>= 1) s = s + __shfl_xor(s, dd, 64);
    const float ms = __fdiv_rn(s, (float)R);
    const float r = __fdiv_rn(1.0f, sqrt_rn(ms + a.eps));
    float xh = v * r;
    if (a.g_dt) xh = gl < R ? xh * gv : 0.0f;
    float m = fabsf(xh);
    for (int dd = G / 2; dd >= 1; dd >>= 1) m = fmaxf(m, __shfl_xor(m, dd, 64));
    const float sigma = __fdiv_rn(127.0f, fmaxf(m, 1e-5f));
    float q = rintf(xh * sigma);
    q = fminf(fmaxf(q, -128.0f), 127.0f);
    if (lane < 64) s_qd[lane] = lane < R ? (int8_t)(int)q : (int8_t)0;
    if (lane == 0) s_deq[1] = (double)fmaxf(m, 1e-5f) / 127.0;
  }
  bar_lds();
  // every channel's dt and its states, one step; y rounded to the activation type
  {
    const float s_dt = sc_dt;
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
      float dtv = (s_dt * (float)acc) * dq;
      dtv += bias[j];
      dtv = softplus_f(dtv);
      const float xv = s_v[c];
      const float ddy = dtv * xv;
      float y = 0.0f;
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
      const float yo = y + Dc[j] * xv;
      T r;
      st_act(&r, yo);
      s_v[c] = act_f32(r);  // x of channel c is no longer needed
      float4* st = (float4*)(a.state + (b * a.Di + c) * NS);
#pragma unroll
      for (int n4 = 0; n4 < NS / 4; ++n4)
        st[n4] = make_float4(h[j][4 * n4], h[j][4 * n4 + 1], h[j][4 * n4 + 2], h[j][4 * n4 + 3]);
    }
  }
  bar_lds();
  // out_proj: y's norm and codes (wave 0), then the tiles, residual added in fp64
  if (wave == 0) norm_quant_one<KPL>(s_v, gy, DI, a.eps, s_q, &s_deq[0], lane);
  bar_lds();
  const double sw = (double)sc_out, deq = s_deq[0];
  T* Og = (T*)a.out + b * a.Dm;
  for (int t0 = 0; t0 < nto; t0 += 8 * OT) {
    if (t0 > 0) {
#pragma unroll
      for (int j = 0; j < OT; ++j)
        if (t0 + wave + 8 * j < nto) dec_load_w<KPL>(wo[j], a.w_out, a.Dm, t0 + wave + 8 * j, lane);
    }
#pragma unroll
    for (int j = 0; j < OT; ++j) {
      const int t = t0 + wave + 8 * j;
      if (t >= nto) continue;
      const v4i acc = dec_tile<KPL>(wo[j], s_q, lane);
      if (lm == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = t * 16 + kq * 4 + q;
          if (n >= a.Dm) continue;
          double v = (sw * (double)acc[q]) * deq;
          if (a.add_residual) v += (double)(t0 == 0 ? res[j][q] : ld_act(Ug + n));
          st_act(Og + n, (float)v);
        }
      }
    }
  }
}

template <typename T, int KPM, int KPL>
hipError_t launch_dec_t(const DecodeArgs& a, hipStream_t s) {
  if (a.NS != 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_dec_layer<T, KPM, KPL, 16>), dim3((unsigned)a.B), dim3(512), 0, s, a);
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
  return dm && di && NS == 16 && R >= 1 && R <= 64 && PW == R + 2 * NS && PW <= 64;
}

hipError_t launch_decode_m1(const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (!decode_supported(a.Dm, a.Di, a.NS, a.R, a.PW)) return hipErrorInvalidValue;
  return a.act_bf16 ? launch_decode_t<bf16_t>(a, s) : launch_decode_t<float>(a, s);
}

}  // namespace ssm
