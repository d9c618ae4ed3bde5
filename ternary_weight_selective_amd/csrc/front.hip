// Front of the Mamba-1 kind mixer (TriSSM README: the BitLinear projections that produce the
// input-dependent Delta, B, C; Mamba, cited by title in "Baseline Shape Decides the Verdict
// ...", Builds on): x = BitLinear(u; W_in), p = BitLinear(x; W_x) = [dr | B | C], and the int8
// codes + fp64 dequantisation factors of dr, the input of the dt projection that the scan
// evaluates, in one persistent kernel.  x still goes to HBM (the scan reads it) but is not read
// back: x_proj takes it from LDS.
//
// A block of 8 waves walks over blocks of 16 token rows (row block blockIdx.x, + gridDim.x,
// ...).  Per row block, three phases separated by LDS-only barriers:
//   A  producers (waves 0-3) normalise and quantise the NEXT row block's u (4 rows each, the
//      fixed-order norm) into one of two code buffers and, behind it, quantise the previous
//      row block's dr; consumers (waves 4-7) contract this row block's codes with W_in
//      (int8 MFMA 16x16x64) and write x, rounded to the activation type, to HBM and to LDS;
//   B  all 8 waves normalise and quantise x from LDS (2 rows each);
//   C  consumers contract those codes with W_x and write p to HBM and dr to LDS.
// Every value is the one the separate kernels compute: the same fixed-order norm, the same
// fp64 epilogue, the same rounding of x and p to the activation type before they are used.
#include "launch.hpp"

namespace ssm {

namespace {
constexpr int FBR = 16;     // token rows per row block
constexpr int FRMAX = 64;   // widest dr


template <typename T> struct V4;
template <> struct V4<float> { typedef float4 type; };
template <> struct V4<bf16_t> { typedef uint2 type; };

}  // namespace

template <typename T, int KPL1, int KPL2>
__global__ __launch_bounds__(512) void k_m1_front(FrontArgs f) {
  constexpr int BR = FBR;
  constexpr int QS1 = 64 * KPL1 + 16, QS2 = 64 * KPL2 + 16;
  constexpr int DIM = 64 * KPL2;                        // x row stride in LDS (floats)
  constexpr int TPR = (32 / KPL1) < 8 ? (32 / KPL1) : 8;  // in_proj tiles per weight round
  __shared__ __align__(16) int8_t s_q1[2][BR * QS1];
  __shared__ double s_deq1[2][BR];
  __shared__ __align__(16) float s_x[BR * DIM];
  // element (r, c) of x in s_x: the 16-byte granule c / 4 of row r at position (c / 4) ^ (r mod 8),
  // so that the in_proj epilogue's 16-byte writes (16 rows at one column) spread over the banks
  auto xs = [](int r, int c) { return r * DIM + ((((c >> 2) ^ (r & 7))) << 2) + (c & 3); };
  __shared__ __align__(16) int8_t s_q2[BR * QS2];
  __shared__ double s_deq2[BR];
  __shared__ float s_dr[BR * FRMAX];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = lane >> 4, lm = lane & 15;
  const int64_t M = f.M;
  const int Dm = f.Dm, Di = f.Di, PW = f.PW, R = f.R;
  const int64_t nrb = cdiv(M, BR), G = gridDim.x, b = blockIdx.x;
  const int niter = b < nrb ? (int)((nrb - 1 - b) / G + 1) : 0;
  if (niter == 0) return;
  const T* U = (const T*)f.u;
  T* X = (T*)f.x;
  T* Pp = (T*)f.p;
  auto row0 = [&](int it) { return (b + (int64_t)it * G) * BR; };

  // ---------------- producer state: u rows (RPW = 4 per wave) ----------------
  float gn1[KPL1];
#pragma unroll
  for (int i = 0; i < KPL1; ++i) gn1[i] = f.g_in ? f.g_in[lane + 64 * i] : 1.0f;
  float vc[4][KPL1], vn[4][KPL1];
  auto load_u = [&](int it, float (&v)[4][KPL1]) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      int64_t row = row0(it) + wave * 4 + rr;
      row = row < M ? row : M - 1;
      const T* ur = U + row * Dm;
#pragma unroll
      for (int i = 0; i < KPL1; ++i) v[rr][i] = ld_act(ur + lane + 64 * i);
    }
  };
  auto norm_u = [&](int it, float (&v)[4][KPL1]) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const bool rv = row0(it) + wave * 4 + rr < M;
#pragma unroll
      for (int i = 0; i < KPL1; ++i) v[rr][i] = rv ? v[rr][i] : 0.0f;
    }
    norm_quant_rows<4, KPL1>(v, gn1, Dm, f.eps, &s_q1[it & 1][wave * 4 * QS1], QS1, &s_deq1[it & 1][wave * 4], lane);
  };
  // dt input codes of row block it (from dr in LDS), G-lane groups, one token per group; the
  // lane's gain is loaded once, here
  const int Gl = R <= 16 ? 16 : (R <= 32 ? 32 : 64);
  const int gl = lane & (Gl - 1);
  const float gdt = f.g_dt ? f.g_dt[gl < R ? gl : 0] : 1.0f;
  auto dt_codes = [&](int it) {
    const int tpw = 64 / Gl;
    for (int t0 = 0; t0 < BR; t0 += 4 * tpw) {
      const int t = t0 + wave * tpw + lane / Gl;
      const int64_t tok = row0(it) + t;
      const float v = (t < BR && gl < R) ? s_dr[t * FRMAX + gl] : 0.0f;
      float s = __builtin_fmaf(v, v, 0.0f);
      for (int dd = Gl / 2; dd >= 1; dd >>= 1) s = s + __shfl_xor(s, dd, 64);
      const float ms = __fdiv_rn(s, (float)R);
      const float r = __fdiv_rn(1.0f, sqrt_rn(ms + f.eps));
      float xh = v * r;
      if (f.g_dt) xh = gl < R ? xh * gdt : 0.0f;
      float m = fabsf(xh);
      for (int dd = Gl / 2; dd >= 1; dd >>= 1) m = fmaxf(m, __shfl_xor(m, dd, 64));
      const float sigma = __fdiv_rn(127.0f, fmaxf(m, 1e-5f));
      float q = rintf(xh * sigma);
      q = fminf(fmaxf(q, -128.0f), 127.0f);
      if (t < BR && tok < M) {
        if (gl < f.cw) f.codes[tok * f.cw + gl] = (int8_t)(int)q;
        if (gl == 0) f.deq[tok] = (double)fmaxf(m, 1e-5f) / 127.0;
      }
    }
  };

  // ---------------- consumer state: weights ----------------
  const int cw_ = wave - 4;
  const int nct1 = (int)cdiv(Di, 16), tpw1 = (nct1 + 3) / 4;
  const int ct0 = cw_ * tpw1, ct1 = (ct0 + tpw1 < nct1) ? ct0 + tpw1 : nct1;
  const bool one_round = ct1 - ct0 <= TPR;
  uint32_t wv[TPR][KPL1];
  const int wrw1 = Dm / 16, wrw2 = Di / 16;
  // every load is issued (rows past the weight clamped to row 0) before any is selected, so the
  // loads of a round are in flight together rather than one round trip each
  auto load_round = [&](int c) {
    uint32_t raw[TPR][KPL1];
#pragma unroll
    for (int j = 0; j < TPR; ++j) {
      const int n = (c + j) * 16 + lm;
      const bool ok = (c + j < ct1) && n < Di;
      const uint32_t* wr = f.w_in + (int64_t)(ok ? n : 0) * wrw1 + kq * KPL1;
#pragma unroll
      for (int ks = 0; ks < KPL1; ++ks) raw[j][ks] = wr[ks];
    }
#pragma unroll
    for (int j = 0; j < TPR; ++j) {
      const int n = (c + j) * 16 + lm;
      const bool ok = (c + j < ct1) && n < Di;
#pragma unroll
      for (int ks = 0; ks < KPL1; ++ks) wv[j][ks] = ok ? raw[j][ks] : 0u;
    }
  };
  const int nct2 = (int)cdiv(PW, 16);
  uint32_t wx[KPL2];
  {
    const int n = cw_ * 16 + lm;
    const bool ok = wave >= 4 && cw_ < nct2 && n < PW;
    const uint32_t* wr = f.w_x + (int64_t)(ok ? n : 0) * wrw2 + kq * KPL2;
    uint32_t raw[KPL2];
#pragma unroll
    for (int ks = 0; ks < KPL2; ++ks) raw[ks] = wr[ks];
#pragma unroll
    for (int ks = 0; ks < KPL2; ++ks) wx[ks] = ok ? raw[ks] : 0u;
  }
  if (wave >= 4 && ct0 < ct1) load_round(ct0);
  const double sw1 = (double)f.s_in[0], sw2 = (double)f.s_x[0];
  const int vb = (int)sizeof(typename V4<T>::type);
  const bool vx = (Di % 4 == 0) && ((uintptr_t)X % vb == 0);
  const bool vp = (PW % 4 == 0) && ((uintptr_t)Pp % vb == 0);

  // ---------------- prologue ----------------
  if (wave < 4) {
    load_u(0, vc);
    norm_u(0, vc);
    if (niter > 1) load_u(1, vn);
  }
  bar_lds();

  for (int it = 0; it < niter; ++it) {
    const int64_t m0 = row0(it);
    // ---- phase A ----
    if (wave < 4) {
      if (it + 1 < niter) {
        norm_u(it + 1, vn);
        if (it + 2 < niter) load_u(it + 2, vn);
      }
      if (it >= 1) dt_codes(it - 1);
    } else {
      const int buf = it & 1;
      const double deq = s_deq1[buf][lm];
      const int64_t m = m0 + lm;
      v4i bq[KPL1];
#pragma unroll
      for (int ks = 0; ks < KPL1; ++ks) bq[ks] = *(const v4i*)(&s_q1[buf][lm * QS1 + (kq * KPL1 + ks) * 16]);
      for (int c = ct0; c < ct1; c += TPR) {
        if (!one_round && !(c == ct0 && it == 0)) load_round(c);
        v4i acc[TPR];
#pragma unroll
        for (int j = 0; j < TPR; ++j) {
          acc[j] = v4i{0, 0, 0, 0};
          if (c + j < ct1) {
#pragma unroll
            for (int ks = 0; ks < KPL1; ++ks)
              acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16_i8(wv[j][ks]), bq[ks], acc[j], 0, 0, 0);
          }
        }
#pragma unroll
        for (int j = 0; j < TPR; ++j) {
          const int n = (c + j) * 16 + kq * 4;
          if (c + j >= ct1 || n >= Di) continue;
          T o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) st_act(&o[q], (float)((sw1 * (double)acc[j][q]) * deq));
          *(float4*)(&s_x[xs(lm, n)]) = make_float4(ld_act(&o[0]), ld_act(&o[1]), ld_act(&o[2]), ld_act(&o[3]));
          if (m < M) {
            if (vx && n + 3 < Di) {
              *(typename V4<T>::type*)(X + m * Di + n) = *(const typename V4<T>::type*)o;
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (n + q < Di) X[m * Di + n + q] = o[q];
            }
          }
        }
      }
    }
    bar_lds();
    // ---- phase B: x rows 2 wave, 2 wave + 1 ----
    {
      float v[2][KPL2], gn2[KPL2];
#pragma unroll
      for (int i = 0; i < KPL2; ++i) gn2[i] = f.g_x ? f.g_x[lane + 64 * i] : 1.0f;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int r = wave * 2 + rr;
        const bool rv = m0 + r < M;
#pragma unroll
        for (int i = 0; i < KPL2; ++i) v[rr][i] = rv ? s_x[xs(r, lane + 64 * i)] : 0.0f;
      }
      norm_quant_rows<2, KPL2>(v, gn2, Di, f.eps, &s_q2[wave * 2 * QS2], QS2, &s_deq2[wave * 2], lane);
    }
    bar_lds();
    // ---- phase C: x_proj ----
    if (wave >= 4 && cw_ < nct2) {
      const double deq = s_deq2[lm];
      const int64_t m = m0 + lm;
      v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KPL2; ++ks) {
        const v4i bq = *(const v4i*)(&s_q2[lm * QS2 + (kq * KPL2 + ks) * 16]);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16_i8(wx[ks]), bq, acc, 0, 0, 0);
      }
      const int n = cw_ * 16 + kq * 4;
      if (n < PW) {
        T o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) st_act(&o[q], (float)((sw2 * (double)acc[q]) * deq));
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (n + q < R) s_dr[lm * FRMAX + n + q] = ld_act(&o[q]);
        if (m < M) {
          if (vp && n + 3 < PW) {
            *(typename V4<T>::type*)(Pp + m * PW + n) = *(const typename V4<T>::type*)o;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (n + q < PW) Pp[m * PW + n + q] = o[q];
          }
        }
      }
    }
    bar_lds();
  }
  if (wave < 4) dt_codes(niter - 1);
}

// Shapes whose registers fit without spilling: d_model 64 .. 512, d_inner 128 .. 1024, but not
// both 512 and 1024.
bool front_supported(int Dm, int Di, int PW, int R) {
  const bool dm = Dm == 64 || Dm == 128 || Dm == 256 || Dm == 512;
  const bool di = Di == 128 || Di == 256 || Di == 512 || Di == 1024;
  return dm && di && !(Dm == 512 && Di == 1024) && PW <= 64 && R >= 1 && R <= FRMAX && R <= PW;
}

namespace {
template <typename T, int KPL1, int KPL2>
void launch_front_t(const FrontArgs& f, hipStream_t s) {
  const int64_t nrb = cdiv(f.M, FBR);
  const dim3 grid((unsigned)(nrb < 256 ? nrb : 256)), block(512);
  hipLaunchKernelGGL((k_m1_front<T, KPL1, KPL2>), grid, block, 0, s, f);
}

template <typename T, int KPL1>
hipError_t launch_front_k2(const FrontArgs& f, hipStream_t s) {
  switch (f.Di) {
    case 128: launch_front_t<T, KPL1, 2>(f, s); break;
    case 256: launch_front_t<T, KPL1, 4>(f, s); break;
    case 512: launch_front_t<T, KPL1, 8>(f, s); break;
    case 1024: launch_front_t<T, KPL1, 16>(f, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_front_k1(const FrontArgs& f, hipStream_t s) {
  switch (f.Dm) {
    case 64: return launch_front_k2<T, 1>(f, s);
    case 128: return launch_front_k2<T, 2>(f, s);
    case 256: return launch_front_k2<T, 4>(f, s);
    case 512: return launch_front_k2<T, 8>(f, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_m1_front(const FrontArgs& f, hipStream_t s) {
  if (f.M == 0) return hipSuccess;
  if (!front_supported(f.Dm, f.Di, f.PW, f.R)) return hipErrorInvalidValue;
  return f.act_bf16 ? launch_front_k1<bf16_t>(f, s) : launch_front_k1<float>(f, s);
}

}  // namespace ssm
