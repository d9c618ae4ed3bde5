// Ternary contraction of BitLinear (TriSSM README: ternary weights, int8 activations; the
// TernarySSM abstract's multiply-free contraction; W1.58A16 from the Ternary Mamba abstract).
//
// A8: int8 codes x ternary weights -> exact int32 on gfx950 int8 MFMA (16x16x64).  The
// weights stay 2-bit in HBM; each K-step unpacks one packed tile into LDS as int8 and every
// wave of the tile reuses it.  Epilogue in fp64: (s_w * acc) (exact) times
// max(absmax, 1e-5) / 127, plus bias, plus residual, rounded once to fp32 (then bf16): the
// output is the correctly rounded value of that expression, so it does not depend on the
// tiling and the next projection's int8 codes see the same input as any exact evaluation.
// A16: bf16 normalised activations x ternary weights (unpacked to bf16 +-1 / 0) on bf16
// MFMA (16x16x32), fp32 accumulation, each group's partial times its scale.
#include "launch.hpp"

namespace ssm {

namespace {
constexpr int BM = 64, BN = 64, BK = 64;
constexpr int LDS_I8 = BK + 16;   // int8 row stride of the LDS tiles (bytes)
constexpr int LDS_BF = BK + 8;    // bf16 row stride (elements)

template <typename Tout, typename V>
__device__ __forceinline__ void store_out(const GemmArgs& a, int64_t m, int64_t n, V v) {
  if (a.bias) v += (V)a.bias[n];
  if (a.residual) v += (V)ld_act((const Tout*)a.residual + m * a.ld_res + n);
  st_act((Tout*)a.y + m * a.ldy + n, (float)v);
}
}  // namespace

// Grid: (ceil(N / 64), ceil(M / 64)); 4 waves, wave (wr, wc) owns a 32 x 32 quarter of the
// 64 x 64 output tile as 2 x 2 MFMA 16x16 blocks.
template <typename Tout, bool GROUPED, bool DBG>
__global__ __launch_bounds__(256) void k_gemm_i8(GemmArgs a) {
  __shared__ __align__(16) int8_t As[BM * LDS_I8];
  __shared__ __align__(16) int8_t Bs[BN * LDS_I8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
  const int8_t* A = (const int8_t*)a.A;
  v4i acc[2][2];
  double facc[2][2][4];
  int tot[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) { facc[i][j][r] = 0.0; tot[i][j][r] = 0; }
    }
  const int64_t ng = GROUPED ? a.K / a.group : 1;
  for (int64_t k0 = 0; k0 < a.Kp; k0 += BK) {
    {  // activation tile: 64 rows x 64 int8, 16 bytes per thread
      const int r = tid >> 2, c = (tid & 3) * 16;
      const int64_t gm = m0 + r;
      v4i val = v4i{0, 0, 0, 0};
      if (gm < a.M) val = *(const v4i*)(A + gm * a.lda + k0 + c);
      *(v4i*)(As + r * LDS_I8 + c) = val;
    }
    {  // weight tile: 64 output columns x 4 packed words -> int8 in LDS
      const int cn = tid >> 2, ws = tid & 3;
      const int64_t gn = n0 + cn, kw = k0 / 16 + ws;
      uint32_t wv = 0;
      if (gn < a.N && kw < a.w_row_words) wv = a.W[gn * a.w_row_words + kw];
      *(v4i*)(Bs + cn * LDS_I8 + ws * 16) = unpack16_i8(wv);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const v4i af = *(const v4i*)(As + (wr * 32 + i * 16 + (lane & 15)) * LDS_I8 + (lane >> 4) * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const v4i bf = *(const v4i*)(Bs + (wc * 32 + j * 16 + (lane & 15)) * LDS_I8 + (lane >> 4) * 16);
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf, acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
    if (GROUPED && ((k0 + BK) % a.group) == 0) {
      const int64_t g = k0 / a.group;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wc * 32 + j * 16 + (lane & 15);
        const double sc = n < a.N ? (double)a.w_scale[n * ng + g] : 0.0;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            facc[i][j][r] = facc[i][j][r] + sc * (double)acc[i][j][r];  // exact product, groups in order
            tot[i][j][r] += acc[i][j][r];
            acc[i][j][r] = 0;
          }
      }
    }
  }
  // epilogue: lane holds column (lane & 15) and rows 4 * (lane >> 4) + r of each 16x16 block
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wr * 32 + i * 16 + (lane >> 4) * 4 + r;
      if (m >= a.M) continue;
      const double deq = (double)fmaxf(a.absmax[m], 1e-5f) / 127.0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wc * 32 + j * 16 + (lane & 15);
        if (n >= a.N) continue;
        double v = GROUPED ? facc[i][j][r] : (double)a.w_scale[0] * (double)acc[i][j][r];
        v = v * deq;
        store_out<Tout>(a, m, n, v);
        if (DBG) a.dbg_acc[m * a.N + n] = GROUPED ? tot[i][j][r] : acc[i][j][r];
      }
    }
}

// A16: same tiling; bf16 MFMA 16x16x32, two per 64-deep K-step.  With SPLIT each activation
// is the sum of two bf16 terms (A + A2) and both are contracted (fp32-accurate outputs).
template <typename Tout, bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmArgs a) {
  __shared__ __align__(16) bf16_t As[BM * LDS_BF];
  __shared__ __align__(16) bf16_t As2[SPLIT ? BM * LDS_BF : 8];
  __shared__ __align__(16) bf16_t Bs[BN * LDS_BF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
  const bf16_t* A = (const bf16_t*)a.A;
  v4f acc[2][2];
  float facc[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) facc[i][j][r] = 0.0f;
    }
  const int64_t ng = a.group ? a.K / a.group : 1;
  const int64_t glen = a.group ? a.group : a.Kp;
  for (int64_t k0 = 0; k0 < a.Kp; k0 += BK) {
    {  // activation tile: 64 rows x 64 bf16, 32 bytes per thread
      const int r = tid >> 2, c = (tid & 3) * 16;
      const int64_t gm = m0 + r;
      v4i v0 = v4i{0, 0, 0, 0}, v1 = v4i{0, 0, 0, 0};
      if (gm < a.M) {
        const v4i* src = (const v4i*)(A + gm * a.lda + k0 + c);
        v0 = src[0];
        v1 = src[1];
      }
      v4i* dst = (v4i*)(As + r * LDS_BF + c);
      dst[0] = v0;
      dst[1] = v1;
      if (SPLIT) {
        v4i w0 = v4i{0, 0, 0, 0}, w1 = v4i{0, 0, 0, 0};
        if (gm < a.M) {
          const v4i* src = (const v4i*)((const bf16_t*)a.A2 + gm * a.lda + k0 + c);
          w0 = src[0];
          w1 = src[1];
        }
        v4i* dst2 = (v4i*)(As2 + r * LDS_BF + c);
        dst2[0] = w0;
        dst2[1] = w1;
      }
    }
    {  // weight tile: 16 codes per thread -> 16 bf16
      const int cn = tid >> 2, ws = tid & 3;
      const int64_t gn = n0 + cn, kw = k0 / 16 + ws;
      uint32_t wv = 0;
      if (gn < a.N && kw < a.w_row_words) wv = a.W[gn * a.w_row_words + kw];
      const v4i q = unpack16_i8(wv);
      v4i o0, o1;
      o0[0] = (int)tern2_to_bf16x2((uint32_t)q[0]);
      o0[1] = (int)tern2_to_bf16x2((uint32_t)q[0] >> 16);
      o0[2] = (int)tern2_to_bf16x2((uint32_t)q[1]);
      o0[3] = (int)tern2_to_bf16x2((uint32_t)q[1] >> 16);
      o1[0] = (int)tern2_to_bf16x2((uint32_t)q[2]);
      o1[1] = (int)tern2_to_bf16x2((uint32_t)q[2] >> 16);
      o1[2] = (int)tern2_to_bf16x2((uint32_t)q[3]);
      o1[3] = (int)tern2_to_bf16x2((uint32_t)q[3] >> 16);
      v4i* dst = (v4i*)(Bs + cn * LDS_BF + ws * 16);
      dst[0] = o0;
      dst[1] = o1;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int aoff = (wr * 32 + i * 16 + (lane & 15)) * LDS_BF + ks + (lane >> 4) * 8;
        const v8bf af = __builtin_bit_cast(v8bf, *(const v4i*)(As + aoff));
        v8bf af2;
        if (SPLIT) af2 = __builtin_bit_cast(v8bf, *(const v4i*)(As2 + aoff));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const v4i bi = *(const v4i*)(Bs + (wc * 32 + j * 16 + (lane & 15)) * LDS_BF + ks + (lane >> 4) * 8);
          const v8bf bfr = __builtin_bit_cast(v8bf, bi);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc[i][j], 0, 0, 0);
          if (SPLIT) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af2, bfr, acc[i][j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    if (((k0 + BK) % glen) == 0 || k0 + BK >= a.Kp) {
      const int64_t g = a.group ? k0 / a.group : 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wc * 32 + j * 16 + (lane & 15);
        const float sc = n < a.N ? (a.group ? a.w_scale[n * ng + g] : a.w_scale[0]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            facc[i][j][r] = __builtin_fmaf(acc[i][j][r], sc, facc[i][j][r]);
            acc[i][j][r] = 0.0f;
          }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wr * 32 + i * 16 + (lane >> 4) * 4 + r;
      if (m >= a.M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wc * 32 + j * 16 + (lane & 15);
        if (n < a.N) store_out<Tout>(a, m, n, facc[i][j][r]);
      }
    }
}


// ------------------------------------------------------------------------------------------
// Row-block A8 BitLinear for k <= 1024 (the HBM-bound projections): a block normalises and
// quantises BR = 16 token rows into LDS (one wave per row at a time, the fixed-order norm),
// then its 4 waves contract them against every 16-column tile of W with int8 MFMA 16x16x64
// (packed weights read from L2 and unpacked in registers) and write y from the
// accumulators with the fp64 epilogue.  x is read once and y written once.
namespace {
constexpr int BR = 16;            // token rows per block (one MFMA row tile)
constexpr int RPW = BR / 4;       // rows per wave in the norm phase
}

template <typename Tin, typename Tout, int KPL, bool DBG>
__global__ __launch_bounds__(256) void k_bl_rows(GemmArgs g, RowArgs r) {
  constexpr int KMAX = 64 * KPL;
  constexpr int QS = KMAX + 16;               // LDS row stride (bytes): conflict-free b128 reads
  constexpr int RB = KPL <= 8 ? RPW : (RPW < 4 ? RPW : 4);  // rows per load batch in the norm phase
  __shared__ __align__(16) int8_t s_q[BR * QS];
  __shared__ double s_deq[BR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * BR;
  const int K = (int)g.K;
  const Tin* X = (const Tin*)r.x;
  const int nct = (int)cdiv(g.N, 16);
  const double sw = (double)g.w_scale[0];
  auto load_w = [&](int ct, uint32_t* dst) {
    const int64_t n = (int64_t)ct * 16 + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < KPL; ++ks) {
      const int64_t kw = (int64_t)ks * 4 + (lane >> 4);
      dst[ks] = (n < g.N && kw < g.w_row_words) ? g.W[n * g.w_row_words + kw] : 0u;
    }
  };
  uint32_t wv[KPL];
  if (wave < nct) load_w(wave, wv);

  // 1. norm + int8 codes: wave w owns rows RPW w .. RPW w + RPW - 1
  for (int rb = 0; rb < RPW; rb += RB) {
    float v[RB][KPL];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int64_t row = m0 + wave * RPW + rb + rr;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int k = lane + 64 * i;
        v[rr][i] = (row < g.M && k < K) ? ld_act(X + row * r.ldx + k) : 0.0f;
      }
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int lr = wave * RPW + rb + rr;
      const int64_t row = m0 + lr;
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < KPL; ++i) s = __builtin_fmaf(v[rr][i], v[rr][i], s);
      s = wave_sum_butterfly(s);
      const float ms = __fdiv_rn(s, (float)K);
      const float rs = __fdiv_rn(1.0f, sqrt_rn(ms + r.eps));
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int k = lane + 64 * i;
        float t = v[rr][i] * rs;
        if (r.gain) t = (k < K) ? t * r.gain[k] : 0.0f;
        v[rr][i] = t;
        m = fmaxf(m, fabsf(t));
      }
      m = wave_max(m);
      const float sigma = __fdiv_rn(127.0f, fmaxf(m, 1e-5f));
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int k = lane + 64 * i;
        float q = rintf(v[rr][i] * sigma);
        q = fminf(fmaxf(q, -128.0f), 127.0f);
        s_q[lr * QS + k] = (int8_t)(int)q;
        if (DBG && r.dbg_xq && row < g.M && k < K) r.dbg_xq[row * K + k] = (int8_t)(int)q;
      }
      if (lane == 0) {
        s_deq[lr] = (double)fmaxf(m, 1e-5f) / 127.0;
        if (DBG && r.dbg_absmax && row < g.M) r.dbg_absmax[row] = m;
      }
    }
  }
  __syncthreads();

  // 2. contraction: wave w owns column tiles w, w + 4, ...; the next tile's packed weights
  //    are in flight while the current tile runs (the first tile's before the norm phase).
  for (int ct = wave; ct < nct; ct += 4) {
    const int64_t n = (int64_t)ct * 16 + (lane & 15);
    const bool nv = n < g.N;
    uint32_t wn[KPL];
    if (ct + 4 < nct) load_w(ct + 4, wn);
    constexpr int RT = BR / 16;  // MFMA row tiles
    v4i acc[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) acc[i] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KPL; ++ks) {
      const v4i bfr = unpack16_i8(wv[ks]);
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const v4i af = *(const v4i*)(s_q + (i * 16 + (lane & 15)) * QS + ks * 64 + (lane >> 4) * 16);
        acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bfr, acc[i], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lr = i * 16 + (lane >> 4) * 4 + q;
        const int64_t m = m0 + lr;
        if (m < g.M && nv) {
          double y = sw * (double)acc[i][q];
          y = y * s_deq[lr];
          store_out<Tout>(g, m, n, y);
          if (DBG && g.dbg_acc) g.dbg_acc[m * g.N + n] = acc[i][q];
        }
      }
#pragma unroll
    for (int ks = 0; ks < KPL; ++ks) wv[ks] = wn[ks];
  }
}

hipError_t launch_gemm_i8(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv(a.N, BN), (unsigned)cdiv(a.M, BM)), block(256);
  const bool g = a.group > 0, d = a.dbg_acc != nullptr;
#define SSM_GEMM_I8(T, G, D) hipLaunchKernelGGL((k_gemm_i8<T, G, D>), grid, block, 0, s, a)
  if (a.y_bf16) {
    if (g) { if (d) SSM_GEMM_I8(bf16_t, true, true); else SSM_GEMM_I8(bf16_t, true, false); }
    else { if (d) SSM_GEMM_I8(bf16_t, false, true); else SSM_GEMM_I8(bf16_t, false, false); }
  } else {
    if (g) { if (d) SSM_GEMM_I8(float, true, true); else SSM_GEMM_I8(float, true, false); }
    else { if (d) SSM_GEMM_I8(float, false, true); else SSM_GEMM_I8(float, false, false); }
  }
#undef SSM_GEMM_I8
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv(a.N, BN), (unsigned)cdiv(a.M, BM)), block(256);
  if (a.y_bf16) {
    if (a.A2) hipLaunchKernelGGL((k_gemm_bf16<bf16_t, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm_bf16<bf16_t, false>), grid, block, 0, s, a);
  } else {
    if (a.A2) hipLaunchKernelGGL((k_gemm_bf16<float, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm_bf16<float, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ssm

namespace ssm {
template <typename Tin, typename Tout, int KPL>
static void launch_rows_t(const GemmArgs& g, const RowArgs& r, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(g.M, BR)), block(256);
  if (g.dbg_acc || r.dbg_xq || r.dbg_absmax)
    hipLaunchKernelGGL((k_bl_rows<Tin, Tout, KPL, true>), grid, block, 0, s, g, r);
  else
    hipLaunchKernelGGL((k_bl_rows<Tin, Tout, KPL, false>), grid, block, 0, s, g, r);
}

template <typename Tin, typename Tout>
static hipError_t launch_rows_k(const GemmArgs& g, const RowArgs& r, hipStream_t s) {
  if (g.K <= 64) launch_rows_t<Tin, Tout, 1>(g, r, s);
  else if (g.K <= 128) launch_rows_t<Tin, Tout, 2>(g, r, s);
  else if (g.K <= 256) launch_rows_t<Tin, Tout, 4>(g, r, s);
  else if (g.K <= 512) launch_rows_t<Tin, Tout, 8>(g, r, s);
  else if (g.K <= 1024) launch_rows_t<Tin, Tout, 16>(g, r, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bitlinear_rows(const GemmArgs& g, const RowArgs& r, hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  if (g.group != 0) return hipErrorInvalidValue;
  if (r.x_bf16) return g.y_bf16 ? launch_rows_k<bf16_t, bf16_t>(g, r, s) : launch_rows_k<bf16_t, float>(g, r, s);
  return g.y_bf16 ? launch_rows_k<float, bf16_t>(g, r, s) : launch_rows_k<float, float>(g, r, s);
}
}  // namespace ssm
