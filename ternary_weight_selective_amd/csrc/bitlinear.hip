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
