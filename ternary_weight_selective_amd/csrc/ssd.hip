// Selective scan, SSD kind ("Transformers are SSMs", cited by title in "SSDi8 ...", Builds
// on; the Mamba-2 shape of the Ternary Mamba abstract): scalar A per head, a state of
// headdim x d_state per head, B and C shared by all heads.
//
// Two evaluations: the chunked one on the matrix cores (below, bf16 activations, headdim 64,
// d_state 64 or 128), and a recurrent one for every other shape: each lane owns 8 states of
// one (head, channel) pair; the d_state / 8 lanes of a channel add their readout partials with
// xor shuffles.  The decay exp(dt A) is one value per (token, head), computed once per tile.
#include "launch.hpp"

namespace ssm {

namespace {
__device__ __forceinline__ float softplus_s(float v) { return v > 20.0f ? v : log1pf(expf(v)); }
}  // namespace

template <int NS, typename T>
__global__ __launch_bounds__(256) void k_scan_ssd_rec(ScanArgs a) {
  constexpr int SPL = 8;
  constexpr int LPP = NS / SPL;    // lanes per channel
  constexpr int PPB = 256 / LPP;   // channels per block
  constexpr int TT = 32;
  __shared__ float s_B[TT][NS];
  __shared__ float s_C[TT][NS];
  __shared__ float s_a[TT];
  __shared__ float s_dt[TT];
  __shared__ float s_ux[TT][PPB];
  __shared__ float s_dx[TT][PPB];
  __shared__ float s_y[TT][PPB];

  const int tid = threadIdx.x;
  const int64_t L = a.L, H = a.H, P = a.P;
  const int64_t hd = blockIdx.y, b = blockIdx.z;
  const int pl = tid / LPP, qq = tid % LPP;
  const int64_t p = (int64_t)blockIdx.x * PPB + pl;
  const bool pv = p < P;
  const float A_h = a.A[hd];
  const float bias_h = a.delta_bias ? a.delta_bias[hd] : 0.0f;
  const float D_h = a.D ? a.D[hd] : 0.0f;
  const T* X = (const T*)a.x;
  const T* DT = (const T*)a.delta;
  const T* Bm = (const T*)a.Bm;
  const T* Cm = (const T*)a.Cm;
  T* Y = (T*)a.y;

  float h[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i)
    h[i] = (pv && a.h0) ? a.h0[((b * H + hd) * P + p) * NS + qq * SPL + i] : 0.0f;

  for (int64_t t0 = 0; t0 < L; t0 += TT) {
    for (int e = tid; e < TT * NS; e += 256) {
      const int t = e / NS, n = e % NS;
      const bool valid = t0 + t < L;
      const int64_t tok = b * L + t0 + t;
      s_B[t][n] = valid ? ld_act(Bm + tok * a.ld_B + n) : 0.0f;
      s_C[t][n] = valid ? ld_act(Cm + tok * a.ld_C + n) : 0.0f;
    }
    if (tid < TT) {
      const bool valid = t0 + tid < L;
      float dt = valid ? ld_act(DT + (b * L + t0 + tid) * a.ld_delta + hd) : 0.0f;
      dt += bias_h;
      if (a.softplus) dt = softplus_s(dt);
      s_dt[tid] = dt;
      s_a[tid] = expf(dt * A_h);
    }
    __syncthreads();
    for (int e = tid; e < TT * PPB; e += 256) {
      const int t = e / PPB, pp = e % PPB;
      const int64_t pg = (int64_t)blockIdx.x * PPB + pp;
      const bool valid = (t0 + t < L) && pg < P;
      const float xv = valid ? ld_act(X + (b * L + t0 + t) * a.ld_x + hd * P + pg) : 0.0f;
      s_ux[t][pp] = s_dt[t] * xv;
      s_dx[t][pp] = D_h * xv;
    }
    __syncthreads();
    const int tmax = (int)((L - t0) < TT ? (L - t0) : TT);
    for (int t = 0; t < tmax; ++t) {
      const float ab = s_a[t], ux = s_ux[t][pl];
      float yp = 0.0f;
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int n = qq * SPL + i;
        h[i] = __builtin_fmaf(ab, h[i], ux * s_B[t][n]);
        yp = __builtin_fmaf(s_C[t][n], h[i], yp);
      }
#pragma unroll
      for (int off = LPP / 2; off >= 1; off >>= 1) yp = yp + __shfl_xor(yp, off, 64);
      if (qq == 0) s_y[t][pl] = yp + s_dx[t][pl];
    }
    __syncthreads();
    for (int e = tid; e < TT * PPB; e += 256) {
      const int t = e / PPB, pp = e % PPB;
      const int64_t pg = (int64_t)blockIdx.x * PPB + pp;
      if ((t0 + t < L) && pg < P) {
        float yv = s_y[t][pp];
        if (a.gate) yv = yv * silu_gate(ld_act((const T*)a.gate + (b * L + t0 + t) * a.ld_gate + hd * P + pg));
        st_act(Y + (b * L + t0 + t) * a.ld_y + hd * P + pg, yv);
      }
    }
  }
  if (a.h_last && pv) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) a.h_last[((b * H + hd) * P + p) * NS + qq * SPL + i] = h[i];
  }
}

// ------------------------------------------------------------------------------------------
// Chunked evaluation on the matrix cores (the state-space duality of "Transformers are
// SSMs"): bf16 activations, headdim 64, d_state 64 or 128, chunks of Q = 64 steps.
// A block owns one (sequence, head) and walks its chunks in order, the P x N state in MFMA
// accumulators (8 waves: two per SIMD, so that one wave's dependent MFMAs, exponentials and
// LDS round trips overlap the other's).  With cs_t the inclusive cumulative sum of dt_s A inside a chunk and h_in the
// state entering it, for t in the chunk
//   y_t = sum_{s <= t} (C_t . B_s) exp(cs_t - cs_s) dt_s x_s  +  exp(cs_t) C_t h_in^T  +  D x_t
//   h_out = exp(cs_end) h_in + sum_s exp(cs_end - cs_s) dt_s x_s B_s^T
// which is the recurrence h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t, y_t = C_t h_t + D x_t
// regrouped.  Per chunk (wave w owning chunk rows 16 (w mod 4) .. + 15 and half the columns):
//   G = C B^T (bf16 x bf16, exact products, fp32 sums), then the masked, decayed M (fp32);
//   Y = M X and Z = C h_in^T; y = Y + exp(cs_t) Z + D x;
//   h = exp(cs_end) h + (w X)^T B, w_s = exp(cs_end - cs_s) dt_s.
// The fp32 operands (M, h_in, w X) enter the bf16 MFMAs as two bf16 terms (value = hi + lo,
// about 16 significant bits), the bf16 activations as they are.
// LDS holds the chunk's x, x^T, B, B^T, C (bf16), the waves' M rows and h_in (hi, lo).
namespace {
__device__ __forceinline__ uint16_t bf_bits(float f) { return f32_to_bf16(f); }
__device__ __forceinline__ float bf_val(uint16_t b) { return bf16_to_f32(b); }
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
// softplus(v) = log(1 + e^v) (the identity above 20) on the hardware exp2 / log2, with the
// rounding error c = (u - 1) - z of u = fl(1 + z) subtracted while u < 2 (where it dominates
// the error of log(u) relative to the small result); below e^v = 1e-4 the series
// e^v (1 - e^v / 2).
__device__ __forceinline__ float softplus_hw(float v) {
  const float z = exp_hw(v);
  const float u = 1.0f + z;
  const float c = u < 2.0f ? (u - 1.0f) - z : 0.0f;
  const float big = 0.69314718055994531f * __builtin_amdgcn_logf(u) - c;
  const float small = z * __builtin_fmaf(-0.5f, z, 1.0f);
  const float r = z < 1e-4f ? small : big;
  return v > 20.0f ? v : r;
}
}  // namespace

constexpr int kSsdQ = 64, kSsdP = 64;

// 8 waves, two per SIMD: wave w works on row tile rt = w mod 4 (chunk rows, or state rows p)
// and half hf = w / 4 of the tiles along the other dimension; every output tile is computed
// by one wave with the same MFMA sequence as with one wave per row tile.
template <int NS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_ssd_chunk(ScanArgs a) {
  constexpr int Q = kSsdQ, P = kSsdP;
  constexpr int XS = Q + 8;          // row stride (elements) of the [.][Q] arrays
  constexpr int NSP = NS + 8;        // row stride of the [.][NS] arrays
  constexpr int NTN = NS / 16;       // 16-wide n tiles
  constexpr int NTH = NTN / 2;       // n tiles of a wave's state share
  constexpr int KN = NS / 32;        // k steps over n
  __shared__ __align__(16) uint16_t sX[Q * XS];        // x  [t][p]
  __shared__ __align__(16) uint16_t sG[Q * XS];        // gate [t][p] (gated block)
  __shared__ __align__(16) uint16_t sXT[P * XS];       // x^T [p][s]
  __shared__ __align__(16) uint16_t sB[Q * NSP];       // B  [s][n]
  __shared__ __align__(16) uint16_t sBT[NS * XS];      // B^T [n][s]
  __shared__ __align__(16) uint16_t sC[Q * NSP];       // C  [t][n]
  __shared__ __align__(16) uint16_t sM[4][2][16 * XS]; // per wave: M rows (hi, lo) [t][s]
  __shared__ __align__(16) uint16_t sH[2][P * NSP];    // h_in (hi, lo) [p][n]
  __shared__ float s_dt[Q], s_cs[Q];
  __shared__ float s_w[Q], s_et[Q];  // exp(cs_end - cs_s) dt_s and exp(cs_t)

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = w & 3, hf = w >> 2;
  const int kq = lane >> 4, l16 = lane & 15;
  const int64_t L = a.L, H = a.H;
  const int64_t hd = blockIdx.x % H, b = blockIdx.x / H;
  const float A_h = a.A[hd];
  const float bias_h = a.delta_bias ? a.delta_bias[hd] : 0.0f;
  const float D_h = a.D ? a.D[hd] : 0.0f;
  const bf16_t* X = (const bf16_t*)a.x;
  const bf16_t* Bm = (const bf16_t*)a.Bm;
  const bf16_t* Cm = (const bf16_t*)a.Cm;
  const bf16_t* DT = (const bf16_t*)a.delta;
  bf16_t* Y = (bf16_t*)a.y;

  // state: lane holds h[p = 16 rt + 4 kq + r][n = 16 (NTH hf + jn) + l16]
  v4f h[NTH];
#pragma unroll
  for (int jn = 0; jn < NTH; ++jn)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = 16 * rt + 4 * kq + r, n = 16 * (NTH * hf + jn) + l16;
      h[jn][r] = a.h0 ? a.h0[((b * H + hd) * P + pp) * NS + n] : 0.0f;
    }
  auto write_h = [&]() {
#pragma unroll
    for (int jn = 0; jn < NTH; ++jn)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pp = 16 * rt + 4 * kq + r, n = 16 * (NTH * hf + jn) + l16;
        const uint16_t hi = bf_bits(h[jn][r]);
        sH[0][pp * NSP + n] = hi;
        sH[1][pp * NSP + n] = bf_bits(h[jn][r] - bf_val(hi));
      }
  };
  write_h();

  // chunk loads, 16-byte chunks with the step index fastest across the lanes (lane = step t,
  // chunk column q = wave + 8 i), so that the transposed LDS copies are written along rows
  constexpr int XC = Q * P / 8 / 512, BC = Q * NS / 8 / 512;
  v4i px[XC], pg[XC], pb[BC], pc[BC];
  float pdt = 0.0f;
  const bf16_t* G = (const bf16_t*)a.gate;
  auto load = [&](int64_t c0) {
    const bool ok = c0 + lane < L;
    const int64_t tok = b * L + c0 + lane;
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int q = w + 8 * i;
      px[i] = ok ? *(const v4i*)(X + tok * a.ld_x + hd * P + q * 8) : v4i{0, 0, 0, 0};
      if (G) pg[i] = ok ? *(const v4i*)(G + tok * a.ld_gate + hd * P + q * 8) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int q = w + 8 * i;
      pb[i] = ok ? *(const v4i*)(Bm + tok * a.ld_B + q * 8) : v4i{0, 0, 0, 0};
      pc[i] = ok ? *(const v4i*)(Cm + tok * a.ld_C + q * 8) : v4i{0, 0, 0, 0};
    }
    if (w == 0) pdt = ok ? bf16_to_f32(DT[tok * a.ld_delta + hd]) : 0.0f;
  };
  auto stage = [&](int64_t c0) {
    const int t = lane;
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int q = w + 8 * i;
      *(v4i*)(&sX[t * XS + q * 8]) = px[i];
      if (G) *(v4i*)(&sG[t * XS + q * 8]) = pg[i];
      const uint16_t* v = (const uint16_t*)&px[i];
#pragma unroll
      for (int u = 0; u < 8; ++u) sXT[(q * 8 + u) * XS + t] = v[u];
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int q = w + 8 * i;
      *(v4i*)(&sB[t * NSP + q * 8]) = pb[i];
      *(v4i*)(&sC[t * NSP + q * 8]) = pc[i];
      const uint16_t* v = (const uint16_t*)&pb[i];
#pragma unroll
      for (int u = 0; u < 8; ++u) sBT[(q * 8 + u) * XS + t] = v[u];
    }
    if (w == 0) {  // dt = softplus(delta + bias) (0 past the end), cs = inclusive cumsum of dt A
      float dt = 0.0f;
      if (c0 + lane < L) {
        dt = pdt + bias_h;
        if (a.softplus) dt = softplus_hw(dt);
      }
      float cs = dt * A_h;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(cs, d, 64);
        if (lane >= d) cs += o;
      }
      const float cend = __shfl(cs, 63, 64);
      s_dt[lane] = dt;
      s_cs[lane] = cs;
      s_w[lane] = exp_hw(cend - cs) * dt;
      s_et[lane] = exp_hw(cs);
    }
  };

  const int64_t nch = cdiv(L, Q);
  load(0);
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int64_t c0 = ch * Q;
    stage(c0);
    __syncthreads();
    if (ch + 1 < nch) load(c0 + Q);
    const float cs_end = s_cs[Q - 1];

    // G = C B^T for rows 16 rt .., s tiles j = 2 hf, 2 hf + 1 when j <= rt (the rest is
    // masked); then those columns of M into LDS
    {
      v4f g[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) g[jj] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
        const v8bf af = __builtin_bit_cast(v8bf, *(const v4i*)(&sC[(16 * rt + l16) * NSP + kk * 32 + kq * 8]));
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = 2 * hf + jj;
          if (j > rt) continue;
          const v8bf bfr = __builtin_bit_cast(v8bf, *(const v4i*)(&sB[(16 * j + l16) * NSP + kk * 32 + kq * 8]));
          g[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, g[jj], 0, 0, 0);
        }
      }
      // M[t][s] = G exp(cs_t - cs_s) dt_s for s <= t; lane holds t = 16 rt + 4 kq + r, s = 16 j + l16
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 2 * hf + jj;
          const int tl = 4 * kq + r, t = 16 * rt + tl, sidx = 16 * j + l16;
          float m = 0.0f;
          if (j <= rt && sidx <= t) m = g[jj][r] * (exp_hw(s_cs[t] - s_cs[sidx]) * s_dt[sidx]);
          const uint16_t hi = bf_bits(m);
          sM[rt][0][tl * XS + sidx] = hi;
          sM[rt][1][tl * XS + sidx] = bf_bits(m - bf_val(hi));
        }
    }
    __syncthreads();

    // Y = M X (s < 16 rt + 16) and Z = C h_in^T for p tiles jp = 2 hf, 2 hf + 1; lane holds
    // t = 16 rt + 4 kq + r, p = 16 jp + l16
    v4f yacc[2], zacc[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) { yacc[jj] = v4f{0.f, 0.f, 0.f, 0.f}; zacc[jj] = v4f{0.f, 0.f, 0.f, 0.f}; }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (kk * 32 > 16 * rt + 15) continue;
      const v8bf mh = __builtin_bit_cast(v8bf, *(const v4i*)(&sM[rt][0][l16 * XS + kk * 32 + kq * 8]));
      const v8bf ml = __builtin_bit_cast(v8bf, *(const v4i*)(&sM[rt][1][l16 * XS + kk * 32 + kq * 8]));
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int jp = 2 * hf + jj;
        const v8bf xf = __builtin_bit_cast(v8bf, *(const v4i*)(&sXT[(16 * jp + l16) * XS + kk * 32 + kq * 8]));
        yacc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mh, xf, yacc[jj], 0, 0, 0);
        yacc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ml, xf, yacc[jj], 0, 0, 0);
      }
    }
#pragma unroll
    for (int kk = 0; kk < KN; ++kk) {
      const v8bf cf = __builtin_bit_cast(v8bf, *(const v4i*)(&sC[(16 * rt + l16) * NSP + kk * 32 + kq * 8]));
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int jp = 2 * hf + jj;
        const int off = (16 * jp + l16) * NSP + kk * 32 + kq * 8;
        const v8bf hh = __builtin_bit_cast(v8bf, *(const v4i*)(&sH[0][off]));
        const v8bf hl = __builtin_bit_cast(v8bf, *(const v4i*)(&sH[1][off]));
        zacc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cf, hh, zacc[jj], 0, 0, 0);
        zacc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cf, hl, zacc[jj], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * rt + 4 * kq + r;
      if (c0 + t >= L) continue;
      const float et = s_et[t];
      bf16_t* yr = Y + (b * L + c0 + t) * a.ld_y + hd * P;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int jp = 2 * hf + jj;
        const int pp = 16 * jp + l16;
        float yv = yacc[jj][r] + et * zacc[jj][r] + D_h * bf_val(sX[t * XS + pp]);
        if (G) yv = yv * silu_gate(bf_val(sG[t * XS + pp]));
        yr[pp] = f32_to_bf16(yv);
      }
    }

    // state: h = exp(cs_end) h + (w X)^T B; A fragment: p = 16 rt + l16, s = 32 kk + 8 kq + u
    const float ed = exp_hw(cs_end);
#pragma unroll
    for (int jn = 0; jn < NTH; ++jn)
#pragma unroll
      for (int r = 0; r < 4; ++r) h[jn][r] *= ed;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint16_t* xr = &sXT[(16 * rt + l16) * XS + kk * 32 + kq * 8];
      uint16_t ahi[8], alo[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sidx = kk * 32 + kq * 8 + u;
        const float v = bf_val(xr[u]) * s_w[sidx];
        ahi[u] = bf_bits(v);
        alo[u] = bf_bits(v - bf_val(ahi[u]));
      }
      const v8bf ah = __builtin_bit_cast(v8bf, *(const v4i*)ahi);
      const v8bf al = __builtin_bit_cast(v8bf, *(const v4i*)alo);
#pragma unroll
      for (int jn = 0; jn < NTH; ++jn) {
        const int n0t = 16 * (NTH * hf + jn);
        const v8bf bfr = __builtin_bit_cast(v8bf, *(const v4i*)(&sBT[(n0t + l16) * XS + kk * 32 + kq * 8]));
        h[jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bfr, h[jn], 0, 0, 0);
        h[jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bfr, h[jn], 0, 0, 0);
      }
    }
    __syncthreads();
    write_h();
  }
  if (a.h_last) {
#pragma unroll
    for (int jn = 0; jn < NTH; ++jn)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pp = 16 * rt + 4 * kq + r, n = 16 * (NTH * hf + jn) + l16;
        a.h_last[((b * H + hd) * P + pp) * NS + n] = h[jn][r];
      }
  }
}

// The chunked kernel takes bf16 activations with headdim 64, d_state 64 or 128, and row
// strides and bases that allow 16-byte loads of x, B and C.
static bool ssd_chunk_ok(const ScanArgs& a) {
  auto al = [](const void* p) { return ((uintptr_t)p % 16) == 0; };
  return a.act_bf16 && a.P == kSsdP && (a.N == 64 || a.N == 128) && a.ld_x % 8 == 0 && a.ld_B % 8 == 0 &&
         a.ld_C % 8 == 0 && al(a.x) && al(a.Bm) && al(a.Cm) && (!a.gate || (a.ld_gate % 8 == 0 && al(a.gate)));
}

template <int NS, typename T>
static void launch_ssd_t(const ScanArgs& a, hipStream_t s) {
  constexpr int PPB = 256 / (NS / 8);
  const dim3 grid((unsigned)cdiv(a.P, PPB), (unsigned)a.H, (unsigned)a.batch), block(256);
  hipLaunchKernelGGL((k_scan_ssd_rec<NS, T>), grid, block, 0, s, a);
}

template <typename T>
static hipError_t launch_ssd_n(const ScanArgs& a, hipStream_t s) {
  switch (a.N) {
    case 16: launch_ssd_t<16, T>(a, s); break;
    case 32: launch_ssd_t<32, T>(a, s); break;
    case 64: launch_ssd_t<64, T>(a, s); break;
    case 128: launch_ssd_t<128, T>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t scan_ssd_workspace(const ScanArgs&) { return 0; }

hipError_t launch_scan_ssd(const ScanArgs& a, void*, size_t, hipStream_t s) {
  if (a.batch == 0 || a.L == 0) return hipSuccess;
  if (ssd_chunk_ok(a)) {
    const dim3 grid((unsigned)(a.batch * a.H)), block(512);
    if (a.N == 128) hipLaunchKernelGGL((k_ssd_chunk<128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_ssd_chunk<64>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  return a.act_bf16 ? launch_ssd_n<bf16_t>(a, s) : launch_ssd_n<float>(a, s);
}

}  // namespace ssm
