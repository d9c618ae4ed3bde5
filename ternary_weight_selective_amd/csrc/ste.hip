// Training side of BitLinear: the backward pass with straight-through estimators and one step
// of quantisation-aware training with learnable scales (TriSSM README: BitLinear trained with
// straight-through estimators; Ternary Mamba abstract: grouped QAT with learnable quantisation
// scales and the zero ratio they can collapse).  The estimator passes gradients through both
// roundings: dx̂ = dy W̃ with W̃ = s q (the ternary codes times their scale), dW = dy^T x̃ with
// x̃ the forward's int8 codes dequantised, then the RMSNorm backward.  With one scale per tensor
// dx comes from k_ste_dx (the codes on the matrix cores, the RMSNorm backward in its epilogue);
// with grouped scales (or k > 1024) dx̂ is a dense fp32 GEMM (sgemm_nn) followed by k_rms_bwd.  dW
// comes from k_ste_dw (the activation codes on the matrix cores, split over token chunks).  The
// other kernels here rebuild the forward's codes and the transposed weight codes, and take the
// scale gradient.
#include <algorithm>

#include "launch.hpp"
#include "mixer_bwd.hpp"

namespace ssm {

// One wave per token row: the forward's RMSNorm and absmax int8 codes in the forward's own
// arithmetic order (so the codes are the forward's), kept as the codes q [M, K] and the row's
// step max(m, 1e-5) / 127 (x̃ = q step), and the row's RMSNorm scale r.  Columns past K load
// column K - 1 and are zeroed (no lane-dependent condition around the loads).
template <int KPL, typename Tin>
__global__ __launch_bounds__(256) void k_ste_act(const Tin* __restrict__ x, int64_t M, int K, int64_t ldx,
                                                 const float* __restrict__ gain, float eps, int8_t* __restrict__ xq,
                                                 float* __restrict__ st, float* __restrict__ rs) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // uniform per wave
  const Tin* xr = x + row * ldx;
  float v[KPL], gv[KPL];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    const int kc = k < K ? k : K - 1;
    const float xv = ld_act(xr + kc);
    gv[i] = gain ? gain[kc] : 1.0f;
    v[i] = k < K ? xv : 0.0f;
    s = __builtin_fmaf(v[i], v[i], s);
  }
  s = wave_sum_butterfly(s);
  const float ms = __fdiv_rn(s, (float)K);
  const float r = __fdiv_rn(1.0f, sqrt_rn(ms + eps));
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    float t = v[i] * r;
    if (gain) t = (k < K) ? t * gv[i] : 0.0f;
    v[i] = t;
    m = fmaxf(m, fabsf(t));
  }
  m = wave_absmax(m);
  const float mf = fmaxf(m, 1e-5f);
  const float sigma = __fdiv_rn(127.0f, mf);
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    float q = rintf(v[i] * sigma);
    q = fminf(fmaxf(q, -128.0f), 127.0f);
    if (k < K) xq[row * K + k] = (int8_t)(int)q;
  }
  if (lane == 0) {
    rs[row] = r;
    st[row] = (float)((double)mf / 127.0);
  }
}

// dW = dy^T x̃ over one token chunk per blockIdx.z, on the bf16 matrix cores.  x̃ = q st (int8
// codes, exact in bf16, times the row's step), so dW[n][k] = sum_m (dy[m][n] st_m) q[m][k]; the
// first factor is rounded once to fp32 and enters as three truncated bf16 terms (as in k_ste_dx),
// so the products carry fp32 accuracy.  A block owns 64 x 16 KT outputs, its 4 waves 16 rows (n)
// x 16 KT columns (k) each (KT tiles).  Per step of 32 tokens the block stages both operands in LDS
// transposed ([n][m] and [k][m]), so that each MFMA fragment (8 consecutive tokens) is one 16-byte
// read; a step's tokens are loaded into registers two steps ahead, and the LDS is
// double-buffered (one barrier per step).  Tokens past the chunk and rows / columns
// past N / K enter as zeros.  The chunk's partial dW goes to part[chunk][n][k] (fp32); the
// chunks are added in order afterwards.
constexpr int kDwB = 64;   // outputs per block in n
constexpr int kDwLS = 40;  // LDS row stride (bf16) of the transposed tiles: 32 tokens + padding
template <int KT>
__global__ __launch_bounds__(256) void k_ste_dw(const float* __restrict__ dy, int64_t ld_dy,
                                                const int8_t* __restrict__ xq, const float* __restrict__ st, int64_t M,
                                                int N, int K, int64_t chunk, float* __restrict__ part) {
  constexpr int KW = 16 * KT;   // outputs per block in k
  constexpr int TPC = 256 / KW; // threads per staged code column
  constexpr int TQ = 32 / TPC;  // tokens per thread of the code staging (8 or 16)
  __shared__ __align__(16) bf16_t s_a[2][3][kDwB * kDwLS];
  __shared__ __align__(16) bf16_t s_b[2][KW * kDwLS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ng = lane >> 4, nc = lane & 15;
  const int n0 = blockIdx.x * kDwB, k0 = blockIdx.y * KW;
  const int64_t mb = (int64_t)blockIdx.z * chunk;
  const int64_t me = mb + chunk < M ? mb + chunk : M;
  // staging roles: dy column c (an n), tokens 8 mg .. 8 mg + 7; code column cq (a k), tokens
  // TQ qg .. TQ qg + TQ - 1
  const int c = tid & 63, mg = tid >> 6;
  const int cq = tid % KW, qg = tid / KW;
  const bool nv = n0 + c < N, kv = k0 + cq < K;
  const int ncl = nv ? n0 + c : N - 1, kcl = kv ? k0 + cq : K - 1;
  // two register sets of staged tokens: a step's tokens are requested two steps before they are
  // written to LDS, so that a whole step's products and barrier cover their latency
  struct Regs {
    float a[8], s[8];
    int8_t q[TQ];
  } r0, r1;
  // 32-bit offsets from the chunk's first token (uniform bases)
  const float* dyb = dy + mb * ld_dy;
  const int8_t* xqb = xq + mb * K;
  const float* stb = st + mb;
  const int last = (int)(me - 1 - mb);
  auto load = [&](int64_t m0, Regs& r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = (int)(m0 - mb) + 8 * mg + i;
      const int mc = m < last ? m : last;
      r.a[i] = dyb[mc * (int)ld_dy + ncl];
      r.s[i] = stb[mc];
    }
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
      const int m = (int)(m0 - mb) + TQ * qg + i;
      r.q[i] = xqb[(m < last ? m : last) * K + kcl];
    }
  };
  auto stage = [&](int64_t m0, const Regs& r, int buf) {
    v4i hi, mid, lo;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t hb[2], mbb[2], lb[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * p + e;
        const bool mv = m0 + 8 * mg + i < me;
        const float v = (mv && nv) ? r.a[i] * r.s[i] : 0.0f;
        hb[e] = __float_as_uint(v) & 0xFFFF0000u;
        const float r1 = v - __uint_as_float(hb[e]);
        mbb[e] = __float_as_uint(r1) & 0xFFFF0000u;
        const float r2 = r1 - __uint_as_float(mbb[e]);
        lb[e] = __float_as_uint(r2) & 0xFFFF0000u;
      }
      hi[p] = (int)((hb[0] >> 16) | hb[1]);
      mid[p] = (int)((mbb[0] >> 16) | mbb[1]);
      lo[p] = (int)((lb[0] >> 16) | lb[1]);
    }
    const int off = c * kDwLS + 8 * mg;
    *(v4i*)(&s_a[buf][0][off]) = lo;
    *(v4i*)(&s_a[buf][1][off]) = mid;
    *(v4i*)(&s_a[buf][2][off]) = hi;
#pragma unroll
    for (int g = 0; g < TQ / 8; ++g) {
      v4i qb;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t qq[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int i = 8 * g + 2 * p + e;
          const bool mv = m0 + TQ * qg + i < me;
          qq[e] = __float_as_uint((mv && kv) ? (float)r.q[i] : 0.0f) & 0xFFFF0000u;  // exact in bf16
        }
        qb[p] = (int)((qq[0] >> 16) | qq[1]);
      }
      *(v4i*)(&s_b[buf][cq * kDwLS + TQ * qg + 8 * g]) = qb;
    }
  };
  v4f acc[KT];
#pragma unroll
  for (int j = 0; j < KT; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  auto products = [&](int buf) {
    const int aoff = (16 * w + nc) * kDwLS + 8 * ng;
    const v8bf al = __builtin_bit_cast(v8bf, *(const v4i*)(&s_a[buf][0][aoff]));
    const v8bf am = __builtin_bit_cast(v8bf, *(const v4i*)(&s_a[buf][1][aoff]));
    const v8bf ah = __builtin_bit_cast(v8bf, *(const v4i*)(&s_a[buf][2][aoff]));
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const v8bf b = __builtin_bit_cast(v8bf, *(const v4i*)(&s_b[buf][(16 * j + nc) * kDwLS + 8 * ng]));
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, b, acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc[j], 0, 0, 0);
    }
  };
  if (mb < me) {
    load(mb, r0);
    if (mb + 32 < me) load(mb + 32, r1);
    stage(mb, r0, 0);
  }
  // step m0 reads buffer 0, step m0 + 32 buffer 1; a buffer is rewritten after the next barrier
  for (int64_t m0 = mb; m0 < me; m0 += 64) {
    __syncthreads();
    if (m0 + 64 < me) load(m0 + 64, r0);
    products(0);
    if (m0 + 32 >= me) break;
    stage(m0 + 32, r1, 1);
    __syncthreads();
    if (m0 + 96 < me) load(m0 + 96, r1);
    products(1);
    if (m0 + 64 < me) stage(m0 + 64, r0, 0);
  }
  float* pc = part + (int64_t)blockIdx.z * N * K;
#pragma unroll
  for (int j = 0; j < KT; ++j) {
    const int k = k0 + 16 * j + nc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 16 * w + 4 * ng + i;
      if (n < N && k < K) pc[(int64_t)n * K + k] = acc[j][i];
    }
  }
}

// W̃[n, k] = s(n, k / group) q[n, k] (one scale when group == 0); thread per packed word.
__global__ __launch_bounds__(256) void k_ste_weights(const uint32_t* __restrict__ W, int64_t N, int64_t K,
                                                     int64_t row_words, const float* __restrict__ scale,
                                                     int64_t group, float* __restrict__ wt) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= N * row_words) return;
  const int64_t n = t / row_words, w = t % row_words;
  const v4i c = unpack16_i8(W[t]);
  const int8_t* cb = (const int8_t*)&c;
  const int64_t ng = group ? K / group : 1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t k = w * 16 + i;
    if (k < K) {
      const float sc = group ? scale[n * ng + k / group] : scale[0];
      wt[n * K + k] = sc * (float)cb[i];
    }
  }
}

// The ternary codes widened to bf16 (exactly -1, 0 or +1) in the order k_ste_dx reads them as
// its B operand: for inner step s (32 values of n), column tile t (16 values of k) and lane l,
// 8 consecutive elements hold q[n][k] for n = 32 s + 8 (l >> 4) + 0..7, k = 16 t + (l & 15), so
// each fragment load of a wave is 1 KB contiguous.  Zero for n >= N or k >= K (the padding of
// the tiles).  Thread per element.  A packed word holds weights 16w .. 16w + 15; weight i of a
// word sits in bits 2 (i / 4) + 8 (i % 4) (01 = +1, 11 = -1, 00 = 0).
__global__ __launch_bounds__(256) void k_ste_codes_t(const uint32_t* __restrict__ W, int64_t N, int64_t K,
                                                     int64_t row_words, int64_t np, int64_t kp,
                                                     bf16_t* __restrict__ qt) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= kp * np) return;
  const int64_t kt = kp / 16, l = (e >> 3) & 63, rest = e >> 9;
  const int64_t n = 32 * (rest / kt) + 8 * (l >> 4) + (e & 7), k = 16 * (rest % kt) + (l & 15);
  bf16_t v = 0;
  if (n < N && k < K) {
    const int i = (int)(k % 16);
    const uint32_t f = (W[n * row_words + k / 16] >> (2 * (i >> 2) + 8 * (i & 3))) & 3u;
    v = f == 1u ? (bf16_t)0x3F80u : (f == 3u ? (bf16_t)0xBF80u : (bf16_t)0u);
  }
  qt[e] = v;
}

// dx for one scale per tensor, on the matrix cores: dx̂ = s (dy q) with bf16 MFMA 16x16x32, then
// the RMSNorm backward in the epilogue, so dx̂ never reaches memory:
//   dx = r g dx̂ - x (r^3 / K) sum_j g_j dx̂_j x_j.
// The codes are exact in bf16.  dy enters as three bf16 terms, each the truncation of what the
// previous ones leave (hi = trunc(dy), mid = trunc(dy - hi), lo = trunc(dy - hi - mid); every
// difference is exact), which add up to dy within 2^-24 of its magnitude; their products are
// accumulated in fp32, smallest first.
// A block of 4 waves owns RW row tiles of 16 token rows; the 4 / RW waves of a row tile split the
// ceil(K / 16) column tiles (16 columns each), TW per wave, so that narrow outputs spread over
// rows rather than leave waves idle.  MFMA operands: A = dy (lane: row lane & 15, inner
// elements 8 (lane >> 4) .. + 7 of the step), B = qt (lane: column lane & 15, the same inner
// elements; one contiguous 1 KB load per tile in k_ste_codes_t's order), C: lane holds rows
// 4 (lane >> 4) + 0..3 of column lane & 15.  Each row's dot
// product is summed over the wave's tiles in order, over the 16 lanes of its column group
// (xor 1, 2, 4, 8), then over the row tile's waves in order through LDS.
template <int RW, int TW, typename Tin>
__global__ __launch_bounds__(256) void k_ste_dx(const Tin* __restrict__ x, int64_t ldx, const float* __restrict__ dy,
                                                int64_t ld_dy, int vec, const bf16_t* __restrict__ qt, int64_t np,
                                                int64_t M, int K, int N, const float* __restrict__ gain,
                                                const float* __restrict__ scale, const float* __restrict__ rs,
                                                const float* add, int64_t ld_add, float* dx, int64_t ld_dx) {
  constexpr int CWV = 4 / RW;  // waves per row tile
  __shared__ float s_dot[4][16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = w / CWV, cw = w % CWV;
  const int64_t mb = (int64_t)blockIdx.x * 16 * RW;  // the block's first row (< M)
  const int64_t m0 = mb + 16 * rt;                    // this wave's row tile (may start past M)
  const int kt = (K + 15) / 16;
  const int t0 = cw * TW;
  const int ng = lane >> 4, nc = lane & 15;
  int64_t arow = m0 + nc;
  const bool arv = arow < M;
  arow = arv ? arow : M - 1;
  const float* dyr = dy + arow * ld_dy + 8 * ng;
  v4f acc[TW];
#pragma unroll
  for (int j = 0; j < TW; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // the operands of step n0: dy values (raw) and the codes of the wave's tiles; the next step's
  // are requested before this step's products.  (Requesting dy two steps ahead costs a wave per
  // SIMD of occupancy and measured no faster.)
  float a[8];
  v4i bq[TW];
  auto load_step = [&](int n0) {
    if (vec && n0 + 32 <= N) {
      const v4f u0 = *(const v4f*)(dyr + n0), u1 = *(const v4f*)(dyr + n0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = u0[i];
        a[4 + i] = u1[i];
      }
    } else {  // the ragged last step: clamped addresses; values past N are zeroed when used
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int n = n0 + 8 * ng + i;
        a[i] = dyr[(n < N ? n : N - 1) - 8 * ng];
      }
    }
    // tiles past the last read the last tile's codes (in bounds); their columns are never stored
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int tj = t0 + j < kt ? t0 + j : kt - 1;
      bq[j] = *(const v4i*)(qt + ((((n0 >> 5) * kt + tj) * 64 + lane) * 8));
    }
  };
  load_step(0);
#pragma unroll 1
  for (int n0 = 0; n0 < N; n0 += 32) {
    float ac[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ac[i] = (arv && n0 + 8 * ng + i < N) ? a[i] : 0.0f;
    v8bf bc[TW];
#pragma unroll
    for (int j = 0; j < TW; ++j) bc[j] = __builtin_bit_cast(v8bf, bq[j]);
    if (n0 + 32 < N) load_step(n0 + 32);
    v4i hi, mid, lo;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t hb[2], mb[2], lb[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float v = ac[2 * p + e];
        hb[e] = __float_as_uint(v) & 0xFFFF0000u;
        const float r1 = v - __uint_as_float(hb[e]);
        mb[e] = __float_as_uint(r1) & 0xFFFF0000u;
        const float r2 = r1 - __uint_as_float(mb[e]);
        lb[e] = __float_as_uint(r2) & 0xFFFF0000u;
      }
      hi[p] = (int)((hb[0] >> 16) | hb[1]);
      mid[p] = (int)((mb[0] >> 16) | mb[1]);
      lo[p] = (int)((lb[0] >> 16) | lb[1]);
    }
    const v8bf ah = __builtin_bit_cast(v8bf, hi), am = __builtin_bit_cast(v8bf, mid),
               al = __builtin_bit_cast(v8bf, lo);
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bc[j], acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bc[j], acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bc[j], acc[j], 0, 0, 0);
    }
  }

  // epilogue: g dx̂ and x at the lane's positions (rows 4 (lane >> 4) + 0..3 of the row tile,
  // column lane & 15 of each tile); 32-bit offsets from the block's first row (uniform); rows past
  // M read row M - 1 and columns past K column K - 1 (neither is stored).  (Requesting x before
  // the contraction costs a wave per SIMD of occupancy and measured slower.)
  const Tin* xb = x + mb * ldx;
  const int rows = (int)(M - m0 < 16 ? M - m0 : 16);  // valid rows of the tile (<= 0: none)
  const int last = (int)(M - 1 - mb);                  // the last valid row, from the block's first
  const float sc = scale[0];
  float rq[4];  // the rows' RMSNorm scales, requested together with x
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rb = 16 * rt + 4 * ng + q;
    rq[q] = rs[mb + (rb < last ? rb : last)];
  }
  float xv[TW][4];
  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    const int k = (t0 + j) * 16 + nc;
    const bool kv = k < K;  // also false for tiles past the last
    const int kcl = kv ? k : K - 1;
    const float gv = gain ? gain[kcl] : 1.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lr = 4 * ng + q;
      const int rb = 16 * rt + lr;
      const float xr = ld_act(xb + ((rb < last ? rb : last) * (int)ldx + kcl));
      const bool ok = kv && lr < rows;
      xv[j][q] = ok ? xr : 0.0f;
      const float gd = ok ? gv * (sc * acc[j][q]) : 0.0f;
      acc[j][q] = gd;
      part[q] = __builtin_fmaf(gd, xv[j][q], part[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) part[q] = part[q] + __shfl_xor(part[q], d, 64);
  }
  if (nc == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) s_dot[w][4 * ng + q] = part[q];
  }
  // the accumulated input, from clamped positions with no lane-dependent condition (so that the
  // loads are in flight together, across the barrier)
  float av[TW][4];
  if (add) {
    const float* ab = add + mb * ld_add;
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int k = (t0 + j) * 16 + nc;
      const int kcl = k < K ? k : K - 1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rb = 16 * rt + 4 * ng + q;
        av[j][q] = ab[(rb < last ? rb : last) * (int)ld_add + kcl];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < TW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) av[j][q] = 0.0f;
  }
  __syncthreads();
  float* db = dx + mb * ld_dx;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lr = 4 * ng + q;
    const int rb = 16 * rt + lr;
    float dot = s_dot[rt * CWV][lr];
#pragma unroll
    for (int c = 1; c < CWV; ++c) dot = dot + s_dot[rt * CWV + c][lr];
    const float r = rq[q];
    const float c = r * r * r / (float)K * dot;
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int k = (t0 + j) * 16 + nc;
      if (k < K && lr < rows) db[rb * (int)ld_dx + k] = av[j][q] + (r * acc[j][q] - xv[j][q] * c);
    }
  }
}

// RMSNorm backward, one wave per row: dx = r g dx̂ - x (r^3 / K) sum_j g_j dx̂_j x_j.
template <int KPL, typename Tin>
__global__ __launch_bounds__(256) void k_rms_bwd(const Tin* __restrict__ x, int64_t M, int K, int64_t ldx,
                                                 const float* __restrict__ gain, const float* __restrict__ rs,
                                                 const float* __restrict__ dxh, const float* add, int64_t ld_add,
                                                 float* dx, int64_t ld_dx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  float xv[KPL], gd[KPL];
  float dot = 0.0f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    const bool ok = k < K;
    xv[i] = ok ? ld_act(x + row * ldx + k) : 0.0f;
    gd[i] = ok ? (gain ? gain[k] : 1.0f) * dxh[row * K + k] : 0.0f;
    dot = __builtin_fmaf(gd[i], xv[i], dot);
  }
  dot = wave_sum_butterfly(dot);
  const float r = rs[row];
  const float c = r * r * r / (float)K * dot;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    if (k < K) {
      const float v = r * gd[i] - xv[i] * c;
      dx[row * ld_dx + k] = add ? add[row * ld_add + k] + v : v;
    }
  }
}

// Scale gradient per (row, group) (or per row for one scale, summed afterwards): one wave per
// segment, ds = sum dW (q - v) where |v| <= 1, dW q elsewhere, v = W / s.
__global__ __launch_bounds__(256) void k_scale_grad(const float* __restrict__ dw, const float* __restrict__ wl,
                                                    const float* __restrict__ scale, int64_t N, int64_t K,
                                                    int64_t group, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t G = group ? group : K, ng = K / G;
  if (seg >= N * ng) return;
  const int64_t n = seg / ng, g = seg % ng;
  const float sc = group ? scale[n * ng + g] : scale[0];
  float acc = 0.0f;
  for (int64_t j = lane; j < G; j += 64) {
    const int64_t k = g * G + j;
    const float w = wl[n * K + k];
    const float v = w / sc;
    const float q = fminf(fmaxf(rintf(v), -1.0f), 1.0f);
    const float f = fabsf(v) <= 1.0f ? q - v : q;
    acc = __builtin_fmaf(dw[n * K + k], f, acc);
  }
  acc = wave_sum_butterfly(acc);
  if (lane == 0) out[seg] = acc;
}

// Sum of n per-row partials (one scale per tensor), one wave in a fixed order: lane j adds
// rows j, j + 64, ... in fp64, then the wave's butterfly.
__global__ void k_sum_rows(const float* __restrict__ part, int64_t n, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  double s = 0.0;
  for (int64_t i = lane; i < n; i += 64) s += (double)part[i];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  if (lane == 0) out[0] = (float)s;
}

// dW = sum of the token chunks' partial products, in chunk order; the loads of eight chunks are
// issued together (clamped to the last chunk, whose extra values are not added).
__global__ __launch_bounds__(256) void k_sum_chunks(const float* __restrict__ part, int64_t count, int64_t chunks,
                                                    float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float s = 0.0f;
  for (int64_t c0 = 0; c0 < chunks; c0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = part[(c0 + j < chunks ? c0 + j : chunks - 1) * count + i];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < chunks) s = (c0 + j == 0) ? v[0] : s + v[j];
  }
  dw[i] = s;
}

namespace {
// Token chunks of k_ste_dw: enough blocks for the chip (about 512 output tiles x chunks;
// more chunks cost more in partial sums than they gain), chunks of at least 128 tokens (a
// multiple of 32), partials within 64 MB, and short enough that the kernel's 32-bit offsets
// within a chunk (tokens x max(ld_dy, K)) cannot overflow.
// column tiles per wave of k_ste_dw: 8 (128 outputs per block in k), 4 for narrow K
int dw_kt(int64_t K) { return K <= 64 ? 4 : 8; }

int64_t dw_chunk_len(int64_t M, int64_t N, int64_t K, int64_t ld_dy) {
  const int64_t tiles = cdiv(N, kDwB) * cdiv(K, 16 * dw_kt(K));
  int64_t c = std::min<int64_t>(64, std::max<int64_t>(1, cdiv(512, tiles)));
  c = std::min(c, std::max<int64_t>(1, M / 128));
  while (c > 1 && c * N * K * 4 > (64ll << 20)) --c;
  const int64_t row = std::max(ld_dy, K);
  while (c < M && round_up(cdiv(M, c), 32) * row >= (1ll << 31) - row) ++c;  // ends: 33 row < 2^31 (checked)
  return round_up(cdiv(M, c), 32);
}
}  // namespace

// W -= lr dW; s -= lr_s ds (fp32 fused multiply-adds).
__global__ __launch_bounds__(256) void k_sgd(float* __restrict__ w, const float* __restrict__ dw, int64_t n,
                                             float lr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) w[i] = __builtin_fmaf(-lr, dw[i], w[i]);
}

namespace {
template <typename Tin>
hipError_t launch_act_k(const SteArgs& a, int8_t* xq, float* st, float* rs, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(a.M, 4)), block(256);
  const Tin* x = (const Tin*)a.x;
#define SSM_ACT(KK) hipLaunchKernelGGL((k_ste_act<KK, Tin>), grid, block, 0, s, x, a.M, (int)a.K, a.ldx, a.gain, a.eps, xq, st, rs)
  if (a.K <= 64) SSM_ACT(1);
  else if (a.K <= 128) SSM_ACT(2);
  else if (a.K <= 256) SSM_ACT(4);
  else if (a.K <= 512) SSM_ACT(8);
  else if (a.K <= 1024) SSM_ACT(16);
  else if (a.K <= 2048) SSM_ACT(32);
  else if (a.K <= 4096) SSM_ACT(64);
  else return hipErrorInvalidValue;
#undef SSM_ACT
  return hipGetLastError();
}

// k_ste_dx serves one scale per tensor and K <= 1024 (the accumulators of 16 tiles per wave).
bool ste_dx_fused(const SteArgs& a) { return a.group == 0 && a.K <= 1024; }

// (row tiles per block, column tiles per wave) by the number of column tiles: at least 8 tiles
// per wave where K allows, so that each step's dy conversion feeds 24 products
template <int RW, int TW, typename Tin>
hipError_t launch_dx_rt(const SteArgs& a, const bf16_t* qt, int64_t np, const float* rs, int vec, const float* add,
                        int64_t ld_add, hipStream_t s) {
  hipLaunchKernelGGL((k_ste_dx<RW, TW, Tin>), dim3((unsigned)cdiv(a.M, 16 * RW)), dim3(256), 0, s, (const Tin*)a.x,
                     a.ldx, a.dy, a.ld_dy, vec, qt, np, a.M, (int)a.K, (int)a.N, a.gain, a.scale, rs, add, ld_add,
                     a.dx, a.ld_dx);
  return hipGetLastError();
}

template <typename Tin>
hipError_t launch_dx_k(const SteArgs& a, const bf16_t* qt, int64_t np, const float* rs, const float* add,
                       int64_t ld_add, hipStream_t s) {
  const int vec = (a.ld_dy % 4 == 0) && ((uintptr_t)a.dy % 16 == 0);
  const int64_t kt = cdiv(a.K, 16);
  if (kt <= 1) return launch_dx_rt<4, 1, Tin>(a, qt, np, rs, vec, add, ld_add, s);
  if (kt <= 2) return launch_dx_rt<4, 2, Tin>(a, qt, np, rs, vec, add, ld_add, s);
  if (kt <= 4) return launch_dx_rt<4, 4, Tin>(a, qt, np, rs, vec, add, ld_add, s);
  if (kt <= 8) return launch_dx_rt<2, 4, Tin>(a, qt, np, rs, vec, add, ld_add, s);
  if (kt <= 16) return launch_dx_rt<2, 8, Tin>(a, qt, np, rs, vec, add, ld_add, s);
  if (kt <= 32) return launch_dx_rt<1, 8, Tin>(a, qt, np, rs, vec, add, ld_add, s);
  if (kt <= 64) return launch_dx_rt<1, 16, Tin>(a, qt, np, rs, vec, add, ld_add, s);
  return hipErrorInvalidValue;
}

template <typename Tin>
hipError_t launch_rms_bwd_k(const SteArgs& a, const float* rs, const float* dxh, const float* add, int64_t ld_add,
                            hipStream_t s) {
  const dim3 grid((unsigned)cdiv(a.M, 4)), block(256);
  const Tin* x = (const Tin*)a.x;
#define SSM_RB(KK) hipLaunchKernelGGL((k_rms_bwd<KK, Tin>), grid, block, 0, s, x, a.M, (int)a.K, a.ldx, a.gain, rs, dxh, add, ld_add, a.dx, a.ld_dx)
  if (a.K <= 64) SSM_RB(1);
  else if (a.K <= 128) SSM_RB(2);
  else if (a.K <= 256) SSM_RB(4);
  else if (a.K <= 512) SSM_RB(8);
  else if (a.K <= 1024) SSM_RB(16);
  else if (a.K <= 2048) SSM_RB(32);
  else if (a.K <= 4096) SSM_RB(64);
  else return hipErrorInvalidValue;
#undef SSM_RB
  return hipGetLastError();
}
}  // namespace

size_t ste_workspace(const SteArgs& a) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t b = al((size_t)a.M * a.K);           // the activation codes q (x̃ = q st)
  b += al((size_t)a.M * 4);                   // st
  b += al((size_t)a.M * 4);                   // r
  // W̃ (fp32 [N, K]), or for k_ste_dx the transposed bf16 codes (padded [K16, N32])
  b += al(std::max((size_t)a.N * a.K * 4, (size_t)round_up(a.K, 16) * round_up(a.N, 32) * 2));
  b += al((size_t)a.M * a.K * 4);             // dx̂
  b += al((size_t)a.N * 4);                   // per-row scale partials
  const int64_t ch = a.M > 0 ? cdiv(a.M, dw_chunk_len(a.M, a.N, a.K, a.ld_dy)) : 1;
  if (ch > 1) b += al((size_t)ch * a.N * a.K * 4);  // dW partials per token chunk
  return b;
}

hipError_t launch_ste_bwd(const SteArgs& a, void* ws, hipStream_t s) { return launch_ste_bwd_add(a, nullptr, 0, ws, s); }

hipError_t launch_ste_bwd_add(const SteArgs& a, const float* add, int64_t ld_add, void* ws, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  char* p = (char*)ws;
  int8_t* xq = (int8_t*)p; p += al((size_t)a.M * a.K);
  float* st = (float*)p; p += al((size_t)a.M * 4);
  float* rs = (float*)p; p += al((size_t)a.M * 4);
  float* wt = (float*)p;
  p += al(std::max((size_t)a.N * a.K * 4, (size_t)round_up(a.K, 16) * round_up(a.N, 32) * 2));
  float* dxh = (float*)p; p += al((size_t)a.M * a.K * 4);
  float* part = (float*)p; p += al((size_t)a.N * 4);
  float* dwp = (float*)p;
  hipError_t e = a.x_bf16 ? launch_act_k<bf16_t>(a, xq, st, rs, s) : launch_act_k<float>(a, xq, st, rs, s);
  if (e != hipSuccess) return e;
  if (ste_dx_fused(a)) {
    const int64_t np = round_up(a.N, 32), kp = round_up(a.K, 16);
    bf16_t* qt = (bf16_t*)wt;
    hipLaunchKernelGGL(k_ste_codes_t, dim3((unsigned)cdiv(kp * np, 256)), dim3(256), 0, s, a.W, a.N, a.K,
                       a.w_row_words, np, kp, qt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = a.x_bf16 ? launch_dx_k<bf16_t>(a, qt, np, rs, add, ld_add, s) : launch_dx_k<float>(a, qt, np, rs, add, ld_add, s);
    if (e != hipSuccess) return e;
  } else {
    const int64_t words = a.N * a.w_row_words;
    hipLaunchKernelGGL(k_ste_weights, dim3((unsigned)cdiv(words, 256)), dim3(256), 0, s, a.W, a.N, a.K,
                       a.w_row_words, a.scale, a.group, wt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dx̂ [M, K] = dy [M, N] W̃ [N, K]
    e = sgemm_nn(a.M, a.K, a.N, a.dy, a.ld_dy, wt, a.K, dxh, a.K, s);
    if (e != hipSuccess) return e;
    e = a.x_bf16 ? launch_rms_bwd_k<bf16_t>(a, rs, dxh, add, ld_add, s)
                 : launch_rms_bwd_k<float>(a, rs, dxh, add, ld_add, s);
    if (e != hipSuccess) return e;
  }
  if (a.dw) {  // dW [N, K] = dy^T [N, M] x̃ [M, K], per token chunk, then the chunks in order
    const int64_t cl = dw_chunk_len(a.M, a.N, a.K, a.ld_dy), ch = cdiv(a.M, cl);
    const int kt = dw_kt(a.K);
    const dim3 grid((unsigned)cdiv(a.N, kDwB), (unsigned)cdiv(a.K, 16 * kt), (unsigned)ch);
    if (kt == 4)
      hipLaunchKernelGGL(k_ste_dw<4>, grid, dim3(256), 0, s, a.dy, a.ld_dy, xq, st, a.M, (int)a.N, (int)a.K, cl,
                         ch > 1 ? dwp : a.dw);
    else
      hipLaunchKernelGGL(k_ste_dw<8>, grid, dim3(256), 0, s, a.dy, a.ld_dy, xq, st, a.M, (int)a.N, (int)a.K, cl,
                         ch > 1 ? dwp : a.dw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ch > 1) {
      hipLaunchKernelGGL(k_sum_chunks, dim3((unsigned)cdiv(a.N * a.K, 256)), dim3(256), 0, s, dwp, a.N * a.K, ch,
                         a.dw);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (a.dscale) {
    const int64_t segs = a.group ? a.N * (a.K / a.group) : a.N;
    float* dst = a.group ? a.dscale : part;
    hipLaunchKernelGGL(k_scale_grad, dim3((unsigned)cdiv(segs, 4)), dim3(256), 0, s, a.dw, a.w_latent, a.scale, a.N,
                       a.K, a.group, dst);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!a.group) {
      hipLaunchKernelGGL(k_sum_rows, dim3(1), dim3(64), 0, s, part, a.N, a.dscale);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_sgd(float* w, const float* dw, int64_t n, float lr, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_sgd, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, w, dw, n, lr);
  return hipGetLastError();
}

}  // namespace ssm
