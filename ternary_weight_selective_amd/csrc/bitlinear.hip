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
constexpr int kA16MaxGroups = 64;  // scale groups per row the large A16 tile stages in LDS

template <typename Tout> struct Vec4;
template <> struct Vec4<float> { typedef float4 type; };
template <> struct Vec4<bf16_t> { typedef uint2 type; };

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

// ------------------------------------------------------------------------------------------
// Large-tile A8 contraction, one scale per tensor: the MFMA-bound shapes (k > 1024, e.g. the
// Mamba-2 projections (8192, 4416, 2048) and (8192, 2048, 4096)).
//
// Block tile 256 tokens x BN outputs and 4 waves, each owning 128 tokens x BN / 2 outputs as
// 8 x BN / 32 MFMA 16x16x64 tiles with int32 accumulators, so that every operand fragment read
// from LDS feeds 8 (weights) or BN / 32 (activations) MFMAs.  BN = 256 and 192 run one wave
// per SIMD (accumulators in the AGPRs); BN = 128 fits two blocks per compute unit (registers
// and LDS ring halved), so that one block's epilogue runs under the other's MFMAs.
// Operands go from global memory straight into a ring of ST LDS stages (ST - 1 k steps in
// flight); the weights stay 2-bit in LDS and each wave unpacks its own fragments (about 11
// vector instructions per 16 weights, hidden under the MFMAs).  W is the A operand (rows =
// outputs) and the activations the B operand, so a lane ends with 4 consecutive outputs of
// one token and stores them as one vector.
//
// Tile order: blocks are dealt to the 8 XCDs round-robin, so block b works on tile
// (b mod 8) * ceil(T / 8) + b / 8: each XCD takes a contiguous run of tiles (outputs
// fastest) and its L2 serves the activation rows of few token tiles.
constexpr int kBigStages = 4;  // LDS stages of k_gemm_i8_big (ST - 1 k steps in flight)

template <typename Tout, int BN, bool DBG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BN == 128 ? 2 : 1, BN == 128 ? 2 : 1))) void k_gemm_i8_big(GemmArgs a) {
  constexpr int BMT = 256, BKT = 64, ST = kBigStages;
  constexpr int WN = BN / 2, NT = WN / 16, MT = 8;
  constexpr int ABYTES = BMT * BKT, WWORDS = BN * 4;
  constexpr int AL = BMT / 16 / 4;      // 16-row activation loads per wave and stage
  constexpr int WL = WWORDS / 64 / 4;   // 64-word weight loads per wave and stage
  constexpr int L = AL + WL;            // loads per wave and stage
  // one LDS array for both operands (with two the compiler makes every LDS read wait for
  // all loads in flight)
  __shared__ __align__(16) int8_t smem[ST * (ABYTES + WWORDS * 4)];
  int8_t* const s_a = smem;
  uint32_t* const s_w = (uint32_t*)(smem + ST * ABYTES);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int kq = lane >> 4, l16 = lane & 15;
  const int64_t nb = cdiv(a.N, BN), T = cdiv(a.M, BMT) * nb;
  const int64_t chunk = cdiv(T, 8);
  const int64_t li = blockIdx.x / 8, t = (blockIdx.x % 8) * chunk + li;
  if (li >= chunk || t >= T) return;
  const int64_t m0 = (t / nb) * BMT, n0 = (t % nb) * BN;
  const int nk = (int)(a.Kp / BKT);
  // activation scales of the lane's rows, loaded now for the epilogue
  float amx[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int64_t m = m0 + wm * 128 + i * 16 + l16;
    amx[i] = a.absmax[m < a.M ? m : a.M - 1];
  }
  // Operands go from global memory straight into LDS (each lane's 16 or 4 bytes land at
  // lane * size past the wave's LDS base), ST - 1 steps ahead of the MFMAs.  Rows past the
  // end are clamped to the last row (their results are never stored) and weight words past a
  // row's end to its last word (they meet the zero padding of the activations), so every wave
  // issues the same L loads per step and the wait for the oldest step is a constant count.
  // Activation rows are stored as four 16-byte chunks in the order q ^ ((row / 2) mod 4).
  const int8_t* ag[AL];
#pragma unroll
  for (int c = 0; c < AL; ++c) {
    const int r = wave * (BMT / 4) + c * 16 + (lane >> 2);
    const int64_t gm = m0 + r < a.M ? m0 + r : a.M - 1;
    ag[c] = (const int8_t*)a.A + gm * a.lda + (((lane & 3) ^ ((lane >> 3) & 3)) << 4);
  }
  const uint32_t* wg[WL];
#pragma unroll
  for (int c = 0; c < WL; ++c) {
    const int e = (wave * WL + c) * 64 + lane;
    const int64_t gn = n0 + (e >> 2) < a.N ? n0 + (e >> 2) : a.N - 1;
    wg[c] = a.W + gn * a.w_row_words;
  }
  const int wq = lane & 3;
  const int64_t wlast = a.w_row_words - 1;
  auto issue = [&](int ks, int8_t* __restrict__ da, uint32_t* __restrict__ dw) {
    const int k = ks < nk ? ks : nk - 1;
#pragma unroll
    for (int c = 0; c < AL; ++c)
      __builtin_amdgcn_global_load_lds((const void*)(ag[c] + (int64_t)k * BKT),
                                       (__attribute__((address_space(3))) void*)(da + (wave * (BMT / 4) + c * 16) * BKT),
                                       16, 0, 0);
    const int64_t kw = (int64_t)k * 4 + wq;
#pragma unroll
    for (int c = 0; c < WL; ++c)
      __builtin_amdgcn_global_load_lds((const void*)(wg[c] + (kw < wlast ? kw : wlast)),
                                       (__attribute__((address_space(3))) void*)(dw + (wave * WL + c) * 64),
                                       4, 0, 0);
  };
  v4i acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  const int aoff = (wm * 128 + l16) * BKT + ((kq ^ ((l16 >> 1) & 3)) << 4);
  const int woff = (wn * WN + l16) * 4 + kq;
  // The prologue fills stages 0 .. ST - 2 and waits for them; from then on iteration ks issues
  // the loads of k step ks + ST - 1 and contracts step ks.  The loads and the LDS reads of one
  // iteration go through separate restrict-qualified slot pointers (they never touch the same
  // slot), which lets the reads start without waiting for the loads in flight.
#pragma unroll
  for (int st = 0; st < ST - 1; ++st) issue(st, s_a + st * ABYTES, s_w + st * WWORDS);
  vm_wait<0>();
  auto iter = [&](int ks, const int8_t* __restrict__ ra, const uint32_t* __restrict__ rw,
                  int8_t* __restrict__ da, uint32_t* __restrict__ dw) {
    issue(ks + ST - 1, da, dw);
    uint32_t wpk[NT];
    v4i wf[NT], bfr[MT];
#pragma unroll
    for (int j = 0; j < NT; ++j) wpk[j] = rw[woff + j * 64];
#pragma unroll
    for (int i = 0; i < MT; ++i) bfr[i] = *(const v4i*)(ra + aoff + i * 16 * BKT);
#pragma unroll
    for (int j = 0; j < NT; ++j) wf[j] = unpack16_i8(wpk[j]);
    if constexpr (BN == 256) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[j], bfr[i], acc[i][j], 0, 0, 0);
  };
  // this wave's loads of step ks are done once at most (ST - 2) * L of its loads are in flight;
  // the barrier makes every wave's loads of step ks visible and retires step ks - 1's reads of
  // the slot about to be refilled.  (The two loop forms differ only in how the register
  // allocator treats them: each keeps its accumulators in place, without copies.)
  auto step = [&](int ks) {
    vm_wait<(ST - 2) * L>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int rs = ks % ST, ws = (ks + ST - 1) % ST;
    iter(ks, s_a + rs * ABYTES, s_w + rs * WWORDS, s_a + ws * ABYTES, s_w + ws * WWORDS);
  };
  if constexpr (BN == 256) {
    for (int ks = 0; ks < nk; ++ks) step(ks);
  } else {
    int ks = 0;
    do step(ks); while (++ks < nk);
  }

  // epilogue: lane holds token l16 of each token tile and outputs 4 kq .. 4 kq + 3 of each
  // output tile.  Every global load of a row (its activation scale, bias, residual) is issued
  // before the row's first use, so the row waits for memory once.
  const double sw = (double)a.w_scale[0];
  const int vb = (int)sizeof(typename Vec4<Tout>::type);
  const bool vec_ok = (a.ldy % 4 == 0) && (((uintptr_t)a.y) % vb == 0) &&
                      (!a.bias || ((uintptr_t)a.bias) % 16 == 0) &&
                      (!a.residual || (a.ld_res % 4 == 0 && ((uintptr_t)a.residual) % vb == 0));
  double deq[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) deq[i] = (double)fmaxf(amx[i], 1e-5f) / 127.0;
  if (vec_ok && n0 + BN <= a.N) {
    float4 bb[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
      bb[j] = a.bias ? *(const float4*)(a.bias + n0 + wn * WN + j * 16 + kq * 4) : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int64_t m = m0 + wm * 128 + i * 16 + l16;
      if (m >= a.M) continue;
      typename Vec4<Tout>::type res[NT];
      if (a.residual) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
          res[j] = *(const typename Vec4<Tout>::type*)((const Tout*)a.residual + m * a.ld_res + n0 + wn * WN + j * 16 + kq * 4);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int64_t n = n0 + wn * WN + j * 16 + kq * 4;
        double y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) y[q] = (sw * (double)acc[i][j][q]) * deq[i];
        if (a.bias) { y[0] += bb[j].x; y[1] += bb[j].y; y[2] += bb[j].z; y[3] += bb[j].w; }
        if (a.residual) {
          const Tout* rv = (const Tout*)&res[j];
#pragma unroll
          for (int q = 0; q < 4; ++q) y[q] += (double)ld_act(rv + q);
        }
        Tout o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) st_act(&o[q], (float)y[q]);
        *(typename Vec4<Tout>::type*)((Tout*)a.y + m * a.ldy + n) = *(const typename Vec4<Tout>::type*)o;
        if (DBG)
#pragma unroll
          for (int q = 0; q < 4; ++q) a.dbg_acc[m * a.N + n + q] = acc[i][j][q];
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int64_t m = m0 + wm * 128 + i * 16 + l16;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t n = n0 + wn * WN + j * 16 + kq * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (n + q >= a.N) continue;
        store_out<Tout>(a, m, n + q, (sw * (double)acc[i][j][q]) * deq[i]);
        if (DBG) a.dbg_acc[m * a.N + n + q] = acc[i][j][q];
      }
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
// Row-block A8 BitLinear for k <= 1024 (the HBM-bound projections), one scale per tensor.
//
// A persistent block of 8 waves walks over blocks of BR = 16 token rows (row block
// blockIdx.x, then + gridDim.x, ...), in two roles:
//   producers (waves 0-3) load x two row blocks ahead, normalise and quantise 4 rows each
//     (a wave per row: the fixed-order norm) into one of two LDS code buffers, and stage the
//     residual rows there too;
//   consumers (waves 4-7) contract the codes against W with int8 MFMA 16x16x64 and write y
//     with the fp64 epilogue.
// One barrier per row block hands a buffer over; it orders LDS only, so the producers' loads
// in flight and the consumers' stores in flight never wait for each other, and HBM sees
// loads and stores of different row blocks at the same time.  x is read once, y written once.
//
// Producer scalar tail: the lane-partial sums and the absmax of a row are reduced across the
// wave; the per-row scalar work (the correctly rounded divisions, the square root, the fp64
// dequantisation factor) is done once for the wave's 4 rows, lane j taking row j mod 4, and
// read back with readlane.
//
// Consumer c owns a contiguous run of 16-column tiles of W.  Their packed words sit in
// registers, loaded once when the run fits in one round of up to TPR tiles (every projection
// of the TriSSM and TernarySSM shapes but the widest), else round by round.  W is the MFMA's
// A operand (rows = output columns), the int8 codes its B operand, so each lane ends with 4
// consecutive outputs of one token row and stores them as one vector.  The 16-wide k chunks
// are assigned to (k-step, lane quarter) so that a lane's KPL packed words are consecutive in
// memory (one vector load per tile); A and B use the same assignment, so the int32 sums are
// unchanged.
namespace {


// Block barrier that orders LDS accesses only (outstanding global loads and stores of the
// waves are not waited for).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
}  // namespace

constexpr int kRowsBR = 16;       // token rows per row block of k_bl_rows

// RES: a residual of at most kRowsResN columns, staged through registers and LDS.
template <typename Tin, typename Tout, int KPL, bool RES, bool DBG>
__global__ __launch_bounds__(512) void k_bl_rows(GemmArgs g, RowArgs r) {
  constexpr int BR = kRowsBR;
  constexpr int RPW = BR / 4;                 // rows per producer wave
  constexpr int KMAX = 64 * KPL;
  constexpr int QS = KMAX + 16;               // LDS row stride of the codes (bytes)
  constexpr int TPR = (32 / KPL) < 8 ? (32 / KPL) : 8;  // column tiles per weight round
  constexpr bool PF2 = KPL <= 8;              // producers keep two row blocks of x in flight
  constexpr int RN = RES ? kRowsResN / 64 : 1;  // residual elements per lane per row
  __shared__ __align__(16) int8_t s_q[2][BR * QS];
  __shared__ double s_deq[2][BR];
  __shared__ __align__(16) float s_res[RES ? 2 * BR * kRowsResN : 1];  // staged residual rows
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nrb = cdiv(g.M, BR);
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int niter = b < nrb ? (int)((nrb - 1 - b) / G + 1) : 0;
  const int K = (int)g.K;
  const int N = (int)g.N;

  if (wave < 4) {
    // ---------------- producer ----------------
    const Tin* X = (const Tin*)r.x;
    const Tout* RS = (const Tout*)g.residual;
    const bool kfull = K == KMAX;
    float gn[KPL];  // gain, 1 when absent (an exact multiplication)
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int k = lane + 64 * i;
      gn[i] = (r.gain && k < K) ? r.gain[k] : 1.0f;
    }
    const int64_t last = b + (int64_t)(niter - 1) * G;  // a row block loaded again past the end
    // x (and the residual) of the wave's rows of row block it; rows past M and columns past
    // K read a valid element and are zeroed when used
    auto load_x = [&](int it, float (&v)[RPW][KPL], float (&res)[RPW][RN]) {
      int64_t rb = b + (int64_t)it * G;
      rb = rb < last ? rb : last;
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        int64_t row = rb * BR + wave * RPW + rr;
        row = row < g.M ? row : g.M - 1;
        const Tin* xr = X + row * r.ldx;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          int k = lane + 64 * i;
          if (!kfull) k = k < K ? k : K - 1;
          v[rr][i] = ld_act(xr + k);
        }
        if (RES) {
          const Tout* rp = RS + row * g.ld_res;
#pragma unroll
          for (int j = 0; j < RN; ++j) {
            int n = lane + 64 * j;
            n = n < N ? n : N - 1;
            res[rr][j] = ld_act(rp + n);
          }
        }
      }
    };
    auto produce = [&](int it, float (&v)[RPW][KPL], const float (&res)[RPW][RN]) {
      const int buf = it & 1;
      const int64_t m0 = (b + (int64_t)it * G) * BR;
      int8_t* sq = s_q[buf];
      if (RES) {  // residual rows of this row block into LDS (fp32 holds every Tout exactly)
        float* sr = s_res + buf * BR * kRowsResN;
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
          for (int j = 0; j < RN; ++j) sr[(wave * RPW + rr) * kRowsResN + lane + 64 * j] = res[rr][j];
      }
      float ss[RPW];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const bool rv = m0 + wave * RPW + rr < g.M;
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          v[rr][i] = (rv && (kfull || lane + 64 * i < K)) ? v[rr][i] : 0.0f;
          s = __builtin_fmaf(v[rr][i], v[rr][i], s);
        }
        ss[rr] = wave_sum_butterfly(s);
      }
      float sel = ss[0];
#pragma unroll
      for (int rr = 1; rr < RPW; ++rr) sel = (lane % RPW) == rr ? ss[rr] : sel;
      const float rs_l = __fdiv_rn(1.0f, sqrt_rn(__fdiv_rn(sel, (float)K) + r.eps));
      float mx[RPW];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const float rs = readlane_f(rs_l, rr);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const float t = (v[rr][i] * rs) * gn[i];
          v[rr][i] = t;
          m = fmaxf(m, fabsf(t));
        }
        mx[rr] = wave_absmax(m);
      }
      float msel = mx[0];
#pragma unroll
      for (int rr = 1; rr < RPW; ++rr) msel = (lane % RPW) == rr ? mx[rr] : msel;
      const float mf = fmaxf(msel, 1e-5f);
      const float sigma_l = __fdiv_rn(127.0f, mf);
      if (lane < RPW) {
        const int lr = wave * RPW + lane;
        s_deq[buf][lr] = (double)mf / 127.0;
        if (DBG && r.dbg_absmax && m0 + lr < g.M) r.dbg_absmax[m0 + lr] = msel;
      }
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const int lr = wave * RPW + rr;
        const float sigma = readlane_f(sigma_l, rr);
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const int k = lane + 64 * i;
          float q = rintf(v[rr][i] * sigma);
          q = fminf(fmaxf(q, -128.0f), 127.0f);
          sq[lr * QS + k] = (int8_t)(int)q;
          if (DBG && r.dbg_xq && m0 + lr < g.M && k < K) r.dbg_xq[(m0 + lr) * K + k] = (int8_t)(int)q;
        }
      }
    };
    float va[RPW][KPL], vb[RPW][KPL], ra[RPW][RN], rb_[RPW][RN];
    if (niter > 0) load_x(0, va, ra);
    if (PF2) {
      if (niter > 1) load_x(1, vb, rb_);
      for (int it = 0; it < niter; it += 2) {
        produce(it, va, ra);
        lds_barrier();
        load_x(it + 2, va, ra);
        if (it + 1 >= niter) break;
        produce(it + 1, vb, rb_);
        lds_barrier();
        load_x(it + 3, vb, rb_);
      }
    } else {
      for (int it = 0; it < niter; ++it) {
        produce(it, va, ra);
        lds_barrier();
        load_x(it + 1, va, ra);
      }
    }
  } else {
    // ---------------- consumer ----------------
    const int cw = wave - 4;
    const int nct = (int)cdiv(g.N, 16);
    const int tpw = (nct + 3) / 4;
    const int ct0 = cw * tpw;
    const int ct1 = (ct0 + tpw < nct) ? ct0 + tpw : nct;
    const bool one_round = ct1 - ct0 <= TPR;
    const double sw = (double)g.w_scale[0];
    const int vb_ = (int)sizeof(typename Vec4<Tout>::type);
    const bool vec_ok = (g.ldy % 4 == 0) && (((uintptr_t)g.y) % vb_ == 0) &&
                        (!g.bias || ((uintptr_t)g.bias) % 16 == 0);
    const int kq = lane >> 4, lm = lane & 15;
    const bool wvec = (KPL % 4 == 0) && (g.w_row_words == 4 * KPL) && (((uintptr_t)g.W) % 16 == 0);
    uint32_t wv[TPR][KPL];
    // packed words of tiles c .. c + TPR - 1: lane (n, kq) holds words kq KPL .. kq KPL + KPL - 1
    // of row n (k chunk kq KPL + ks at k-step ks)
    auto load_round = [&](int c) {
#pragma unroll
      for (int j = 0; j < TPR; ++j) {
        const int64_t n = (int64_t)(c + j) * 16 + lm;
        const bool ok = (c + j < ct1) && n < g.N;
        const uint32_t* wr = g.W + n * g.w_row_words + kq * KPL;
        if (KPL % 4 == 0 && wvec) {
#pragma unroll
          for (int v4 = 0; v4 < KPL / 4; ++v4) {
            const uint4 u = ok ? ((const uint4*)wr)[v4] : make_uint4(0u, 0u, 0u, 0u);
            wv[j][4 * v4] = u.x; wv[j][4 * v4 + 1] = u.y; wv[j][4 * v4 + 2] = u.z; wv[j][4 * v4 + 3] = u.w;
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < KPL; ++ks) {
            const int64_t kw = (int64_t)kq * KPL + ks;
            wv[j][ks] = (ok && kw < g.w_row_words) ? wr[ks] : 0u;
          }
        }
      }
    };
    if (ct0 < ct1) load_round(ct0);
    for (int it = 0; it < niter; ++it) {
      lds_barrier();
      const int buf = it & 1;
      const int64_t m0 = (b + (int64_t)it * G) * BR;
      const int64_t m = m0 + lm;
      const double deq = s_deq[buf][lm];
      const float* sr = s_res + (RES ? buf * BR * kRowsResN + lm * kRowsResN : 0);
      v4i bq[KPL];  // codes of row lm, k chunk kq KPL + ks
#pragma unroll
      for (int ks = 0; ks < KPL; ++ks) bq[ks] = *(const v4i*)(s_q[buf] + lm * QS + (kq * KPL + ks) * 16);
      for (int c = ct0; c < ct1; c += TPR) {
        if (!one_round && !(c == ct0 && it == 0)) load_round(c);
        v4i acc[TPR];
#pragma unroll
        for (int j = 0; j < TPR; ++j) {
          acc[j] = v4i{0, 0, 0, 0};
          if (c + j < ct1) {
#pragma unroll
            for (int ks = 0; ks < KPL; ++ks)
              acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16_i8(wv[j][ks]), bq[ks], acc[j], 0, 0, 0);
          }
        }
#pragma unroll
        for (int j = 0; j < TPR; ++j) {
          const int64_t n = (int64_t)(c + j) * 16 + kq * 4;
          if (c + j < ct1 && m < g.M && n < g.N) {
            double y[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) y[q] = (sw * (double)acc[j][q]) * deq;
            if (vec_ok && n + 3 < g.N) {
              if (g.bias) {
                const float4 bb = *(const float4*)(g.bias + n);
                y[0] += bb.x; y[1] += bb.y; y[2] += bb.z; y[3] += bb.w;
              }
              if (RES) {
                const float4 rr4 = *(const float4*)(sr + n);
                y[0] += rr4.x; y[1] += rr4.y; y[2] += rr4.z; y[3] += rr4.w;
              }
              Tout o[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) st_act(&o[q], (float)y[q]);
              *(typename Vec4<Tout>::type*)((Tout*)g.y + m * g.ldy + n) = *(const typename Vec4<Tout>::type*)o;
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                if (n + q >= g.N) continue;
                double v = y[q];
                if (g.bias) v += (double)g.bias[n + q];
                if (RES) v += (double)sr[n + q];
                st_act((Tout*)g.y + m * g.ldy + n + q, (float)v);
              }
            }
            if (DBG && g.dbg_acc)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (n + q < g.N) g.dbg_acc[m * g.N + n + q] = acc[j][q];
          }
        }
      }
    }
  }
}

// A16 large tile (one bf16 activation term): x̂ x ternary weights on bf16 MFMA 16x16x32.
// Block tile 256 tokens x 128 outputs, 8 waves (two per SIMD) with 64 x 64 tiles of 4 x 4 MFMA
// blocks; k steps of 64 double-buffered through LDS; each packed weight word is unpacked to
// bf16 +-1 / 0 once per block.  The MFMA accumulators hold one scale group's partial sums; at
// the group's end each is folded into an fp32 total with that group's scale (one FMA per
// output, VALU work that overlaps the matrix cores), the block's scales staged in LDS.  With
// one scale per tensor the accumulators run over all of k and are scaled once.
template <typename Tout>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_a16_big(GemmArgs a) {
  constexpr int NTH = 512;
  constexpr int BMT = 256, BNT = 128, BKT = 64, AS = BKT + 8;  // AS: LDS row stride in bf16 elements
  constexpr int WM = 64, WN = 64, NT = WN / 16, MT = WM / 16;
  constexpr int CPT = BMT * BKT * 2 / 16 / NTH;  // 16-byte activation chunks per thread and k step
  constexpr int WPT = BNT * (BKT / 16) / NTH;    // packed weight words per thread and k step
  constexpr int NGP = kA16MaxGroups + 1;         // LDS row stride of the scales
  __shared__ __align__(16) bf16_t s_a[2][BMT * AS];
  __shared__ __align__(16) bf16_t s_w[2][BNT * AS];
  __shared__ float s_sc[BNT * NGP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 waves
  const int kq = lane >> 4, l16 = lane & 15;
  const int64_t nb = cdiv(a.N, BNT), T = cdiv(a.M, BMT) * nb;
  const int64_t chunk = cdiv(T, 8);
  const int64_t li = blockIdx.x / 8, t = (blockIdx.x % 8) * chunk + li;  // an XCD walks consecutive tiles
  if (li >= chunk || t >= T) return;
  const int64_t m0 = (t / nb) * BMT, n0 = (t % nb) * BNT;
  const bf16_t* A = (const bf16_t*)a.A;
  const int ng = a.group ? (int)(a.K / a.group) : 1;
  const int gsteps = a.group ? (int)(a.group / BKT) : (int)(a.Kp / BKT);  // k steps per scale group
  for (int e = tid; e < BNT * ng; e += NTH) {
    const int nl = e / ng, g = e % ng;
    const int64_t n = n0 + nl;
    s_sc[nl * NGP + g] = n < a.N ? (a.group ? a.w_scale[n * ng + g] : a.w_scale[0]) : 0.0f;
  }
  v4i pa[2][CPT];  // two k steps in flight in registers
  uint32_t pw[2][WPT];
  auto load = [&](int64_t k0, v4i (&pa)[CPT], uint32_t (&pw)[WPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int e = tid + NTH * c, r = e >> 3, q = e & 7;
      const int64_t gm = m0 + r;
      pa[c] = gm < a.M ? *(const v4i*)(A + gm * a.lda + k0 + q * 8) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < WPT; ++c) {
      const int e = tid + NTH * c, r = e >> 2, q = e & 3;
      const int64_t gn = n0 + r, kw = k0 / 16 + q;
      pw[c] = (gn < a.N && kw < a.w_row_words) ? a.W[gn * a.w_row_words + kw] : 0u;
    }
  };
  auto store = [&](int buf, const v4i (&pa)[CPT], const uint32_t (&pw)[WPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int e = tid + NTH * c, r = e >> 3, q = e & 7;
      *(v4i*)(&s_a[buf][r * AS + q * 8]) = pa[c];
    }
#pragma unroll
    for (int c = 0; c < WPT; ++c) {
      const int e = tid + NTH * c, r = e >> 2, q = e & 3;
      v4i o0, o1;
      unpack16_bf16(pw[c], o0, o1);
      v4i* dst = (v4i*)(&s_w[buf][r * AS + q * 16]);
      dst[0] = o0;
      dst[1] = o1;
    }
  };
  v4f acc[MT][NT];
  float tot[MT][NT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[i][j][q] = 0.0f;
    }
  const int nk = (int)(a.Kp / BKT);
  // step ks: tile ks is in LDS buffer ks & 1 and tile ks + 1 in registers pa[(ks + 1) & 1];
  // the step requests tile ks + 2 into pa[ks & 1], contracts tile ks, then moves tile ks + 1
  // into the other buffer (read at step ks - 1, which ended with a barrier): each load has
  // two steps of work to arrive
  load(0, pa[0], pw[0]);
  if (nk > 1) load(BKT, pa[1], pw[1]);
  store(0, pa[0], pw[0]);
  __syncthreads();
  auto step = [&](int ks, v4i (&pn)[CPT], uint32_t (&wn_)[WPT], const v4i (&pc)[CPT], const uint32_t (&wc)[WPT]) {
    const int buf = ks & 1;
    if (ks + 2 < nk) load((int64_t)(ks + 2) * BKT, pn, wn_);
    // fragments of both 32-deep halves of the k step: the second half's are read while the
    // first half's MFMAs run
    v8bf wf[2][NT], bfr[2][MT];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
        wf[h][j] = __builtin_bit_cast(v8bf, *(const v4i*)(&s_w[buf][(wn * WN + j * 16 + l16) * AS + h * 32 + kq * 8]));
#pragma unroll
      for (int i = 0; i < MT; ++i)
        bfr[h][i] = __builtin_bit_cast(v8bf, *(const v4i*)(&s_a[buf][(wm * WM + i * 16 + l16) * AS + h * 32 + kq * 8]));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[h][j], bfr[h][i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NT + MT, 0);  // first half's LDS reads
#pragma unroll
    for (int r = 0; r < NT + MT; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // two MFMAs of the first half
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // one read of the second half
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MT * NT, 0);  // second half's MFMAs
    if ((ks + 1) % gsteps == 0) {  // end of a scale group: fold its partials with the group's scale
      const int g = a.group ? ks / gsteps : 0;
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sc = s_sc[(wn * WN + j * 16 + kq * 4 + q) * NGP + g];
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            tot[i][j][q] = __builtin_fmaf(acc[i][j][q], sc, tot[i][j][q]);
            acc[i][j][q] = 0.0f;
          }
        }
    }
    if (ks + 1 < nk) store(buf ^ 1, pc, wc);
    __syncthreads();
  };
  for (int ks = 0; ks < nk; ks += 2) {
    step(ks, pa[0], pw[0], pa[1], pw[1]);
    if (ks + 1 < nk) step(ks + 1, pa[1], pw[1], pa[0], pw[0]);
  }

  // epilogue: lane holds token l16 of each token tile and outputs 4 kq .. 4 kq + 3 of each
  // output tile
  const int vb = (int)sizeof(typename Vec4<Tout>::type);
  const bool vec_ok = (a.ldy % 4 == 0) && (((uintptr_t)a.y) % vb == 0) &&
                      (!a.bias || ((uintptr_t)a.bias) % 16 == 0);
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int64_t m = m0 + wm * WM + i * 16 + l16;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t n = n0 + wn * WN + j * 16 + kq * 4;
      if (n >= a.N) continue;
      float y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = tot[i][j][q];
      if (vec_ok && n + 3 < a.N) {
        if (a.bias) {
          const float4 bb = *(const float4*)(a.bias + n);
          y[0] += bb.x; y[1] += bb.y; y[2] += bb.z; y[3] += bb.w;
        }
        if (a.residual) {
          const Tout* rp = (const Tout*)a.residual + m * a.ld_res + n;
#pragma unroll
          for (int q = 0; q < 4; ++q) y[q] += ld_act(rp + q);
        }
        Tout o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) st_act(&o[q], y[q]);
        *(typename Vec4<Tout>::type*)((Tout*)a.y + m * a.ldy + n) = *(const typename Vec4<Tout>::type*)o;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (n + q < a.N) store_out<Tout>(a, m, n + q, y[q]);
      }
    }
  }
}

// Output-tile width of k_gemm_i8_big.  256 and 192 run one block per compute unit (one wave
// per SIMD), 128 two (its accumulators fit in half the registers and its LDS ring in half the
// LDS), so one block's epilogue overlaps the other's k loop.  The width with the fewest
// rounds of tiles over the chip, weighted by the tile width, is taken; two co-resident 128-wide
// tiles take 1.7x the time of one (measured at the Mamba-2 out_proj shape, (8192, 2048, 4096):
// 86 -> 78 us against 256-wide tiles).  When the 128-wide tiles fit one round (two per compute
// unit) they are taken outright: at k <= 1024 a 192-wide tile per compute unit runs latency-bound
// (TernarySSM out_proj (16384, 512, 1024): 44.7 us with 128-wide tiles, 78.8 with 192).
static int big_bn(int64_t M, int64_t N) {
  const int64_t mt = cdiv(M, 256);
  if (mt * cdiv(N, 128) <= 512) return 128;
  auto cost = [&](int bn, int per_cu, double f) {
    const int64_t T = mt * cdiv(N, bn);
    return (double)cdiv(T, 256 * per_cu) * bn * f;
  };
  const double c128 = cost(128, 2, 1.7), c192 = cost(192, 1, 1.0), c256 = cost(256, 1, 1.0);
  if (c128 < c192 && c128 < c256) return 128;
  return c192 < c256 ? 192 : 256;
}

template <typename Tout, bool DBG>
static void launch_big(const GemmArgs& a, hipStream_t s) {
  const int bn = big_bn(a.M, a.N);
  const int64_t T = cdiv(a.M, 256) * cdiv(a.N, bn);
  const dim3 grid((unsigned)(8 * cdiv(T, 8))), block(256);
  if (bn == 128) hipLaunchKernelGGL((k_gemm_i8_big<Tout, 128, DBG>), grid, block, 0, s, a);
  else if (bn == 192) hipLaunchKernelGGL((k_gemm_i8_big<Tout, 192, DBG>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_gemm_i8_big<Tout, 256, DBG>), grid, block, 0, s, a);
}

hipError_t launch_gemm_i8(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (a.Kp < 64 || a.Kp % 64 != 0) return hipErrorInvalidValue;
  if (a.group == 0) {
    const bool d = a.dbg_acc != nullptr;
    if (a.y_bf16) { if (d) launch_big<bf16_t, true>(a, s); else launch_big<bf16_t, false>(a, s); }
    else { if (d) launch_big<float, true>(a, s); else launch_big<float, false>(a, s); }
    return hipGetLastError();
  }
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
  if (!a.A2 && (a.group == 0 || (a.group % 64 == 0 && a.K / a.group <= kA16MaxGroups))) {
    const int64_t T = cdiv(a.M, 256) * cdiv(a.N, 128);
    const dim3 grid((unsigned)(8 * cdiv(T, 8))), block(512);
    if (a.y_bf16) hipLaunchKernelGGL((k_gemm_a16_big<bf16_t>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm_a16_big<float>), grid, block, 0, s, a);
    return hipGetLastError();
  }
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
// Persistent grid: as many blocks of 8 waves as fit on every compute unit at once (two where
// registers and LDS allow, which doubles the loads in flight), never more than row blocks.
// Results do not depend on it (every row is computed the same way by whichever block owns it).
template <typename K>
static int64_t rows_grid(K kernel) {
  int dev = 0, ncu = 256, occ = 1;
  if (hipGetDevice(&dev) == hipSuccess) {
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1) ncu = 256;
  }
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 512, 0) != hipSuccess || occ < 1) occ = 1;
  return (int64_t)ncu * (occ < 2 ? occ : 2);
}

template <typename Tin, typename Tout, int KPL>
static void launch_rows_t(const GemmArgs& g, const RowArgs& r, hipStream_t s) {
  const int64_t nrb = cdiv(g.M, kRowsBR);
  const bool dbg = g.dbg_acc || r.dbg_xq || r.dbg_absmax;
#define SSM_ROWS(RES, DBG)                                                                  \
  do {                                                                                      \
    static const int64_t cap = rows_grid(k_bl_rows<Tin, Tout, KPL, RES, DBG>);              \
    const dim3 grid((unsigned)(nrb < cap ? nrb : cap)), block(512);                         \
    hipLaunchKernelGGL((k_bl_rows<Tin, Tout, KPL, RES, DBG>), grid, block, 0, s, g, r);     \
  } while (0)
  if (g.residual) { if (dbg) SSM_ROWS(true, true); else SSM_ROWS(true, false); }
  else { if (dbg) SSM_ROWS(false, true); else SSM_ROWS(false, false); }
#undef SSM_ROWS
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
