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
// SSMs"): bf16 activations, headdim 64, d_state 64 or 128, chunks of Q = 64 steps.  With cs_t
// the inclusive cumulative sum of dt_s A inside a chunk and h_in the state entering it, for t
// in the chunk
//   y_t   = sum_{s <= t} (C_t . B_s) exp(cs_t - cs_s) dt_s x_s + exp(cs_t) C_t h_in^T + D x_t
//   h_out = exp(cs_end) h_in + sum_s exp(cs_end - cs_s) dt_s x_s B_s^T
// which is the recurrence h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t, y_t = C_t h_t + D x_t
// regrouped.
//
// Work split.  Time is cut into S segments of whole chunks; a block owns 4 heads of one
// sequence and one segment, and walks the segment's chunks in order (8 waves: wave w takes head
// w / 2 and the state columns p of half w mod 2).  Segments run in parallel: pass 1 computes the
// end state of every segment but the last from a zero state (state update only), a combine
// composes them in order ((P, h_loc) o h = P h + h_loc, P = exp(A sum dt)), and pass 2 runs
// every segment from its true incoming state, writing y.
//
// Per chunk, everything is matrix products on 16 x 16 x 32 bf16 MFMAs in transposed form, so
// that no per-head product's result goes through LDS to become another's operand:
//   G^T = B C^T                       (A: B rows, B-operand: C rows; both staged row-major;
//                                       the same for every head: computed once per block and
//                                       shared through LDS)
//   M^T = G^T (.) exp(cs_t - cs_s) dt_s on s <= t, plus D on the diagonal (the D x term)
//   y^T = x^T M^T + exp(cs_t) (h C^T)  (x^T staged transposed; M^T and h straight from the
//                                       accumulators of G^T and of the state)
//   h^T = exp(cs_end) h^T + B^T (w x) with w_s = exp(cs_end - cs_s) dt_s
// An accumulator tile holds, per lane, 4 consecutive rows of one column; two such tiles give
// the 8 reduction slots a lane feeds to a 16 x 16 x 32 MFMA, in a permuted order of the
// reduction index that the other operand's lane reads in the same order (a sum over k does not
// depend on the order).  Precision: bf16 activations enter as they are; the fp32 operands of
// the readout (M^T and h, whose products only feed the bf16 output y) are rounded to bf16,
// nearest even; the state update's fp32 operand w x enters as two bf16 terms, the truncated
// value and the truncated remainder (about 16 significant bits), so that the carried fp32 state
// keeps that accuracy.
namespace {
constexpr float kLog2e = 1.4426950408889634f;
// softplus(v) = log(1 + e^v) (the identity above 20) on the hardware exp2 / log2, with the
// rounding error c = (u - 1) - z of u = fl(1 + z) subtracted while u < 2 (where it dominates
// the error of log(u) relative to the small result); below e^v = 1e-4 the series
// e^v (1 - e^v / 2).
__device__ __forceinline__ float softplus_hw(float v) {
  const float z = __builtin_amdgcn_exp2f(v * kLog2e);
  const float u = 1.0f + z;
  const float c = u < 2.0f ? (u - 1.0f) - z : 0.0f;
  const float big = 0.69314718055994531f * __builtin_amdgcn_logf(u) - c;
  const float small = z * __builtin_fmaf(-0.5f, z, 1.0f);
  const float r = z < 1e-4f ? small : big;
  return v > 20.0f ? v : r;
}

constexpr int kSsdQ = 64, kSsdP = 64;
constexpr int kSsdHB = 4;           // heads per block
constexpr int kSsdXS = kSsdQ + 8;   // row stride (bf16) of [.][Q] arrays in LDS

struct SsdSeg {
  int S;              // segments per sequence
  int seg_ch;         // chunks per segment
  float* hloc;        // [B, S-1, H, P, N]: pass 1 end states, then (combine) incoming states
  float* sdec;        // [B, S-1, H]: log2 of each segment's decay, sum of dt A log2 e
};

// bf16 pair (a in the low half, b in the high half): the upper 16 bits of each fp32 pattern
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }
// fp32 values a, b as two bf16 terms each, packed in pairs: hi = the values truncated to bf16,
// lo = the remainders v - hi truncated to bf16.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  hi = pack_hi(ua, ub);
  lo = pack_hi(__float_as_uint(a - __uint_as_float(ua & 0xFFFF0000u)),
               __float_as_uint(b - __uint_as_float(ub & 0xFFFF0000u)));
}
// two fp32 values rounded to bf16 (nearest, ties to even), a in the low half
__device__ __forceinline__ uint32_t cvt_pair(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}
// inclusive prefix sum over the 64 lanes of a wave on DPP moves: shifts by 1, 2, 4, 8 inside
// each row of 16 lanes, then the row totals carried forward (lane 15 into rows 1 and 3, lane
// 31 into rows 2 and 3)
__device__ __forceinline__ float dpp_add(float x, float y) { return x + y; }
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_mv(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x = dpp_add(x, dpp_mv<0x111, 0xF>(x));  // row_shr:1
  x = dpp_add(x, dpp_mv<0x112, 0xF>(x));  // row_shr:2
  x = dpp_add(x, dpp_mv<0x114, 0xF>(x));  // row_shr:4
  x = dpp_add(x, dpp_mv<0x118, 0xF>(x));  // row_shr:8
  x = dpp_add(x, dpp_mv<0x142, 0xA>(x));  // row_bcast:15
  x = dpp_add(x, dpp_mv<0x143, 0xC>(x));  // row_bcast:31
  return x;
}

__device__ __forceinline__ v8bf ld8(const uint16_t* p) { return __builtin_bit_cast(v8bf, *(const v4i*)p); }
// 4 + 4 bf16 from two 8-byte locations
__device__ __forceinline__ v8bf ld44(const uint16_t* p0, const uint16_t* p1) {
  const uint2 a = *(const uint2*)p0, b = *(const uint2*)p1;
  return __builtin_bit_cast(v8bf, v4i{(int)a.x, (int)a.y, (int)b.x, (int)b.y});
}
__device__ __forceinline__ v4i buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void buf_st8(uint2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2_t, v), r, off, 0, 0);
}
__device__ __forceinline__ v8bf mk8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(v8bf, v4i{(int)a, (int)b, (int)c, (int)d});
}
}  // namespace

template <int NS, bool LOCAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_ssd_seg(ScanArgs a, SsdSeg sg) {
  constexpr int Q = kSsdQ, P = kSsdP, HB = kSsdHB, XS = kSsdXS;
  constexpr int NT = NS / 16;   // n tiles
  constexpr int NK = NS / 32;   // 32-wide k steps over n
  __shared__ __align__(16) uint16_t sBr[LOCAL ? 1 : Q * NS];  // B [s][n]
  __shared__ __align__(16) uint16_t sC[LOCAL ? 1 : Q * NS];   // C [t][n]
  __shared__ __align__(16) uint16_t sBT[NS * XS];              // B^T [n][s]
  __shared__ __align__(16) uint16_t sXT[HB][P * XS];           // x^T [p][s] per head
  __shared__ __align__(16) float s_cs[HB][Q], s_dt[HB][Q], s_w[HB][Q], s_et[HB][Q];
  __shared__ __align__(16) float s_b[LOCAL ? 1 : HB][Q];
  // G^T = B C^T of the chunk (shared by the heads): its 10 tiles on and below the diagonal in
  // the accumulator layout, tile (t tile jt, s tile ms <= jt) at index jt (jt + 1) / 2 + ms
  __shared__ __align__(16) float sG[LOCAL ? 1 : 10 * 256];

  // Element (r, c) of the [64][NS] arrays B and C (bf16 index): panels of 32 columns, each 64
  // rows of 64 bytes, a row's 16-byte chunk q at position q ^ ((r / 2) mod 4).  A fragment read
  // (16 consecutive rows, one chunk per group of 16 lanes) then reaches every bank once per
  // 8 lanes, and its address is a per-lane base plus a constant.
  auto pm = [](int r, int c) { return (c >> 5) * (Q * 32) + r * 32 + ((((c >> 3) & 3) ^ ((r >> 1) & 3)) << 3) + (c & 7); };
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = w >> 1, ph = w & 1;
  const int kq = lane >> 4, l16 = lane & 15;
  // per-lane base of the fragment reads of B and C: pm(16 i + l16, 32 k + 8 kq) = fb + 2048 k +
  // 512 i
  const int sw = (l16 >> 1) & 3;
  const int fb = l16 * 32 + ((kq ^ sw) << 3);
  const int64_t L = a.L, H = a.H;
  const int64_t nhb = cdiv(H, HB);
  // blocks are dealt to the 8 XCDs round-robin by index: block i takes work item
  // (i mod 8) T / 8 + i / 8, so that each XCD works through a contiguous run of items, heads
  // fastest, and its L2 serves the B and C rows that all heads of a sequence share
  const int64_t T = (int64_t)gridDim.x, i = blockIdx.x;
  const int64_t wi = (T % 8 == 0) ? (i % 8) * (T / 8) + i / 8 : i;
  const int64_t nbh = a.batch * nhb;
  const int seg = (int)(wi / nbh);
  const int64_t b = (wi % nbh) / nhb, hb = wi % nhb;
  const int64_t head = hb * HB + hl;
  const bool hv = head < H;
  const int64_t hc = hv ? head : H - 1;  // parameters of a valid head for waves past the last
  const float A2 = a.A[hc] * kLog2e;
  const float bias_h = a.delta_bias ? a.delta_bias[hc] : 0.0f;
  const float D_h = a.D ? a.D[hc] : 0.0f;
  const bf16_t* X = (const bf16_t*)a.x;
  const bf16_t* Bm = (const bf16_t*)a.Bm;
  const bf16_t* Cm = (const bf16_t*)a.Cm;
  const bf16_t* DT = (const bf16_t*)a.delta;
  const bf16_t* G = (const bf16_t*)a.gate;
  bf16_t* Y = (bf16_t*)a.y;
  const int64_t nch = cdiv(L, Q);
  const int64_t ch0 = (int64_t)seg * sg.seg_ch;
  const int64_t ch1 = ch0 + sg.seg_ch < nch ? ch0 + sg.seg_ch : nch;

  // state h^T: lane holds h[p = 16 (2 ph + ip) + l16][n = nst(mn) + 8 kq + r], where the state
  // tiles are taken in pairs: nst(mn) = 32 (mn / 2) + 4 (mn mod 2).  A pair of tiles then holds
  // eight consecutive n per lane, the k order of one 16-byte fragment read of C's rows in the
  // product h C^T below (the A rows of the state update are read in the same order).
  auto nst = [](int mn) { return 32 * (mn >> 1) + 4 * (mn & 1); };
  v4f hT[NT][2];
  {
    const float* src = nullptr;
    if (!LOCAL) {
      if (seg == 0) src = a.h0 ? a.h0 + (b * H + hc) * (int64_t)P * NS : nullptr;
      else src = sg.hloc + ((b * (sg.S - 1) + seg - 1) * H + hc) * (int64_t)P * NS;
    }
#pragma unroll
    for (int mn = 0; mn < NT; ++mn)
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) {
        const int pp = 16 * (2 * ph + ip) + l16;
        hT[mn][ip] = src ? *(const v4f*)(src + pp * NS + nst(mn) + 8 * kq) : v4f{0.f, 0.f, 0.f, 0.f};
      }
  }

  // ---- chunk loads into registers: 4 consecutive steps x 8 consecutive columns per task ----
  // x of the block's heads (columns hb HB P .. + HB P): tasks (cg = tid % 32, tg = tid / 32)
  // B (and C): NS / 8 column groups x 16 step groups; B on threads [0, NBT), C on [NBT, 2 NBT)
  constexpr int NBT = NS / 8 * 16;
  // a set of prefetch registers: one chunk's x, B (or C) and dt (raw bf16).  Every load is
  // unconditional and kept raw (a load whose value is converted or selected at once makes the
  // compiler wait for all loads in flight right there); rows past the sequence's end, and
  // columns past the last head, read as zeros.
  struct Pre {
    v4i x[4], b[4];
    bf16_t dt;   // raw; converted when the chunk is staged
  };
  // (the step group is the fastest index across lanes, so that the transposed LDS writes of 16
  // lanes fill one row and the next 16 lanes the row 8 below: distinct banks)
  const int xtg = tid & 15, xcg = tid >> 4;
  const bool xv = (int64_t)hb * HB * P + xcg * 8 < H * P;  // the task's columns exist
  // (NBT is a multiple of 64: which of B and C a thread moves is a per-wave choice, and so are
  // the row base and stride below)
  const bool isb = w * 64 < NBT, isc = !LOCAL && !isb && w * 64 < 2 * NBT;
  static_assert(NBT % 64 == 0, "B and C tasks by whole waves");
  const int btask = isb ? tid : tid - NBT;
  const int btg = btask & 15, bcg = btask >> 4;
  const bf16_t* bbase = isc ? Cm : Bm;
  const int64_t bld = isc ? a.ld_C : a.ld_B;
  // Addresses: the chunk's rows as a buffer resource shared by the wave (rows past the
  // sequence's end read as zeros), plus a 32-bit byte offset per lane (row strides below 2^24
  // elements, checked at launch).
  const uint32_t xcol = xcg * 8, bcol = bcg * 8;
  auto rows_in = [&](int64_t c0) -> uint32_t { return (uint32_t)(L - c0 < Q ? L - c0 : Q); };
  // part u of a chunk's loads (the parts are issued spread over a chunk's work)
  auto load_part = [&](Pre& pr, int64_t c0, int u) {
    const uint32_t rv = rows_in(c0);
    const auto rx = buf_rsrc(X + (b * L + c0) * a.ld_x + hb * HB * P, rv * (uint32_t)a.ld_x * 2u);
    pr.x[u] = buf_ld16(rx, xv ? ((uint32_t)(4 * xtg + u) * (uint32_t)a.ld_x + xcol) * 2u : kOutside);
    if (isb || isc) {
      const auto rb = buf_rsrc(bbase + (b * L + c0) * bld, rv * (uint32_t)bld * 2u);
      pr.b[u] = buf_ld16(rb, ((uint32_t)(4 * btg + u) * (uint32_t)bld + bcol) * 2u);
    }
    if (u == 0) {
      const auto rd = buf_rsrc(DT + (b * L + c0) * a.ld_delta + hc, rv * (uint32_t)a.ld_delta * 2u);
      pr.dt = (bf16_t)__builtin_amdgcn_raw_buffer_load_b16(rd, (uint32_t)lane * (uint32_t)a.ld_delta * 2u, 0, 0);
    }
  };
  auto load = [&](Pre& pr, int64_t c0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) load_part(pr, c0, u);
  };

  // transposed 8-byte writes: column u of the 4 step vectors v0..v3 (8 bf16 each)
  auto tcol = [&](const v4i (&v)[4], int u) -> uint2 {
    const int d = u >> 1;
    const uint32_t sel = (u & 1) ? 0x07060302u : 0x05040100u;
    return uint2{__builtin_amdgcn_perm((uint32_t)v[1][d], (uint32_t)v[0][d], sel),
                 __builtin_amdgcn_perm((uint32_t)v[3][d], (uint32_t)v[2][d], sel)};
  };
  float cs_end = 0.0f;  // this chunk's cs at its last step (log2 domain), per wave
  auto stage = [&](Pre& pr, int64_t c0) {
    {
      const int hh = xcg >> 3, p0 = (xcg & 7) * 8;
#pragma unroll
      for (int u = 0; u < 8; ++u) *(uint2*)(&sXT[hh][(p0 + u) * XS + 4 * xtg]) = tcol(pr.x, u);
    }
    if (isb) {
#pragma unroll
      for (int u = 0; u < 8; ++u) *(uint2*)(&sBT[(bcg * 8 + u) * XS + 4 * btg]) = tcol(pr.b, u);
      if (!LOCAL) {
#pragma unroll
        for (int u = 0; u < 4; ++u) *(v4i*)(&sBr[pm(4 * btg + u, bcg * 8)]) = pr.b[u];
      }
    }
    if (!LOCAL && isc) {
#pragma unroll
      for (int u = 0; u < 4; ++u) *(v4i*)(&sC[pm(4 * btg + u, bcg * 8)]) = pr.b[u];
    }
    // dt = softplus(delta + bias) (0 past the end), cs = inclusive cumsum of dt A log2 e
    // (computed on every lane, then selected: no branch around the use of a loaded value)
    float dt = bf16_to_f32(pr.dt) + bias_h;
    if (a.softplus) dt = softplus_hw(dt);
    dt = (ph == 0 && hv && c0 + lane < L) ? dt : 0.0f;
    const float cs = wave_prefix_sum(dt * A2);
    cs_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
    if (ph == 0) {
      s_cs[hl][lane] = cs;
      s_dt[hl][lane] = dt;
      s_w[hl][lane] = __builtin_amdgcn_exp2f(cs_end - cs) * dt;
      s_et[hl][lane] = __builtin_amdgcn_exp2f(cs);
      // the decay from step s to the last step e of its 16-step tile, times dt_s: the factor of
      // exp2(cs_t - cs_s) = exp2(cs_t - cs_e) exp2(cs_e - cs_s) that depends on s alone (cs is
      // monotone, dt >= 0, so neither factor leaves the range of the whole)
      if (!LOCAL) s_b[hl][lane] = __builtin_amdgcn_exp2f(__shfl(cs, lane | 15, 64) - cs) * dt;
    }
  };

  // Loads run DEPTH chunks ahead: the state-only pass (few registers) keeps two sets of
  // prefetch registers, the output pass one.
  constexpr int DEPTH = LOCAL ? 2 : 1;
  float sdec = 0.0f;
  auto body = [&](Pre& pr, int64_t ch) {
    const int64_t c0 = ch * Q;
    stage(pr, c0);
    __syncthreads();
    // the loads of chunk ch + DEPTH go into the set just staged, in four parts spread over this
    // chunk's products (issued at once, 64 KB per block would hold every wave at the address
    // unit); in the state pass unconditional (past the segment's end they repeat its last chunk,
    // from the cache), so that the wait for each set counts the loads issued after it exactly
    const int64_t cn = (ch + DEPTH < ch1 ? ch + DEPTH : ch1 - 1) * Q;
    const bool more = !LOCAL && ch + 1 < ch1;
    // the head's dt comes from its even wave's load: both waves take its staged cs_end
    cs_end = s_cs[hl][Q - 1];
    sdec += cs_end;
    const float* ws_ = s_w[hl];

    if (!LOCAL) {
      // ---- the G^T tiles: wave w computes tile w (waves 0 and 1 also tiles 8 and 9)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int tix = w + 8 * k;
        if (tix < 10) {
          const int jt = tix >= 6 ? 3 : tix >= 3 ? 2 : tix >= 1 ? 1 : 0;
          const int ms = tix - jt * (jt + 1) / 2;
          v4f gt = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NK; ++kk)
            gt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld8(&sBr[fb + 2048 * kk + 512 * ms]),
                                                         ld8(&sC[fb + 2048 * kk + 512 * jt]), gt, 0, 0, 0);
          *(v4f*)(&sG[tix * 256 + lane * 4]) = gt;
        }
      }
      // ---- Z^T = h C^T per (p tile ip, t tile jt), scaled by exp(cs_t): lane holds
      // Z^T[p = 16 (2 ph + ip) + 4 kq + r][t = 16 jt + l16]
      v4f zacc[2][4];
#pragma unroll
      for (int ip = 0; ip < 2; ++ip)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) zacc[ip][jt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m2 = 0; m2 < NT / 2; ++m2) {
        __builtin_amdgcn_sched_barrier(0);
        v8bf ah[2];
#pragma unroll
        for (int ip = 0; ip < 2; ++ip)
          ah[ip] = mk8(cvt_pair(hT[2 * m2][ip][0], hT[2 * m2][ip][1]), cvt_pair(hT[2 * m2][ip][2], hT[2 * m2][ip][3]),
                       cvt_pair(hT[2 * m2 + 1][ip][0], hT[2 * m2 + 1][ip][1]),
                       cvt_pair(hT[2 * m2 + 1][ip][2], hT[2 * m2 + 1][ip][3]));
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          // C rows t = 16 jt + l16 at the slots' n (32 m2 + 8 kq + u)
          const v8bf cf = ld8(&sC[fb + 2048 * m2 + 512 * jt]);
#pragma unroll
          for (int ip = 0; ip < 2; ++ip) {
            zacc[ip][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ip], cf, zacc[ip][jt], 0, 0, 0);
          }
        }
      }
      bar_lds();  // the G^T tiles written
      const float* cs_ = s_cs[hl];
      const float* dt_ = s_dt[hl];
      const float* et_ = s_et[hl];
      const float* bs_ = s_b[LOCAL ? 0 : hl];
      const uint16_t* xt = sXT[hl];
      // x^T rows p = 16 (2 ph + ip) + l16 at the slots' s (32 pr + 4 kq + u, 32 pr + 16 + 4 kq + u)
      v8bf xa[2][2];
#pragma unroll
      for (int ip = 0; ip < 2; ++ip)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const uint16_t* xr = &xt[(16 * (2 * ph + ip) + l16) * XS + 32 * pr + 4 * kq];
          xa[ip][pr] = ld44(xr, xr + 16);
        }
      // ---- per t tile jt: G^T tiles (s tile ms <= jt; lane holds G^T[16 ms + 4 kq + r][16 jt + l16]),
      // M^T = G^T exp(cs_t - cs_s) dt_s on s <= t (+ D on the diagonal), then y^T += x^T M^T
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        // (each t tile's reads, products and stores kept together: hoisted LDS reads of later
        // tiles would need more registers than a wave has)
        __builtin_amdgcn_sched_barrier(0);
        if (more) load_part(pr, cn, jt);
        v4f g[4];
#pragma unroll
        for (int ms = 0; ms <= jt; ++ms) g[ms] = *(const v4f*)(&sG[(jt * (jt + 1) / 2 + ms) * 256 + lane * 4]);
        const int t = 16 * jt + l16;
        const float cst = cs_[t];
        const float e = et_[t];
#pragma unroll
        for (int ip = 0; ip < 2; ++ip)
#pragma unroll
          for (int r = 0; r < 4; ++r) zacc[ip][jt][r] *= e;
        uint32_t mh[4][2];
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          if (ms > jt) {  // above the diagonal: zero (the partner of a diagonal tile in its pair)
            mh[ms][0] = mh[ms][1] = 0u;
            continue;
          }
          float m[4];
          if (ms < jt) {
            // below the diagonal (every s < t): exp2(cs_t - cs_s) dt_s as exp2(cs_t - cs_e) times
            // exp2(cs_e - cs_s) dt_s, e the last step of s's tile (the second factor staged)
            const float at = __builtin_amdgcn_exp2f(cst - cs_[16 * ms + 15]);
            const v4f bs = *(const v4f*)(&bs_[16 * ms + 4 * kq]);
#pragma unroll
            for (int r = 0; r < 4; ++r) m[r] = g[ms][r] * bs[r] * at;
          } else {
            const v4f css = *(const v4f*)(&cs_[16 * ms + 4 * kq]);
            const v4f dts = *(const v4f*)(&dt_[16 * ms + 4 * kq]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int sidx = 16 * ms + 4 * kq + r;
              m[r] = 0.0f;
              if (sidx <= t) m[r] = g[ms][r] * (__builtin_amdgcn_exp2f(cst - css[r]) * dts[r]);
              if (sidx == t) m[r] += D_h;
            }
          }
          mh[ms][0] = cvt_pair(m[0], m[1]);
          mh[ms][1] = cvt_pair(m[2], m[3]);
        }
#pragma unroll
        for (int pr = 0; 2 * pr <= jt; ++pr) {
          const v8bf bh = mk8(mh[2 * pr][0], mh[2 * pr][1], mh[2 * pr + 1][0], mh[2 * pr + 1][1]);
#pragma unroll
          for (int ip = 0; ip < 2; ++ip) {
            zacc[ip][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[ip][pr], bh, zacc[ip][jt], 0, 0, 0);
          }
        }
        // ---- y: lane holds y[t][p = 16 (2 ph + ip) + 4 kq + r] (rows past the sequence's end
        // fall outside the chunk's resource: their stores are dropped)
        if (hv) {
          const uint32_t rv = rows_in(c0);
          const auto ry = buf_rsrc(Y + (b * L + c0) * a.ld_y + head * P, rv * (uint32_t)a.ld_y * 2u);
#pragma unroll
          for (int ip = 0; ip < 2; ++ip) {
            const uint32_t colw = 16 * (2 * ph + ip) + 4 * kq;
            float v[4] = {zacc[ip][jt][0], zacc[ip][jt][1], zacc[ip][jt][2], zacc[ip][jt][3]};
            if (G) {
              const auto rg = buf_rsrc(G + (b * L + c0) * a.ld_gate + head * P, rv * (uint32_t)a.ld_gate * 2u);
              const uint2 gg = buf_ld8(rg, ((uint32_t)t * (uint32_t)a.ld_gate + colw) * 2u);
              v[0] *= silu_gate(bf16_to_f32((bf16_t)(gg.x & 0xFFFFu)));
              v[1] *= silu_gate(bf16_to_f32((bf16_t)(gg.x >> 16)));
              v[2] *= silu_gate(bf16_to_f32((bf16_t)(gg.y & 0xFFFFu)));
              v[3] *= silu_gate(bf16_to_f32((bf16_t)(gg.y >> 16)));
            }
            const uint2 o{cvt_pair(v[0], v[1]), cvt_pair(v[2], v[3])};
            buf_st8(o, ry, ((uint32_t)t * (uint32_t)a.ld_y + colw) * 2u);
          }
        }
      }
    }

    // ---- state: h^T = exp(cs_end) h^T + B^T (w x)
    __builtin_amdgcn_sched_barrier(0);
    const float ed = __builtin_amdgcn_exp2f(cs_end);
#pragma unroll
    for (int mn = 0; mn < NT; ++mn)
#pragma unroll
      for (int ip = 0; ip < 2; ++ip)
#pragma unroll
        for (int r = 0; r < 4; ++r) hT[mn][ip][r] *= ed;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (LOCAL) load_part(pr, cn, 2 * kk);
      const v4f w0 = *(const v4f*)(&ws_[32 * kk + 8 * kq]);
      const v4f w1 = *(const v4f*)(&ws_[32 * kk + 8 * kq + 4]);
      const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      v8bf xh[2], xl[2];
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) {
        const v4i raw = *(const v4i*)(&sXT[hl][(16 * (2 * ph + ip) + l16) * XS + 32 * kk + 8 * kq]);
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t word = (uint32_t)raw[d];
          split_pair(__uint_as_float(word << 16) * wv[2 * d], __uint_as_float(word & 0xFFFF0000u) * wv[2 * d + 1],
                     hi[d], lo[d]);
        }
        xh[ip] = mk8(hi[0], hi[1], hi[2], hi[3]);
        xl[ip] = mk8(lo[0], lo[1], lo[2], lo[3]);
      }
#pragma unroll
      for (int mn = 0; mn < NT; ++mn) {
        if (LOCAL && mn == NT / 2) load_part(pr, cn, 2 * kk + 1);
        // B^T row n = nst(mn) + 8 (l16 / 4) + l16 mod 4 (output row 4 kq + r is then n = nst(mn) + 8 kq + r)
        const v8bf bt = ld8(&sBT[(nst(mn) + 8 * (l16 >> 2) + (l16 & 3)) * XS + 32 * kk + 8 * kq]);
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {
          hT[mn][ip] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt, xh[ip], hT[mn][ip], 0, 0, 0);
          hT[mn][ip] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt, xl[ip], hT[mn][ip], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  };
  Pre p0, p1;
  load(p0, ch0 * Q);
  if (DEPTH == 1) {
    for (int64_t ch = ch0; ch < ch1; ++ch) body(p0, ch);
  } else {
    load(p1, (ch0 + 1 < ch1 ? ch0 + 1 : ch0) * Q);
    int64_t ch = ch0;
    for (; ch + 1 < ch1; ch += 2) {  // the two sets by parity, each named statically
      body(p0, ch);
      body(p1, ch + 1);
    }
    if (ch < ch1) body(p0, ch);
  }

  // ---- the segment's end state: pass 1 keeps it (and the segment's decay) for the combine;
  // the last segment of pass 2 returns it
  float* dst = nullptr;
  if (LOCAL) dst = sg.hloc + ((b * (sg.S - 1) + seg) * H + hc) * (int64_t)P * NS;
  else if (a.h_last && seg == sg.S - 1) dst = a.h_last + (b * H + hc) * (int64_t)P * NS;
  if (dst && hv) {
#pragma unroll
    for (int mn = 0; mn < NT; ++mn)
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) *(v4f*)(dst + (16 * (2 * ph + ip) + l16) * NS + nst(mn) + 8 * kq) = hT[mn][ip];
  }
  if (LOCAL && hv && ph == 0 && lane == 0) sg.sdec[(b * (sg.S - 1) + seg) * H + head] = sdec;
}

// Combine over segments, per (sequence, head, state element): afterwards hloc[b, s] holds the
// state entering segment s + 1.
template <int V>
__global__ __launch_bounds__(256) void k_ssd_combine(const float* __restrict__ h0, float* __restrict__ hloc,
                                                     const float* __restrict__ sdec, int64_t B, int64_t H,
                                                     int64_t PN, int S) {
  typedef float fv __attribute__((ext_vector_type(V)));
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;  // V consecutive state elements
  if (i >= B * H * PN) return;
  const int64_t b = i / (H * PN), hp = i % (H * PN), hd = hp / PN, e = hp % PN;
  fv h = h0 ? *(const fv*)(h0 + i) : fv{};
  // four segments' loads first, then their chain of updates
  for (int s0 = 0; s0 + 1 < S; s0 += 4) {
    const int n = (S - 1 - s0) < 4 ? (S - 1 - s0) : 4;
    fv v[4];
    float d[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t bs = b * (S - 1) + s0 + (k < n ? k : 0);
      v[k] = *(const fv*)(hloc + (bs * H + hd) * PN + e);
      d[k] = __builtin_amdgcn_exp2f(sdec[bs * H + hd]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < n) {
#pragma unroll
        for (int c = 0; c < V; ++c) h[c] = __builtin_fmaf(d[k], h[c], v[k][c]);
        *(fv*)(hloc + ((b * (S - 1) + s0 + k) * H + hd) * PN + e) = h;
      }
    }
  }
}

// The chunked kernels take bf16 activations with headdim 64, d_state 64 or 128, dt through
// softplus (dt >= 0: the decay exponent cs is monotone along a chunk, which the split of the
// decays at tile ends relies on), and row strides and bases that allow 16-byte loads of x, B
// and C (8-byte loads of the gate), below 2^24 elements.
static bool ssd_chunk_ok(const ScanArgs& a) {
  auto al = [](const void* p) { return ((uintptr_t)p % 16) == 0; };
  const int64_t lim = int64_t(1) << 24;
  if (a.ld_x >= lim || a.ld_B >= lim || a.ld_C >= lim || a.ld_delta >= lim || a.ld_y >= lim || a.ld_gate >= lim)
    return false;
  return a.act_bf16 && a.softplus && a.P == kSsdP && (a.N == 64 || a.N == 128) && a.ld_x % 8 == 0 && a.ld_B % 8 == 0 &&
         a.ld_C % 8 == 0 && al(a.x) && al(a.Bm) && al(a.Cm) && (!a.gate || (a.ld_gate % 4 == 0 && ((uintptr_t)a.gate % 8) == 0));
}

namespace {
// Segment count: a function of the shape only.  Blocks of (sequence, 4 heads) below 256 (one
// per MI355X compute unit) are multiplied by time segments of whole chunks.
struct SsdPlan {
  int S = 1, seg_ch = 1;
  size_t ws = 0;
};
SsdPlan plan_ssd(const ScanArgs& a) {
  SsdPlan p;
  const int64_t nch = cdiv(a.L, kSsdQ);
  const int64_t blocks = a.batch * cdiv(a.H, kSsdHB);
  int64_t S = 1;
  if (blocks < 256) S = cdiv(256, blocks);
  if (S > nch) S = nch;
  if (S < 1) S = 1;
  p.seg_ch = (int)cdiv(nch, S);
  p.S = (int)cdiv(nch, p.seg_ch);
  if (p.S > 1)
    p.ws = (size_t)a.batch * (p.S - 1) * a.H * ((size_t)a.P * a.N + 1) * sizeof(float);
  return p;
}
}  // namespace

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

// The segment carries of the chunked kernels (any dtype or alignment: a workspace query knows
// the shape only).
size_t scan_ssd_workspace(const ScanArgs& a) {
  if (a.batch == 0 || a.L == 0 || a.P != kSsdP || (a.N != 64 && a.N != 128)) return 0;
  return plan_ssd(a).ws;
}

hipError_t launch_scan_ssd(const ScanArgs& a, void* ws, size_t wsb, hipStream_t s) {
  if (a.batch == 0 || a.L == 0) return hipSuccess;
  if (ssd_chunk_ok(a)) {
    const SsdPlan p = plan_ssd(a);
    if (p.ws > wsb || (p.ws && !ws)) return hipErrorInvalidValue;
    SsdSeg sg{};
    sg.S = p.S;
    sg.seg_ch = p.seg_ch;
    if (p.S > 1) {
      sg.hloc = (float*)ws;
      sg.sdec = sg.hloc + (size_t)a.batch * (p.S - 1) * a.H * a.P * a.N;
    }
    const unsigned nb = (unsigned)(a.batch * cdiv(a.H, kSsdHB));
    if (p.S > 1) {
      const dim3 g1(nb * (unsigned)(p.S - 1));
      if (a.N == 128) hipLaunchKernelGGL((k_ssd_seg<128, true>), g1, dim3(512), 0, s, a, sg);
      else hipLaunchKernelGGL((k_ssd_seg<64, true>), g1, dim3(512), 0, s, a, sg);
      const int64_t n = a.batch * a.H * a.P * a.N;
      if (!a.h0 || (uintptr_t)a.h0 % 16 == 0)
        hipLaunchKernelGGL(k_ssd_combine<4>, dim3((unsigned)cdiv(n, 1024)), dim3(256), 0, s, a.h0, sg.hloc, sg.sdec,
                           a.batch, a.H, a.P * a.N, p.S);
      else
        hipLaunchKernelGGL(k_ssd_combine<1>, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, a.h0, sg.hloc, sg.sdec,
                           a.batch, a.H, a.P * a.N, p.S);
    }
    const dim3 g2(nb * (unsigned)p.S);
    if (a.N == 128) hipLaunchKernelGGL((k_ssd_seg<128, false>), g2, dim3(512), 0, s, a, sg);
    else hipLaunchKernelGGL((k_ssd_seg<64, false>), g2, dim3(512), 0, s, a, sg);
    return hipGetLastError();
  }
  return a.act_bf16 ? launch_ssd_n<bf16_t>(a, s) : launch_ssd_n<float>(a, s);
}

}  // namespace ssm
