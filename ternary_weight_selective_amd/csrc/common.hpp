// Device helpers shared by the gfx950 kernels of the ternary selective-SSM library.
// Compiled with -ffp-contract=off: every fused multiply-add below is written out.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

typedef uint16_t bf16_t;  // bf16 bit pattern as stored in memory

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest, ties to even (inputs are finite)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float ld_act(const T* p);
template <> __device__ __forceinline__ float ld_act<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_act<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }
// an activation value already in a register (a prefetched raw element) as fp32
__device__ __forceinline__ float act_f32(float v) { return v; }
__device__ __forceinline__ float act_f32(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ void st_act(T* p, float v);
template <> __device__ __forceinline__ void st_act<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st_act<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// A buffer resource over [base, base + bytes): loads past the end read zeros, stores past it
// are dropped; offsets are 32-bit byte offsets (a per-lane part and a wave-uniform part).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOutside = 0x80000000u;  // an offset past any resource here (all < 2^31 bytes)
// One activation element (fp32 or bf16 bits) at byte offset voff + soff.
template <typename T> __device__ __forceinline__ T buf_ld_act(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
template <> __device__ __forceinline__ float buf_ld_act<float>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
template <> __device__ __forceinline__ bf16_t buf_ld_act<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (bf16_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
// Store v as an activation (fp32, or bf16 rounded to nearest even).
template <typename T> __device__ __forceinline__ void buf_st_act(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
template <> __device__ __forceinline__ void buf_st_act<float>(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}
template <> __device__ __forceinline__ void buf_st_act<bf16_t>(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, voff, soff, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding (vmcnt only).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Block barrier ordering LDS only: global loads still in flight are not waited for (for
// phases that exchange data through LDS alone).
__device__ __forceinline__ void bar_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// SiLU of the gate branch, fp32: z / (1 + 2^(-z log2 e)) with the hardware exp2 (an infinite
// exponential for very negative z gives -0).
__device__ __forceinline__ float silu_gate(float z) {
  return z / (1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// Cross-lane moves.  ds_swizzle in bit-mask mode: lane j of each 32-lane half reads lane
// j ^ 16.  DPP (data-parallel primitives): a rotation of each row of 16 lanes, and quad
// permutations.
__device__ __forceinline__ float swz_xor16(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowRor8 = 0x128, kDppRowRor4 = 0x124;
constexpr int kDppXor2 = 0x4E, kDppXor1 = 0xB1;  // quad_perm [2,3,0,1], [1,0,3,2]

// Sum over the 64 lanes of a wave as six rounds in which lane j adds lane j ^ d,
// d = 32, 16, 8, 4, 2, 1.  fp32 addition is commutative, so every lane ends with the same
// value and the order of the additions is fixed.  After the rounds at d = 32 and 16 the lanes
// j, j ^ 16, j ^ 32, j ^ 48 hold equal values, and after d = 8 also j ^ 8: rotating each row
// of 16 lanes by 8 (then by 4) therefore reads a lane holding exactly the value of lane j ^ 8
// (then j ^ 4), so the rotations add the same operands as the xor rounds.
__device__ __forceinline__ float wave_sum_butterfly(float s) {
  s = s + __shfl_xor(s, 32, 64);
  s = s + swz_xor16(s);
  s = s + dpp_f<kDppRowRor8>(s);
  s = s + dpp_f<kDppRowRor4>(s);
  s = s + dpp_f<kDppXor2>(s);
  s = s + dpp_f<kDppXor1>(s);
  return s;
}

// Maximum over the 64 lanes of non-negative values (absolute values); every lane ends with
// it.  For non-negative floats the order of the bit patterns as unsigned integers is the
// numeric order, so the maximum is taken on the bit patterns (exact in any order).
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float wave_absmax(float m) {
  uint32_t u = __float_as_uint(m);
  u = max(u, (uint32_t)__shfl_xor((int)u, 32, 64));
  u = max(u, (uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x401F));
  u = max(u, dpp_u<kDppRowRor8>(u));
  u = max(u, dpp_u<kDppRowRor4>(u));
  u = max(u, dpp_u<kDppXor2>(u));
  u = max(u, dpp_u<kDppXor1>(u));
  return __uint_as_float(u);
}

// Correctly rounded fp32 square root.  The device's fp32 sqrt instruction sequence is not
// correctly rounded (it is off by one ulp on some inputs); a correctly rounded fp64 square
// root rounded once to fp32 is, because 53 >= 2 * 24 + 2 bits make the double rounding
// innocuous for square roots.
__device__ __forceinline__ float sqrt_rn(float x) { return (float)__dsqrt_rn((double)x); }

constexpr float LOG2E = 1.4426950408889634f;

// softplus(v) = log(1 + e^v), the identity above 20.  With z = e^v and u = fl(1 + z), the
// rounding error of u is c = (u - 1) - z (both subtractions exact), and
// log(1 + z) = log(u) - c / u + O(c^2).  While u < 2, |c| <= 2^-24 and taking c for c / u
// changes the result by at most |c| z / (1 + z), below its own rounding.  From u = 2 on, c
// can reach half an ulp of u, far more than c / u <= 2^-24, which is below the rounding of a
// result >= log 2: the correction is dropped there.  Below z = 1e-4 the series z - z^2 / 2.
// Branch-free, on the hardware exp2 and log2 (no reciprocal).
__device__ __forceinline__ float softplus_f(float v) {
  const float z = __builtin_amdgcn_exp2f(v * LOG2E);
  const float u = 1.0f + z;
  const float c = u < 2.0f ? (u - 1.0f) - z : 0.0f;
  const float big = 0.69314718055994531f * __builtin_amdgcn_logf(u) - c;
  const float small = z * __builtin_fmaf(-0.5f, z, 1.0f);
  const float r = z < 1e-4f ? small : big;
  return v > 20.0f ? v : r;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// RMSNorm + absmax int8 codes of RPW rows of K values held in the canonical lane layout (lane
// j holds columns j + 64 i, zero past K): the lane partials, the wave butterfly, the scalar
// tail once for the RPW rows (lane j takes row j mod RPW), codes into sq (row stride qs) and
// max(absmax, 1e-5) / 127 into sdeq.  gn: the gain per lane column (1 when absent).
template <int RPW, int KPL>
__device__ __forceinline__ void norm_quant_rows(float (&v)[RPW][KPL], const float (&gn)[KPL], int K, float eps,
                                                int8_t* sq, int qs, double* sdeq, int lane) {
  float ss[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < KPL; ++i) s = __builtin_fmaf(v[rr][i], v[rr][i], s);
    ss[rr] = wave_sum_butterfly(s);
  }
  float sel = ss[0];
#pragma unroll
  for (int rr = 1; rr < RPW; ++rr) sel = (lane % RPW) == rr ? ss[rr] : sel;
  const float rs_l = __fdiv_rn(1.0f, sqrt_rn(__fdiv_rn(sel, (float)K) + eps));
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
  if (lane < RPW) sdeq[lane] = (double)mf / 127.0;
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const float sigma = readlane_f(sigma_l, rr);
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      float q = rintf(v[rr][i] * sigma);
      q = fminf(fmaxf(q, -128.0f), 127.0f);
      sq[rr * qs + lane + 64 * i] = (int8_t)(int)q;
    }
  }
}

// 16 ternary codes of one packed word -> 16 int8 in weight order.  Dword j of the
// result holds weights 4j..4j+3; their 2-bit codes sit at bits 2j of bytes 0..3, so a
// shift and mask leave one code per byte and a byte permute maps code 0/1/3 to
// 0x00/0x01/0xFF through the table 0xFF000100.
__device__ __forceinline__ v4i unpack16_i8(uint32_t w) {
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, w & 0x03030303u);
  r[1] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, (w >> 2) & 0x03030303u);
  r[2] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, (w >> 4) & 0x03030303u);
  r[3] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, (w >> 6) & 0x03030303u);
  return r;
}

// 16 ternary codes of one packed word -> 16 bf16 (+1 = 0x3F80, -1 = 0xBF80, 0 = 0) in weight
// order, two per dword: o0 holds weights 0..7, o1 weights 8..15.  For j = 0..3 the codes of
// weights 4j..4j+3 are isolated one per byte (x); a byte permute spreads them into selectors
// [c, c | 4, c', c' | 4], and a second one looks the selectors up in an 8-byte table whose
// low half holds the bf16 low bytes (0x00, 0x80, -, 0x80) and high half the high bytes
// (0x00, 0x3F, -, 0xBF), indexed by the code.
__device__ __forceinline__ void unpack16_bf16(uint32_t w, v4i& o0, v4i& o1) {
  uint32_t d[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t x = (w >> (2 * j)) & 0x03030303u;
    const uint32_t x4 = x | 0x04040404u;
    d[2 * j] = __builtin_amdgcn_perm(0xBF003F00u, 0x80008000u, __builtin_amdgcn_perm(x4, x, 0x05010400u));
    d[2 * j + 1] = __builtin_amdgcn_perm(0xBF003F00u, 0x80008000u, __builtin_amdgcn_perm(x4, x, 0x07030602u));
  }
  o0 = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
  o1 = v4i{(int)d[4], (int)d[5], (int)d[6], (int)d[7]};
}

// Two int8 ternary values (low two bytes of b) -> two bf16 (+1 = 0x3F80, -1 = 0xBF80, 0 = 0).
__device__ __forceinline__ uint32_t tern2_to_bf16x2(uint32_t b) {
  uint32_t lo = b & 0xFFu, hi = (b >> 8) & 0xFFu;
  uint32_t vlo = lo ? (0x3F80u | ((lo & 0x80u) << 8)) : 0u;
  uint32_t vhi = hi ? (0x3F80u | ((hi & 0x80u) << 8)) : 0u;
  return vlo | (vhi << 16);
}


__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

}  // namespace ssm
