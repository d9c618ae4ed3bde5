// Full-precision linear layers (the TriSSM model's in and out projections, and every
// projection of its fp_ssm baseline): y = x W^T (+ residual), no norm, no quantisation; and the
// plain fp32 product the straight-through backward uses when its fused kernel does not apply.
// Dense GEMMs on the matrix cores: fp32 operands on MFMA 16x16x4 f32, bf16 operands on MFMA
// 16x16x32 bf16, fp32 accumulation either way.  No library, no device memory of their own.
//
// Block tile 64 outputs x 64 tokens, 4 waves each owning 32 x 32 as 2 x 2 MFMA tiles.  The
// weights are the MFMA A operand (rows = outputs) and the activations the B operand, so a lane
// ends with 4 consecutive outputs of one token.  Each k step (16 fp32 or 32 bf16 values, one
// 64-byte row slice per row) is staged in LDS through registers, double-buffered: the next
// step's 16-byte chunks are loaded while the current one is contracted.  In LDS a row's four
// chunks sit in the order q ^ ((row / 2) mod 4), which keeps the 16-byte fragment reads free of
// bank conflicts.  With fp32 operands lane group kq takes k = 4 kq .. 4 kq + 3 of the step and
// issues one MFMA per k (the sum over the step does not depend on how k is dealt out).
#include "launch.hpp"

namespace ssm {

namespace {
constexpr int kDT = 64;  // tile rows (outputs) and columns (tokens)

template <typename T> struct DenseMath;
template <> struct DenseMath<float> {
  static constexpr int KS = 16;  // k per step
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};
template <> struct DenseMath<bf16_t> {
  static constexpr int KS = 32;
  static __device__ __forceinline__ float to_f(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f(float v) { return f32_to_bf16(v); }
};

// LDS byte offset of 16-byte chunk q of tile row r
__device__ __forceinline__ int chunk_off(int r, int q) { return r * 64 + ((q ^ ((r >> 1) & 3)) << 4); }

struct DenseKernelArgs {
  int64_t M, N, K;
  const void* x; int64_t ldx;           // [M, K] (row stride ldx)
  const void* W; int64_t ldw;           // [N, K] (row stride ldw), or [K, N] when transposed
  const void* residual; int64_t ld_res;
  void* y; int64_t ldy;
};

// One 16-byte chunk of row r (of R rows, starting at column k0 + 4/8 q) of a row-major
// matrix, zero past the row or column end.  VEC: whole chunks are in bounds and aligned.
template <typename T, bool VEC>
__device__ __forceinline__ v4i load_chunk(const T* p, int64_t ld, int64_t r, int64_t R, int64_t c, int64_t C) {
  constexpr int E = 16 / sizeof(T);
  if (VEC) {
    if (r < R && c < C) return *(const v4i*)(p + r * ld + c);
    return v4i{0, 0, 0, 0};
  }
  T v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = (r < R && c + e < C) ? p[r * ld + c + e] : (T)0;
  return *(const v4i*)v;
}

template <typename T, bool VEC, bool WT>
__global__ __launch_bounds__(256) void k_dense(DenseKernelArgs a) {
  using DM = DenseMath<T>;
  constexpr int KS = DM::KS, E = 16 / (int)sizeof(T);
  __shared__ __align__(16) int8_t s_w[2][kDT * 64];
  __shared__ __align__(16) int8_t s_x[2][kDT * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wo = wave >> 1, wt = wave & 1;
  const int kq = lane >> 4, l16 = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * kDT, m0 = (int64_t)blockIdx.y * kDT;
  const T* X = (const T*)a.x;
  const T* Wp = (const T*)a.W;
  // staging: thread t moves chunk t & 3 of row t >> 2 of each tile (transposed weights: a run
  // of E outputs of one k, scattered into the rows in LDS)
  const int sr = tid >> 2, sq = tid & 3;
  v4i px, pw;
  auto load = [&](int64_t k0) {
    px = load_chunk<T, VEC>(X, a.ldx, m0 + sr, a.M, k0 + sq * E, a.K);
    if (!WT) {
      pw = load_chunk<T, VEC>(Wp, a.ldw, n0 + sr, a.N, k0 + sq * E, a.K);
    } else {
      // rows k0 .. k0 + KS - 1 of W^T [K, N], E consecutive outputs per thread
      const int kr = tid / (kDT / E), nc = (tid % (kDT / E)) * E;
      pw = load_chunk<T, VEC>(Wp, a.ldw, k0 + kr, a.K, n0 + nc, a.N);
    }
  };
  auto store = [&](int buf) {
    *(v4i*)(&s_x[buf][chunk_off(sr, sq)]) = px;
    if (!WT) {
      *(v4i*)(&s_w[buf][chunk_off(sr, sq)]) = pw;
    } else {
      const int kr = tid / (kDT / E), nc = (tid % (kDT / E)) * E;
      const T* v = (const T*)&pw;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int r = nc + e;
        ((T*)&s_w[buf][chunk_off(r, kr / E)])[kr % E] = v[e];
      }
    }
  };
  v4f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const int64_t nk = cdiv(a.K, KS);
  load(0);
  store(0);
  __syncthreads();
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = (int)(ks & 1);
    if (ks + 1 < nk) load((ks + 1) * KS);
    v4i fw[2], fx[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) fw[i] = *(const v4i*)(&s_w[buf][chunk_off(wo * 32 + i * 16 + l16, kq)]);
#pragma unroll
    for (int j = 0; j < 2; ++j) fx[j] = *(const v4i*)(&s_x[buf][chunk_off(wt * 32 + j * 16 + l16, kq)]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (sizeof(T) == 4) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(fw[i][s]), __int_as_float(fx[j][s]),
                                                             acc[i][j], 0, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const v8bf*)&fw[i], *(const v8bf*)&fx[j],
                                                              acc[i][j], 0, 0, 0);
        }
      }
    if (ks + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  // lane holds outputs n .. n + 3 of token m for each tile pair
  T* Y = (T*)a.y;
  const T* R = (const T*)a.residual;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t m = m0 + wt * 32 + j * 16 + l16;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t n = n0 + wo * 32 + i * 16 + kq * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (n + r >= a.N) continue;
        float v = acc[i][j][r];
        if (R) v += DM::to_f(R[m * a.ld_res + n + r]);
        Y[m * a.ldy + n + r] = DM::from_f(v);
      }
    }
  }
}

template <typename T, bool WT>
hipError_t launch_dense_t(const DenseKernelArgs& a, hipStream_t s) {
  constexpr int E = 16 / (int)sizeof(T);
  const bool vec = WT ? (a.N % E == 0 && a.ldw % E == 0 && ((uintptr_t)a.W) % 16 == 0 && a.K % E == 0 &&
                         a.ldx % E == 0 && ((uintptr_t)a.x) % 16 == 0)
                      : (a.K % E == 0 && a.ldx % E == 0 && a.ldw % E == 0 && ((uintptr_t)a.x) % 16 == 0 &&
                         ((uintptr_t)a.W) % 16 == 0);
  const dim3 grid((unsigned)cdiv(a.N, kDT), (unsigned)cdiv(a.M, kDT)), block(256);
  if (vec) hipLaunchKernelGGL((k_dense<T, true, WT>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_dense<T, false, WT>), grid, block, 0, s, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_dense(const DenseArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (a.M > 65535LL * kDT || a.N > 0x7fffffffLL * kDT) return hipErrorInvalidValue;
  DenseKernelArgs k{a.M, a.N, a.K, a.x, a.ldx, a.W, a.K, a.residual, a.ld_res, a.y, a.ldy};
  return a.bf16 ? launch_dense_t<bf16_t, false>(k, s) : launch_dense_t<float, false>(k, s);
}

hipError_t sgemm_nn(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                    float* C, int64_t ldc, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (M > 65535LL * kDT) return hipErrorInvalidValue;
  // C = A B with B [K, N] row-major: the dense layer with transposed weights
  DenseKernelArgs k{M, N, K, A, lda, B, ldb, nullptr, 0, C, ldc};
  return launch_dense_t<float, true>(k, s);
}

}  // namespace ssm
