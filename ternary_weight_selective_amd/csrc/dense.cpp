// Full-precision linear layers (the TriSSM model's in and out projections, and every
// projection of its fp_ssm baseline): y = x W^T (+ residual), no norm, no quantisation.  These
// are plain dense GEMMs, so they go to rocBLAS (fp32, or bf16 with fp32 accumulation); the
// ternary projections keep their own kernels.  One rocBLAS handle per device, created on first
// use (rocBLAS sets up its own device workspace then) and kept for the life of the process.
#include <mutex>

#include <rocblas/rocblas.h>

#include "launch.hpp"

namespace ssm {

namespace {
constexpr int kMaxDevices = 64;
rocblas_handle g_handles[kMaxDevices] = {};
std::mutex g_mu;

hipError_t handle_for_device(rocblas_handle* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_handles[dev] && rocblas_create_handle(&g_handles[dev]) != rocblas_status_success) {
    g_handles[dev] = nullptr;
    return hipErrorInitializationError;
  }
  *out = g_handles[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_dense(const DenseArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  rocblas_handle h = nullptr;
  hipError_t e = handle_for_device(&h);
  if (e != hipSuccess) return e;
  const size_t es = a.bf16 ? 2 : 4;
  float beta = 0.0f;
  if (a.residual) {  // y starts as the residual, the product is added to it
    if (a.residual != a.y) {
      e = hipMemcpy2DAsync(a.y, (size_t)a.ldy * es, a.residual, (size_t)a.ld_res * es, (size_t)a.N * es,
                           (size_t)a.M, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return e;
    }
    beta = 1.0f;
  }
  const float alpha = 1.0f;
  // row-major y[M, N] = x[M, K] W[N, K]^T is column-major y^T[N, M] = W^T(op: transposed) x^T
  std::lock_guard<std::mutex> lock(g_mu);  // the stream is handle state
  if (rocblas_set_stream(h, s) != rocblas_status_success) return hipErrorInvalidValue;
  rocblas_status st;
  if (a.bf16) {
    st = rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)a.N, (rocblas_int)a.M,
                         (rocblas_int)a.K, &alpha, a.W, rocblas_datatype_bf16_r, (rocblas_int)a.K, a.x,
                         rocblas_datatype_bf16_r, (rocblas_int)a.ldx, &beta, a.y, rocblas_datatype_bf16_r,
                         (rocblas_int)a.ldy, a.y, rocblas_datatype_bf16_r, (rocblas_int)a.ldy,
                         rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  } else {
    st = rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)a.N, (rocblas_int)a.M,
                       (rocblas_int)a.K, &alpha, (const float*)a.W, (rocblas_int)a.K, (const float*)a.x,
                       (rocblas_int)a.ldx, &beta, (float*)a.y, (rocblas_int)a.ldy);
  }
  return st == rocblas_status_success ? hipSuccess : hipErrorLaunchFailure;
}

hipError_t sgemm_rm(bool ta, bool tb, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                    const float* B, int64_t ldb, float* C, int64_t ldc, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  rocblas_handle h = nullptr;
  hipError_t e = handle_for_device(&h);
  if (e != hipSuccess) return e;
  const float alpha = 1.0f, beta = 0.0f;
  // a row-major matrix is its column-major transpose: C^T = op(B)^T op(A)^T, same flags
  std::lock_guard<std::mutex> lock(g_mu);
  if (rocblas_set_stream(h, s) != rocblas_status_success) return hipErrorInvalidValue;
  const rocblas_status st =
      rocblas_sgemm(h, tb ? rocblas_operation_transpose : rocblas_operation_none,
                    ta ? rocblas_operation_transpose : rocblas_operation_none, (rocblas_int)N, (rocblas_int)M,
                    (rocblas_int)K, &alpha, B, (rocblas_int)ldb, A, (rocblas_int)lda, &beta, C, (rocblas_int)ldc);
  return st == rocblas_status_success ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace ssm
