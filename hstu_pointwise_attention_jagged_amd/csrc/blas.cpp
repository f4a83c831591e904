// Plain GEMMs of the layer backward through rocBLAS: dG = dY w2, dw2 = dY^T G, dX = dZ w1
// and dw1 = dZ^T X, bf16 operands with fp32 accumulation and output.  rocBLAS is
// column-major, so the row-major product C = op(A) op(B) is issued as
// C^T = op(B)^T op(A)^T.  One handle per device, created on first use, with atomics
// disallowed so that results do not depend on scheduling.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <mutex>

#include "kernels.h"

namespace hstu {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_blas_mu;
rocblas_handle g_handles[kMaxDevices] = {};

}  // namespace

hipError_t blas_gemm_bf16(bool a_trans, bool b_trans, int M, int N, int K, const uint16_t *A,
                          int64_t lda, const uint16_t *B, int64_t ldb, float *C, int64_t ldc,
                          float beta, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K <= 0) return hipErrorInvalidValue;  // callers handle empty sums themselves
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle &h = g_handles[dev];
  if (h == nullptr) {
    if (rocblas_create_handle(&h) != rocblas_status_success) {
      h = nullptr;
      return hipErrorUnknown;
    }
    rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed);
  }
  if (rocblas_set_stream(h, stream) != rocblas_status_success) return hipErrorUnknown;
  const float alpha = 1.0f;
  const rocblas_status st = rocblas_gemm_ex(
      h, b_trans ? rocblas_operation_transpose : rocblas_operation_none,
      a_trans ? rocblas_operation_transpose : rocblas_operation_none, N, M, K, &alpha, B,
      rocblas_datatype_bf16_r, (rocblas_int)ldb, A, rocblas_datatype_bf16_r, (rocblas_int)lda,
      &beta, C, rocblas_datatype_f32_r, (rocblas_int)ldc, C, rocblas_datatype_f32_r,
      (rocblas_int)ldc, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? hipSuccess : hipErrorUnknown;
}

}  // namespace hstu
