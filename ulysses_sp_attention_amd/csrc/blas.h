// The vendor GEMM behind the plain dense products of the language-model loss
// and the tiled MLP (rocBLAS gemm_ex, bf16 operands, fp32 arithmetic).
#pragma once

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

namespace ulysses {

// One rocBLAS handle per host thread and device, made on first use with that
// device current (calls on one handle from two threads would race on its
// stream) and kept.  Split-K atomics are off, so every product is a fixed
// sequence of operations and results are bitwise reproducible.
inline rocblas_handle blas_handle() {
  thread_local rocblas_handle handles[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (!handles[dev]) {
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
    if (rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed) != rocblas_status_success) {
      rocblas_destroy_handle(h);
      return nullptr;
    }
    handles[dev] = h;
  }
  return handles[dev];
}

// Column-major D = op(A) op(B) + beta D, m x n, inner size k, with bf16 A and
// B and fp32 arithmetic; D is fp32 or bf16 (d_bf16).
inline bool gemm_bf16(rocblas_handle hd, bool ta, bool tb, int64_t m, int64_t n, int64_t k,
                      const void* a, int64_t lda, const void* b, int64_t ldb, float beta, void* d,
                      bool d_bf16, int64_t ldd) {
  const float alpha = 1.0f;
  const rocblas_datatype dt = d_bf16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  return rocblas_gemm_ex(hd, ta ? rocblas_operation_transpose : rocblas_operation_none,
                         tb ? rocblas_operation_transpose : rocblas_operation_none, (rocblas_int)m,
                         (rocblas_int)n, (rocblas_int)k, &alpha, a, rocblas_datatype_bf16_r,
                         (rocblas_int)lda, b, rocblas_datatype_bf16_r, (rocblas_int)ldb, &beta, d,
                         dt, (rocblas_int)ldd, d, dt, (rocblas_int)ldd, rocblas_datatype_f32_r,
                         rocblas_gemm_algo_standard, 0, 0) == rocblas_status_success;
}

}  // namespace ulysses
