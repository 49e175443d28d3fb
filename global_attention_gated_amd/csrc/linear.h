// Internal interface of the hipBLASLt projections (linear.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zg {

// y[T][N] = x[T][K] . W[N][K]^T, bf16 in/out, fp32 accumulation; returns a hipblasStatus_t value (0 = success).
int linear_bf16_run(const void* x, const void* w, void* y, int64_t T, int32_t K, int32_t N, hipStream_t st);
// y[T][N] = (xq[T][K] . wq[N][K]^T) * (*x_scale_inv) * (*w_scale_inv) with E4M3 operands (OCP), fp32
// accumulation, bf16 result; the scale factors are device fp32 scalars read when the GEMM runs.
int linear_fp8_run(const void* xq, const void* wq, void* y, int64_t T, int32_t K, int32_t N, const float* x_scale_inv,
                   const float* w_scale_inv, hipStream_t st);
const char* blas_status_name(int s);

}  // namespace zg
