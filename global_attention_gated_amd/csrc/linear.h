// Internal interface of the hipBLASLt projections (linear.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zg {

// y[T][N] = x[T][K] . W[N][K]^T, bf16 in/out, fp32 accumulation; returns a hipblasStatus_t value (0 = success).
int linear_bf16_run(const void* x, const void* w, void* y, int64_t T, int32_t K, int32_t N, hipStream_t st);
const char* blas_status_name(int s);

}  // namespace zg
