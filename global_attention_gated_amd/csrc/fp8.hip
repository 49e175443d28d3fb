// FP8 (E4M3) quantisation with delayed scaling for the projections around the core (onedev.kr "What
// differs": the model's matmuls run in FP8, E4M3 in the forward pass, with delayed scaling over a 1,024-step
// amax history, the Transformer Engine recipe).
//
// Per tensor the state keeps a history of the last H amax values (max |x| of a call) and the scale in use,
// s = 448 / max(history) (1 while the history is all zero; 448 is E4M3's largest finite value).  A call
// quantises with the current s (codes = E4M3(x * s), nearest-even, saturating at +-448) and records this
// call's amax; after the GEMM the amax goes into the history and the next call's s is derived from it.
// The scale lags the data by one call: that is the "delayed" in delayed scaling.
//
// E4M3 (OCP): sign, 4 exponent bits (bias 7), 3 mantissa bits; normals 2^(e-7) (1 + m/8) for e = 1..15 except
// e = 15, m = 7 (NaN), so the largest finite value is 448; subnormals m 2^-9; no infinities.
#include "common.h"
#include "launch.h"

namespace zg {
namespace {

// E4M3 codes of 8 bf16 values times s: the product clamped to +-448 (v_med3) and converted by v_cvt_pk_fp8_f32
// (nearest-even into OCP E4M3), which together give the saturating nearest-even code.  Raises m to max |x|.
__device__ __forceinline__ uint2 e4m3x8(uint4 w, float s, float& m) {
  float f[8];
  unpack8(w, f);
  uint32_t out[2];
#pragma unroll
  for (int d = 0; d < 2; d++) {
    float a[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      m = fmaxf(m, fabsf(f[4 * d + e]));
      a[e] = __builtin_amdgcn_fmed3f(f[4 * d + e] * s, -448.0f, 448.0f);
    }
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a[0], a[1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(a[2], a[3], r, true);
    out[d] = (uint32_t)r;
  }
  return make_uint2(out[0], out[1]);
}

// Quantise n bf16 values (n8 = n / 8 groups of 8) with the scale in *scale: codes = E4M3(x * s).  Grid stride,
// two groups in flight per lane, every access a lane-contiguous 16-byte load / 8-byte store.  Each work-group
// writes the max |x| of what it covered to partial[blockIdx.x] (no atomics: a same-address atomic per wave
// serialises at the L2); the finalize kernel reduces the partials.
__global__ void __launch_bounds__(256) fp8_quantize_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                                                          int64_t n8, const float* __restrict__ scale,
                                                          float* __restrict__ partial) {
  const float s = *scale;
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint2* qv = reinterpret_cast<uint2*>(q);
  for (; u + stride < n8; u += 2 * stride) {
    const uint4 a = load_nt16(xv + u), b = load_nt16(xv + u + stride);
    qv[u] = e4m3x8(a, s, m);
    qv[u + stride] = e4m3x8(b, s, m);
  }
  if (u < n8) qv[u] = e4m3x8(xv[u], s, m);
  __shared__ float red[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// After a call: reduce each quantised tensor's partial maxima (nb.n[t] of them) to this call's amax, push it into
// the tensor's history (slot idx), and derive the next scale s = 448 / max(history) (1 if the history is all
// zero) and its inverse (the GEMM's dequantisation factor).  One work-group per tensor; a tensor with
// nb.n[t] = 0 was not quantised in this call and keeps its state.
__global__ void __launch_bounds__(256) fp8_finalize_kernel(Fp8State st, int32_t idx, Fp8Blocks nb) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < kFp8MaxTensors; i++)
    if (i == t) cnt = nb.n[i];
  if (cnt == 0) return;
  const float* part = st.partial + (int64_t)t * kFp8MaxBlocks;
  float* hist = st.hist + (int64_t)t * st.H;
  float m = 0.f;
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) m = fmaxf(m, part[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) hist[idx] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  m = 0.f;
  for (int i = threadIdx.x; i < st.H; i += blockDim.x) m = fmaxf(m, hist[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float mm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = mm > 0.f ? 448.0f / mm : 1.0f;
    st.scale[t] = sc;
    st.scale_inv[t] = 1.0f / sc;
  }
}

}  // namespace

int32_t fp8_quantize_blocks(int64_t n) {
  const int64_t b = (n / 8 + 255) / 256;
  return (int32_t)(b < 1 ? 1 : (b > kFp8MaxBlocks ? kFp8MaxBlocks : b));
}

hipError_t launch_fp8_quantize(const uint16_t* x, uint8_t* q, int64_t n, const float* scale, float* partial,
                               hipStream_t st) {
  hipLaunchKernelGGL(fp8_quantize_kernel, dim3((unsigned)fp8_quantize_blocks(n)), dim3(256), 0, st, x, q, n / 8,
                     scale, partial);
  return hipGetLastError();
}

hipError_t launch_fp8_finalize(const Fp8State& s, int32_t idx, const Fp8Blocks& nb, hipStream_t st) {
  hipLaunchKernelGGL(fp8_finalize_kernel, dim3((unsigned)s.n), dim3(256), 0, st, s, idx, nb);
  return hipGetLastError();
}

}  // namespace zg
