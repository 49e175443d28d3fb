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

// fp32 -> E4M3 code, nearest-even, saturating at +-448 (finite inputs).  Works on the fp32 bits: the three
// kept mantissa bits are rounded on the 20 dropped ones; a carry out of the mantissa moves into the exponent
// field of the code, which is the correct next binade.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7E;                                        // saturate
  } else if (a < 0.015625f) {                          // below 2^-6: multiples of 2^-9 (the scaling is exact)
    mag = (uint32_t)__builtin_rintf(a * 512.0f);       // 0..8 (8 is the smallest normal, code 0x08)
  } else {
    const uint32_t ua = u & 0x7fffffffu;
    const int e = (int)(ua >> 23) - 127;               // -6 .. 8
    uint32_t q = (ua >> 20) & 7u;
    const uint32_t rem = ua & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q += 1;
    mag = ((uint32_t)(e + 7) << 3) + q;
    if (mag > 0x7Eu) mag = 0x7E;
  }
  return sign | mag;
}

// Quantise n bf16 values (n a multiple of 8) with the scale in *scale; atomically raise *amax (fp32 bits, a
// non-negative float compares like its bits) to this tensor's max |x|.
__global__ void __launch_bounds__(256) fp8_quantize_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                                                          int64_t n8, const float* __restrict__ scale,
                                                          uint32_t* __restrict__ amax) {
  const float s = *scale;
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(x + 8 * i), f);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      m = fmaxf(m, fabsf(f[e]));
      lo |= e4m3_code(f[e] * s) << (8 * e);
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
      m = fmaxf(m, fabsf(f[4 + e]));
      hi |= e4m3_code(f[4 + e] * s) << (8 * e);
    }
    *reinterpret_cast<uint2*>(q + 8 * i) = make_uint2(lo, hi);
  }
  // wave max, then one atomic per wave
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) atomicMax(amax, __float_as_uint(m));
}

// After a call: push each tensor's amax into its history (slot idx), clear it, and derive the next scale
// s = 448 / max(history) (1 if the history is all zero) and its inverse (the GEMM's dequantisation factor).
// One work-group; state layout as Fp8State.
__global__ void __launch_bounds__(256) fp8_finalize_kernel(Fp8State st, int32_t idx) {
  __shared__ float red[2][4];
  for (int t = 0; t < 2; t++) {
    float* hist = st.hist + (int64_t)t * st.H;
    if (threadIdx.x == 0) hist[idx] = __uint_as_float(st.amax[t]);
    __syncthreads();
    float m = 0.f;
    for (int i = threadIdx.x; i < st.H; i += blockDim.x) m = fmaxf(m, hist[i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) red[t][threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      const float mm = fmaxf(fmaxf(red[t][0], red[t][1]), fmaxf(red[t][2], red[t][3]));
      const float s = mm > 0.f ? 448.0f / mm : 1.0f;
      st.scale[t] = s;
      st.scale_inv[t] = 1.0f / s;
      st.amax[t] = 0u;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_fp8_quantize(const uint16_t* x, uint8_t* q, int64_t n, const float* scale, uint32_t* amax,
                               hipStream_t st) {
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fp8_quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, q, n8, scale, amax);
  return hipGetLastError();
}

hipError_t launch_fp8_finalize(const Fp8State& s, int32_t idx, hipStream_t st) {
  hipLaunchKernelGGL(fp8_finalize_kernel, dim3(1), dim3(256), 0, st, s, idx);
  return hipGetLastError();
}

}  // namespace zg
