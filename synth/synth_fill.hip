// GPU side of the seeded synthetic-input generator (input generation only).
//
// dst[o * dst_outer_stride + i] = table[splitmix64_output(key, idx_start + o * idx_outer_stride + i) >> 48]
// for o < n_outer, i < n_inner, where splitmix64_output(k, n) is the n-th (0-based) output of a
// SplitMix64 generator seeded with k (Steele, Lea and Flood, OOPSLA 2014).  The table and the key
// come from the host (synth/__init__.py), so both sides produce the same bits.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

__device__ __forceinline__ uint64_t splitmix_out(uint64_t key, uint64_t n) {
  uint64_t z = key + (n + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Each thread writes 8 consecutive elements (16 bytes) when the run allows it.
__global__ void __launch_bounds__(256) fill_kernel(uint16_t* __restrict__ dst, int64_t n_outer, int64_t n_inner,
                                                   int64_t dst_outer_stride, uint64_t key, int64_t idx_start,
                                                   int64_t idx_outer_stride, const uint16_t* __restrict__ table) {
  const int64_t chunks_per_row = (n_inner + 7) / 8;
  const int64_t total = n_outer * chunks_per_row;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t o = c / chunks_per_row;
    const int64_t i0 = (c - o * chunks_per_row) * 8;
    const int64_t base_idx = idx_start + o * idx_outer_stride + i0;
    uint16_t* p = dst + o * dst_outer_stride + i0;
    const int64_t cnt = (n_inner - i0) < 8 ? (n_inner - i0) : 8;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; e++) v[e] = table[splitmix_out(key, (uint64_t)(base_idx + e)) >> 48];
    if (cnt == 8 && ((reinterpret_cast<uintptr_t>(p) & 15) == 0)) {
      uint4 w;
      w.x = v[0] | ((uint32_t)v[1] << 16);
      w.y = v[2] | ((uint32_t)v[3] << 16);
      w.z = v[4] | ((uint32_t)v[5] << 16);
      w.w = v[6] | ((uint32_t)v[7] << 16);
      *reinterpret_cast<uint4*>(p) = w;
    } else {
      for (int e = 0; e < cnt; e++) p[e] = v[e];
    }
  }
}

}  // namespace

extern "C" int synth_fill_bf16(void* dst, int64_t n_outer, int64_t n_inner, int64_t dst_outer_stride, uint64_t key,
                               int64_t idx_start, int64_t idx_outer_stride, const void* table, void* stream) {
  if (!dst || !table || n_outer < 0 || n_inner < 0 || idx_start < 0) return 1;
  if (n_outer == 0 || n_inner == 0) return 0;
  const int64_t chunks = n_outer * ((n_inner + 7) / 8);
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (uint16_t*)dst, n_outer,
                     n_inner, dst_outer_stride, key, idx_start, idx_outer_stride, (const uint16_t*)table);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
