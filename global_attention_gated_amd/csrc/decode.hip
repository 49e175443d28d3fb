// Decode kernels of the ZGCM-1 attention core for gfx950: one new token per sequence in every layer.
//
//   decode_append_kernel  k_hat = RoPE(RMSNorm(k) * w_k) at the token's position, written with raw v to
//                         ring slot p mod W (SWA layers) or row p (global layers): append before attend.
//   decode_attn_kernel    one work-group streams a range of cache rows of one (layer, sequence, KV head)
//                         for the G query heads of the group.  GLOBAL: a split-K chunk of the full cache,
//                         written as fp32 partials (running max, sum, unnormalised output).  SWA: the
//                         whole W-slot ring, validity by position, output gated by sigmoid(g).
//   decode_merge_kernel   log-sum-exp merge of the partials of each global (layer, sequence, KV head).
//
// Decoding reads every cached key and value once and does ~4 flop per byte, so it is bound by HBM
// bandwidth (onedev.kr "How it works": autoregressive decoding is memory-bandwidth bound).  The kernels
// use VALU, not MFMA: 16 lanes hold one 256-byte key row (8 dims each, 16-byte loads), one row read
// serves the G query heads of the group, and v_dot2_f32_bf16 forms the partial dot products.
#include "common.h"
#include "launch.h"

namespace zg {
namespace {

__device__ __forceinline__ float dot8(const uint4& k, const uint32_t* q, float d) {
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.x), __builtin_bit_cast(bf16x2, q[0]), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.y), __builtin_bit_cast(bf16x2, q[1]), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.z), __builtin_bit_cast(bf16x2, q[2]), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.w), __builtin_bit_cast(bf16x2, q[3]), d, false);
  return d;
}

// Sum over each row of 16 lanes, result in every lane of the row: DPP row rotations by 8, 4, 2, 1 (no LDS
// crossbar traffic).
__device__ __forceinline__ float ror16(float x, int n) {
  switch (n) {
    case 8: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
    case 4: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
    case 2: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  }
}
__device__ __forceinline__ float sum16(float x) {
  x += ror16(x, 8);
  x += ror16(x, 4);
  x += ror16(x, 2);
  x += ror16(x, 1);
  return x;
}

// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) decode_append_kernel(DecodeArgs a) {
  const int c = threadIdx.x & 15;
  const int64_t n_rows = (int64_t)a.L * a.B * a.Hkv;
  const int64_t row_raw = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool valid = row_raw < n_rows;
  const int64_t row = valid ? row_raw : n_rows - 1;
  const int h = (int)(row % a.Hkv);
  const int b = (int)((row / a.Hkv) % a.B);
  const int l = (int)(row / ((int64_t)a.Hkv * a.B));
  const int64_t p = a.pos[b];
  float f[8];
  unpack8(*reinterpret_cast<const uint4*>(a.k + row * kHeadDim + 8 * c), f);
  norm_rope8_g16(f, a.kw + (int64_t)l * kHeadDim, c, p, a.eps, a.rot_pairs, a.inv_freq_rev);
  if (valid) {
    const LayerDesc ld = a.layers[l];
    const int64_t slot = ld.is_global ? p : p % a.W;
    const int64_t off = (((int64_t)b * a.Hkv + h) * ld.slots + slot) * kHeadDim + 8 * c;
    *reinterpret_cast<uint4*>(ld.k + off) = pack8(f);
    *reinterpret_cast<uint4*>(ld.v + off) = *reinterpret_cast<const uint4*>(a.v + row * kHeadDim + 8 * c);
  }
}

// ---------------------------------------------------------------------------------------------
// 256 threads = 16 groups of 16 lanes; group g takes rows r0 + g, r0 + g + 16, ...; every group keeps
// its own online-softmax state for the G heads and the groups are merged through LDS at the end.
template <int G, bool GLOBAL>
__global__ void __launch_bounds__(256) decode_attn_kernel(DecodeArgs a, int32_t chunks) {
  __shared__ float sm_m[16][G];
  __shared__ float sm_l[16][G];
  __shared__ float sm_acc[16][G][kHeadDim];

  const int tid = threadIdx.x;
  const int c = tid & 15, g = tid >> 4;
  int layer, b, h, chunk = 0;
  {
    int wg = blockIdx.x;
    if (GLOBAL) { chunk = wg % chunks; wg /= chunks; }
    h = wg % a.Hkv;
    wg /= a.Hkv;
    b = wg % a.B;
    const int li = wg / a.B;
    layer = GLOBAL ? a.glob_ids[li] : a.swa_ids[li];
  }
  const int64_t p = a.pos[b];
  const LayerDesc ld = a.layers[layer];
  int64_t r0, r1;   // cache rows [r0, r1)
  if (GLOBAL) {
    r0 = (int64_t)chunk * kDecodeChunk;
    r1 = r0 + kDecodeChunk;
    if (r1 > p + 1) r1 = p + 1;
    if (r0 >= r1) return;   // this sequence needs fewer chunks (uniform over the work-group)
  } else {
    r0 = 0;
    r1 = a.W;
  }

  // q_hat of the G heads, scaled by log2(e)/sqrt(D), as a bf16 pair hi + lo (lo = bf16 of the residual):
  // two v_dot2_f32_bf16 per pair of dims carry q_hat to ~16 significant bits against the bf16 keys.
  uint32_t qhi[G][4], qlo[G][4];
#pragma unroll
  for (int hh = 0; hh < G; hh++) {
    float f[8];
    const int64_t qrow = ((int64_t)layer * a.B + b) * a.Hq + h * G + hh;
    unpack8(*reinterpret_cast<const uint4*>(a.q + qrow * kHeadDim + 8 * c), f);
    norm_rope8_g16(f, a.qw + (int64_t)layer * kHeadDim, c, p, a.eps, a.rot_pairs, a.inv_freq_rev);
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float x0 = f[2 * e] * a.q_scale, x1 = f[2 * e + 1] * a.q_scale;
      qhi[hh][e] = pack_bf16(x0, x1);
      qlo[hh][e] = pack_bf16(x0 - bf16lo(qhi[hh][e]), x1 - bf16hi(qhi[hh][e]));
    }
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; hh++) {
    m[hh] = -1e30f;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) acc[hh][e] = 0.f;
  }

  // buffer descriptors over this (sequence, KV head)'s rows r0..r1-1 (uniform); lanes add byte offsets
  const int64_t plane = ((int64_t)b * a.Hkv + h) * ld.slots + r0;
  const int nbytes = (int)((r1 - r0) * kHeadDim * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(ld.k + plane * kHeadDim), (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(ld.v + plane * kHeadDim), (short)0, nbytes, 0x00020000);

  constexpr int U = 2;   // rows per group and block
  // software pipeline: the next block's rows are loaded while this block computes
  uint4 kw[U], vw[U];
  auto load_block = [&](int64_t rb, uint4 (&kd)[U], uint4 (&vd)[U]) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      // rows past r1 fall outside the descriptor and read as zero (masked below)
      // non-temporal (nt): the rows are read once; measured, such streaming reads reach 7.1 TB/s against 6.2 without
      const int off = (int)((rb + 16 * u - r0) * kHeadDim + 8 * c) * 2;
      kd[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kCpolNT));
      vd[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kCpolNT));
    }
  };
  load_block(r0 + g, kw, vw);
  for (int64_t rb = r0 + g; rb < r1; rb += 16 * U) {
    uint4 kn[U], vn[U];
    load_block(rb + 16 * U, kn, vn);
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int64_t row = rb + 16 * u;
      ok[u] = row < r1;
      if (!GLOBAL && ok[u]) {
        // ring slot `row` holds position p - ((p - row) mod W); negative positions were never written
        const int64_t back = ((p - row) % a.W + a.W) % a.W;
        ok[u] = p - back >= 0;
      }
    }
    // scores of the U rows, then one running-max check for the block (lazy: the max is raised only when a
    // score exceeds it by more than 2^8, which keeps p <= 256 and the result exact)
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
      for (int hh = 0; hh < G; hh++) {
        const float x = sum16(dot8(kw[u], qhi[hh], dot8(kw[u], qlo[hh], 0.f)));
        s[u][hh] = ok[u] ? x : -INFINITY;
      }
    float bmax[G];
    bool need = false;
#pragma unroll
    for (int hh = 0; hh < G; hh++) {
      bmax[hh] = s[0][hh];
#pragma unroll
      for (int u = 1; u < U; u++) bmax[hh] = fmaxf(bmax[hh], s[u][hh]);
      need = need || (bmax[hh] > m[hh] + 8.0f);
    }
    if (__any(need)) {
#pragma unroll
      for (int hh = 0; hh < G; hh++) {
        const bool nd = bmax[hh] > m[hh] + 8.0f;
        const float alpha = nd ? __builtin_amdgcn_exp2f(m[hh] - bmax[hh]) : 1.0f;
        m[hh] = nd ? bmax[hh] : m[hh];
        l[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; e++) acc[hh][e] *= alpha;
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      float vf[8];
      unpack8(vw[u], vf);
#pragma unroll
      for (int hh = 0; hh < G; hh++) {
        const float pr = __builtin_amdgcn_exp2f(s[u][hh] - m[hh]);
        l[hh] += pr;
#pragma unroll
        for (int e = 0; e < 8; e++) acc[hh][e] += pr * vf[e];
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) { kw[u] = kn[u]; vw[u] = vn[u]; }
  }

  // merge the 16 groups
#pragma unroll
  for (int hh = 0; hh < G; hh++) {
    if (c == 0) {
      sm_m[g][hh] = m[hh];
      sm_l[g][hh] = l[hh];
    }
#pragma unroll
    for (int e = 0; e < 8; e++) sm_acc[g][hh][8 * c + e] = acc[hh][e];
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += 256) {
    const int hh = idx / kHeadDim, d = idx % kHeadDim;
    float M = -1e30f;
#pragma unroll
    for (int gg = 0; gg < 16; gg++) M = fmaxf(M, sm_m[gg][hh]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int gg = 0; gg < 16; gg++) {
      const float w = __builtin_amdgcn_exp2f(sm_m[gg][hh] - M);
      L += sm_l[gg][hh] * w;
      A += sm_acc[gg][hh][d] * w;
    }
    if (GLOBAL) {
      const int li = blockIdx.x / chunks / a.Hkv / a.B;
      const int64_t pidx = ((((int64_t)li * a.B + b) * a.Hkv + h) * a.max_chunks + chunk) * G + hh;
      a.part_acc[pidx * kHeadDim + d] = A;
      if (d == 0) {
        a.part_m[pidx] = M;
        a.part_l[pidx] = L;
      }
    } else {
      const int64_t orow = ((int64_t)layer * a.B + b) * a.Hq + h * G + hh;
      const float gt = bf16lo(a.gate[orow * kHeadDim + d]);
      const float o = (A / L) * (1.0f / (1.0f + __expf(-gt)));
      a.out[orow * kHeadDim + d] = (uint16_t)(pack_bf16(o, 0.f) & 0xffffu);
    }
  }
}

// ---------------------------------------------------------------------------------------------
template <int G>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeArgs a) {
  int wg = blockIdx.x;
  const int h = wg % a.Hkv;
  wg /= a.Hkv;
  const int b = wg % a.B;
  const int li = wg / a.B;
  const int layer = a.glob_ids[li];
  const int64_t p = a.pos[b];
  const int n = (int)((p + 1 + kDecodeChunk - 1) / kDecodeChunk);
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256) {
    const int hh = idx / kHeadDim, d = idx % kHeadDim;
    const int64_t base = (((int64_t)li * a.B + b) * a.Hkv + h) * a.max_chunks;
    float M = -1e30f;
    for (int ch = 0; ch < n; ch++) M = fmaxf(M, a.part_m[(base + ch) * G + hh]);
    float L = 0.f, A = 0.f;
    for (int ch = 0; ch < n; ch++) {
      const int64_t pidx = (base + ch) * G + hh;
      const float w = __builtin_amdgcn_exp2f(a.part_m[pidx] - M);
      L += a.part_l[pidx] * w;
      A += a.part_acc[pidx * kHeadDim + d] * w;
    }
    const int64_t orow = ((int64_t)layer * a.B + b) * a.Hq + h * G + hh;
    a.out[orow * kHeadDim + d] = (uint16_t)(pack_bf16(A / L, 0.f) & 0xffffu);
  }
}

template <bool GLOBAL>
hipError_t launch_attn(const DecodeArgs& a, int32_t chunks, hipStream_t st) {
  const int64_t units = (int64_t)(GLOBAL ? a.n_global : a.n_swa) * a.B * a.Hkv;
  const int64_t blocks = units * (GLOBAL ? chunks : 1);
  if (blocks == 0) return hipSuccess;
  switch (a.G) {
    case 1: hipLaunchKernelGGL((decode_attn_kernel<1, GLOBAL>), dim3((unsigned)blocks), dim3(256), 0, st, a, chunks); break;
    case 2: hipLaunchKernelGGL((decode_attn_kernel<2, GLOBAL>), dim3((unsigned)blocks), dim3(256), 0, st, a, chunks); break;
    case 4: hipLaunchKernelGGL((decode_attn_kernel<4, GLOBAL>), dim3((unsigned)blocks), dim3(256), 0, st, a, chunks); break;
    case 8: hipLaunchKernelGGL((decode_attn_kernel<8, GLOBAL>), dim3((unsigned)blocks), dim3(256), 0, st, a, chunks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_append(const DecodeArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.L * a.B * a.Hkv;
  hipLaunchKernelGGL(decode_append_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode_swa(const DecodeArgs& a, hipStream_t st) { return launch_attn<false>(a, 1, st); }

hipError_t launch_decode_global(const DecodeArgs& a, int32_t chunks, hipStream_t st) {
  return launch_attn<true>(a, chunks, st);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t st) {
  const int64_t blocks = (int64_t)a.n_global * a.B * a.Hkv;
  if (blocks == 0) return hipSuccess;
  switch (a.G) {
    case 1: hipLaunchKernelGGL(decode_merge_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(decode_merge_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(decode_merge_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL(decode_merge_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace zg
