// Shared device helpers of the zgattn HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zg {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kMaxRotPairs = kHeadDim / 2;
constexpr float kLog2e = 1.4426950408889634f;
// Cache-policy operand of the buffer-load builtins on gfx950: the non-temporal (nt) bit, for data read once.
constexpr int kCpolNT = 2;

// 16-byte load of data read once (global_load_dwordx4 ... nt): streaming reads of a large tensor run at ~7.1 TB/s
// non-temporal against ~6.2 TB/s with ordinary loads on MI355X (measured over a 16 GiB buffer).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

// bf16 bit pattern <-> fp32 (bf16 is the top half of an fp32).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two fp32 to bf16 (nearest-even, v_cvt_pk_bf16_f32 on gfx950) and pack (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Round two fp32 to fp16 (nearest-even, v_cvt_pk_f16_f32 on gfx950) and pack (a in the low half).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  half2 h;
  h.x = (_Float16)a;
  h.y = (_Float16)b;
  return __builtin_bit_cast(uint32_t, h);
}

// fp16's largest finite magnitude.
constexpr float kF16Max = 65504.0f;

// Round two fp32 to fp16 after clamping them to +-65504 (v_med3 then v_cvt_pk_f16_f32): values beyond fp16's range
// saturate instead of becoming infinite.
__device__ __forceinline__ uint32_t pack_f16_sat(float a, float b) {
  return pack_f16(__builtin_amdgcn_fmed3f(a, -kF16Max, kF16Max), __builtin_amdgcn_fmed3f(b, -kF16Max, kF16Max));
}

// 8 bf16 -> 8 fp16, saturating.  Exact for magnitudes in [2^-14, 65504]; below 2^-14 the fp16 subnormal keeps an
// absolute error under 2^-25; above 65504 the value becomes +-65504.  Keys (k_hat = RMSNorm * w_k, so |k_hat_d| <=
// sqrt(128) |w_k,d|) and values enter the fp16 MFMAs through this conversion.  Saturation keeps an out-of-range
// value finite, so a masked key's zero weight never meets an infinity (0 * inf would turn every output of the
// MFMA's column into NaN, earlier queries of the tile included).
__device__ __forceinline__ uint4 bf16x8_to_f16x8(const uint4& w) {
  uint4 r;
  r.x = pack_f16_sat(bf16lo(w.x), bf16hi(w.x));
  r.y = pack_f16_sat(bf16lo(w.y), bf16hi(w.y));
  r.z = pack_f16_sat(bf16lo(w.z), bf16hi(w.z));
  r.w = pack_f16_sat(bf16lo(w.w), bf16hi(w.w));
  return r;
}

// Combine a value with the one held by lane l ^ 32 (the other half of the wave): v_permlane32_swap
// returns {x[l & 31], x[32 + (l & 31)]} in every lane, so both lanes of a pair get bit-identical results.
__device__ __forceinline__ void xor32_pair(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  lo = __builtin_bit_cast(float, (unsigned)r[0]);
  hi = __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  float lo, hi;
  xor32_pair(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float xor32_sum(float x) {
  float lo, hi;
  xor32_pair(x, lo, hi);
  return lo + hi;
}

// Unpack 8 bf16 (one 16-byte load) into fp32.
__device__ __forceinline__ void unpack8(const uint4& w, float* f) {
  f[0] = bf16lo(w.x); f[1] = bf16hi(w.x);
  f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
  f[4] = bf16lo(w.z); f[5] = bf16hi(w.z);
  f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 w;
  w.x = pack_bf16(f[0], f[1]);
  w.y = pack_bf16(f[2], f[3]);
  w.z = pack_bf16(f[4], f[5]);
  w.w = pack_bf16(f[6], f[7]);
  return w;
}

// Rotary angle of pair i at absolute position pos, as (cos, sin).  The angle pos * base^(-2i/R) can
// reach 2.6e5 rad at the 256K context, where an fp32 product loses ~1e-2 rad; the host supplies
// inv_freq_rev[i] = base^(-2i/R) / (2 pi) in fp64, the product and its reduction to one revolution are
// done in fp64, and the reduced fraction (24 bits, ~4e-7 rad) goes through v_sin_f32 / v_cos_f32, which
// take their argument in revolutions.
__device__ __forceinline__ void rope_cs(int64_t pos, double inv_freq_rev, float& c, float& s) {
  double r = (double)pos * inv_freq_rev;
  r = __builtin_amdgcn_fract(r);
  const float rf = (float)r;
  s = __builtin_amdgcn_sinf(rf);
  c = __builtin_amdgcn_cosf(rf);
}

// Rotate the pairs of 8 consecutive dims d0..d0+7 (d0 even) of a row at position pos; pairs at or
// beyond rot_pairs are left alone.  Whole chunks past the rotary dims skip the work.  freq(i) gives
// inv_freq_rev of pair i (from an array, or from registers a kernel holds them in).
template <class Freq>
__device__ __forceinline__ void rope8_f(float* f, int d0, int64_t pos, int rot_pairs, Freq freq) {
  if (d0 >= 2 * rot_pairs) return;
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const int i = d0 / 2 + m;
    float c, s;
    rope_cs(pos, freq(i), c, s);
    if (i >= rot_pairs) { c = 1.0f; s = 0.0f; }
    const float x0 = f[2 * m], x1 = f[2 * m + 1];
    f[2 * m] = x0 * c - x1 * s;
    f[2 * m + 1] = x0 * s + x1 * c;
  }
}
__device__ __forceinline__ void rope8(float* f, int d0, int64_t pos, int rot_pairs, const double* inv_freq_rev) {
  rope8_f(f, d0, pos, rot_pairs, [&](int i) { return inv_freq_rev[i]; });
}

// RMSNorm * w then partial RoPE at position pos, for the 8 dims 8c..8c+7 of a 128-dim row held by a
// group of 16 consecutive lanes (c = lane within the group; every lane of the group must be active), with
// the lane's 8 weights wf already unpacked.  Used for every k_hat (and the decode q_hat), so all kernels
// produce the same bits for the same row.
template <class Freq>
__device__ __forceinline__ void norm_rope8_g16_f(float* f, const float* wf, int c, int64_t pos, float eps,
                                                 int rot_pairs, Freq freq) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e++) ss += f[e] * f[e];
  ss += __shfl_xor(ss, 8);
  ss += __shfl_xor(ss, 4);
  ss += __shfl_xor(ss, 2);
  ss += __shfl_xor(ss, 1);
  const float inv = rsqrtf(ss * (1.0f / kHeadDim) + eps);
#pragma unroll
  for (int e = 0; e < 8; e++) f[e] = f[e] * inv * wf[e];
  rope8_f(f, 8 * c, pos, rot_pairs, freq);
}
__device__ __forceinline__ void norm_rope8_g16_w(float* f, const float* wf, int c, int64_t pos, float eps,
                                                 int rot_pairs, const double* inv_freq_rev) {
  norm_rope8_g16_f(f, wf, c, pos, eps, rot_pairs, [&](int i) { return inv_freq_rev[i]; });
}
__device__ __forceinline__ void norm_rope8_g16(float* f, const uint16_t* w, int c, int64_t pos, float eps,
                                               int rot_pairs, const double* inv_freq_rev) {
  float wf[8];
  unpack8(*reinterpret_cast<const uint4*>(w + 8 * c), wf);
  norm_rope8_g16_w(f, wf, c, pos, eps, rot_pairs, inv_freq_rev);
}

}  // namespace zg
