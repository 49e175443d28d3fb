// Tile-path prefill of the ZGCM-1 attention core for gfx950 (CDNA4, wave64, MFMA): every prefill that the streaming
// gated-SWA kernel does not take -- global layers (one-shot, chunked against the KV cache, the training forward) and
// gated layers of other GQA groups or windows above 128 (with or without a cache).
//
//   kv_stage_kernel    writes the keys and values a call attends to, once, as fp16 tiles in the layout that the
//                      attention kernel copies into LDS unchanged: k_hat = RoPE(RMSNorm(k) w_k) of the chunk's own
//                      tokens (rounded to bf16, the KV-cache value; a global layer with a cache also stores it and v
//                      in the cache rows of those positions), the earlier positions read back from the cache (the
//                      global layer's rows or the gated layer's ring), and v^T.
//   attn_pp_kernel     flash-style attention of 256 query rows (G heads x 2P positions of one KV head) per
//                      work-group against 64-key tiles: causal (global layer) or within the window W (gated layer,
//                      whose epilogue multiplies by sigmoid(gate)).  Each tile goes from the workspace straight into
//                      LDS (buffer loads with LDS as the destination: no registers, no LDS write instructions), 16 KB
//                      of keys and 16 KB of transposed values.  A direct load writes 16 bytes per lane at
//                      consecutive LDS addresses; the lanes choose their source chunks so that the LDS rows come out
//                      XOR-swizzled, which keeps the MFMA operand reads free of bank conflicts without padding.
//   ring_write_kernel  after a gated chunk with a cache, its last min(S, W) keys and values go to ring slot p mod W.
//
// Method (ZGCM-1 paper summaries: onedev.kr "How it works"; jaehun.me "How Gated SWA Behaves"): per (token, head)
// q_hat = RoPE(RMSNorm(q) w_q), k_hat likewise; the global output is softmax_{j <= i}(q_hat k_hat_j / sqrt(D)) v_j,
// the gated output softmax_{i-W < j <= i}(...) v_j (.) sigmoid(g).  Positions are absolute: a chunk's queries at
// pos0 .. pos0+S-1 see the cached keys of earlier positions.
//
// Precision: k_hat and v are bf16 values held exactly in fp16 (saturating at +-65504), q_hat and P are rounded
// once to fp16, the MFMAs accumulate in fp32, and the online softmax runs in fp32.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace zg {
namespace {

constexpr int kBN = 64;                          // keys per tile
constexpr int kTileHalves = kBN * kHeadDim;      // 8192 fp16 = 16 KB: one K tile, or one V^T tile
constexpr int kOsStride = 132;                   // floats per output row staged in LDS (epilogue): 128 + 4 pad
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);   // s_waitcnt vmcnt(0), other counters not waited for

typedef __attribute__((address_space(3))) void lds_void;

// ------------------------------------------------------------------------------------------------ staging
// One work-group per (sequence, KV head, 64-row tile).  Staged row r holds position kbase + r: from the chunk's
// input (pos0 <= p < pos0 + S), from the cache (p < pos0), zero past the chunk (padding of the last tile).
__global__ void __launch_bounds__(256) kv_stage_kernel(StageArgs a) {
  const int tid = threadIdx.x;
  const int n_tiles = a.S_kpad / kBN;
  const int unit = blockIdx.x / n_tiles, tile = blockIdx.x % n_tiles;
  const int b = unit / a.Hkv, h = unit % a.Hkv;
  const int64_t row_b = (int64_t)b * a.S;                                      // input row (b, s, h): (row_b + s) * Hkv + h
  const int64_t cbase = ((int64_t)b * a.Hkv + h) * a.slots * kHeadDim;        // cache rows of (b, h)
  const int p0 = a.kbase + tile * kBN;                                          // position of the tile's row 0
  const int pend = a.pos0 + a.S;
  auto cache_row = [&](int p) -> int64_t {   // element offset of position p's row in the cache (ring: slot p mod W)
    const int64_t slot = a.ring ? (int64_t)(p % a.slots) : (int64_t)p;
    return cbase + slot * kHeadDim;
  };
  // k_hat: a 16-lane group per key row (rows g, g + 16, g + 32, g + 48), 8 dims per lane.  Every lane runs the
  // norm on a chunk row (clamped), so the group's exchanges never meet inactive lanes; the row's source selects.
  {
    const int c = tid & 15, g = tid >> 4;
    uint16_t* dst = a.kt + ((int64_t)unit * a.S_kpad + (int64_t)tile * kBN) * kHeadDim + 8 * c;
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      const int r = g + 16 * rr, p = p0 + r;
      const int sc = min(max(p - a.pos0, 0), a.S - 1);
      float f[8];
      unpack8(load_nt16(a.k + ((row_b + sc) * a.Hkv + h) * kHeadDim + 8 * c), f);
      norm_rope8_g16(f, a.kw, c, a.pos0 + sc, a.eps, a.rot_pairs, a.inv_freq_rev);
      uint4 kb = pack8(f);   // the KV-cache value of k_hat (bf16, nearest-even)
      if (p >= a.pos0 && p < pend) {
        if (a.dk) *reinterpret_cast<uint4*>(a.dk + cache_row(p) + 8 * c) = kb;
      } else if (p < a.pos0) {
        kb = load_nt16(a.ck + cache_row(p) + 8 * c);
      } else {
        kb = make_uint4(0u, 0u, 0u, 0u);
      }
      *reinterpret_cast<uint4*>(dst + (int64_t)r * kHeadDim) = bf16x8_to_f16x8(kb);
    }
  }
  // v^T: thread (vq, vd) turns keys 4vq..4vq+3 x dims 8vd..8vd+7 into 8 dim rows of 4 keys (v_perm pairs the
  // 16-bit halves); the 4 keys go to quad slot perm(vq mod 4) of their 16-key group, perm = (0, 2, 1, 3)
  {
    const int vq = tid & 15, vd = tid >> 4;
    uint32_t w[4][4];
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      const int p = p0 + 4 * vq + rr;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (p >= a.pos0 && p < pend) {
        x = load_nt16(a.v + ((row_b + (p - a.pos0)) * a.Hkv + h) * kHeadDim + 8 * vd);
        if (a.dv) *reinterpret_cast<uint4*>(a.dv + cache_row(p) + 8 * vd) = x;
      } else if (p < a.pos0) {
        x = load_nt16(a.cv + cache_row(p) + 8 * vd);
      }
      x = bf16x8_to_f16x8(x);
      w[rr][0] = x.x; w[rr][1] = x.y; w[rr][2] = x.z; w[rr][3] = x.w;
    }
    const int qin = vq & 3;
    const int col = 16 * (vq >> 2) + 4 * (qin == 1 ? 2 : qin == 2 ? 1 : qin);
    uint16_t* dst = a.vt + ((int64_t)unit * kHeadDim + 8 * vd) * a.S_kpad + (int64_t)tile * kBN + col;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint2 o;
      o.x = __builtin_amdgcn_perm(w[1][e >> 1], w[0][e >> 1], sel);
      o.y = __builtin_amdgcn_perm(w[3][e >> 1], w[2][e >> 1], sel);
      *reinterpret_cast<uint2*>(dst + (int64_t)e * a.S_kpad) = o;
    }
  }
}

// ------------------------------------------------------------------------------------------------ ring write
// After a gated chunk with a cache: k_hat (recomputed from k, bit-identical to the staging's) and raw v of the
// chunk's last n rows go to ring slot (position mod W).  One 16-lane group per row.
__global__ void __launch_bounds__(256) ring_write_kernel(RingWriteArgs a) {
  const int c = threadIdx.x & 15;
  const int64_t n_rows = (int64_t)a.B * a.Hkv * a.n;
  const int64_t row_raw = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool valid = row_raw < n_rows;
  const int64_t row = valid ? row_raw : n_rows - 1;
  const int j = (int)(row % a.n);
  const int h = (int)((row / a.n) % a.Hkv);
  const int64_t b = row / ((int64_t)a.n * a.Hkv);
  const int64_t s = a.S - a.n + j;
  const int64_t src = ((b * a.S + s) * a.Hkv + h) * kHeadDim + 8 * c;
  float f[8];
  unpack8(*reinterpret_cast<const uint4*>(a.k + src), f);
  norm_rope8_g16(f, a.kw, c, a.pos0 + s, a.eps, a.rot_pairs, a.inv_freq_rev);
  if (valid) {
    const int64_t slot = (a.pos0 + s) % a.W;
    const int64_t dst = ((b * a.Hkv + h) * a.W + slot) * kHeadDim + 8 * c;
    *reinterpret_cast<uint4*>(a.kring + dst) = pack8(f);
    *reinterpret_cast<uint4*>(a.vring + dst) = *reinterpret_cast<const uint4*>(a.v + src);
  }
}

// ------------------------------------------------------------------------------------------------ attention
// Rows: wave w owns query rows 32w..32w+31 of the work-group's 256 (row r -> head r / 2P, position i0 + r % 2P).
// S^T = K Q^T puts one query per lane column (MFMA 32x32x16, keys as the A rows), so the softmax statistics of a
// query live in lanes l and l + 32 only, and O^T = V^T P^T keeps the output in the same layout.
//
// LDS tile images (fp16, dense):
//   K   [64 keys][128 dims]: 16-byte chunk c (dims 8c..8c+7) of key row r sits at chunk position c ^ (r mod 16)
//   V^T [128 dims][64 keys]: chunk c (8 stored keys) of dim row r sits at chunk position c ^ ((r / 2) mod 8)
// The MFMA A-operand reads take one chunk from each of 16 consecutive rows per LDS cycle group; the swizzles
// spread those 16 chunks over all 64 banks.
//
// Ping-pong: the 8 waves form two groups of 4 (one wave of each group per SIMD) whose phases alternate: while one group runs its MFMA phase M(m) (P V^T of tile m-1,
// then S^T = K Q^T of tile m) the other runs its softmax phase V (max, exponentials, row sums of its last scores) on
// the VALU, so a SIMD's matrix unit is fed by one wave while the other wave's vector work runs beside it.  Every phase
// ends with one work-group barrier; group 1 runs one phase behind group 0, and each group's straight-line sequence
// meets the same 2n + 2 barriers (n tiles).
//
// LDS: keys and transposed values in separate triple buffers (K[3], V^T[3], 16 KB each), loaded two phases ahead: at
// phase 2m every wave issues its eighth of K(m+2) and of V(m+1) (their buffers' previous tiles, K(m-1) and V(m-2),
// were last read in phase 2m-1) and waits for them at the end of phase 2m+1.  M(m) reads K(m) and V(m-1), which are
// in LDS from the end of phase 2m-1 on, so the softmax phase before it ends by reading M(m)'s first four operand
// fragments into registers: the MFMA phase starts without waiting for LDS.  The loop runs three tiles per pass, so
// every buffer is a compile-time constant and each fragment's LDS address is a per-lane register plus an immediate.
constexpr int kPPRows = 256;
constexpr int kPPSmemBytes = kPPRows * kOsStride * 4;   // 135,168 B: the epilogue staging; the tiles use 96 KB of it
static_assert(6 * kTileHalves * 2 <= kPPSmemBytes, "tile buffers exceed the LDS block");

template <bool GATED>
__global__ void __launch_bounds__(512, 1) attn_pp_kernel(TileAttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kPPSmemBytes / 2];
  // K buffer j at smem + j * kTileHalves, V^T buffer j at smem + (3 + j) * kTileHalves

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int l32 = lane & 31, hi = lane >> 5;

  const int unit = blockIdx.x % a.n_units;
  const int qt = a.n_qtiles - 1 - (int)(blockIdx.x / a.n_units);
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int P2 = 2 * a.P;                         // positions per work-group
  const int i0 = qt * P2;

  const int r = wave * 32 + l32;
  const int hq = kvh * a.G + r / P2;
  const int i = i0 + r % P2;
  const bool qvalid = i < a.S;
  const int ic = qvalid ? i : a.S - 1;
  const int qpos = a.pos0 + ic;

  int pl_lo, pl_hi;
  if (P2 >= 32) { pl_lo = (wave * 32) % P2; pl_hi = pl_lo + 31; } else { pl_lo = 0; pl_hi = P2 - 1; }
  const int wlo = a.pos0 + min(i0 + pl_lo, a.S - 1);
  const int whi = a.pos0 + min(i0 + pl_hi, a.S - 1);
  const int khi = a.pos0 + min(i0 + P2, a.S);
  const int klo = GATED ? max(a.kbase, a.pos0 + i0 - a.window + 1) : a.kbase;
  const int t_lo = (klo - a.kbase) / kBN;
  const int n_tiles = (khi - a.kbase + kBN - 1) / kBN - t_lo;
  const unsigned lim = GATED ? (unsigned)a.window : 0x7fffffffu;

  // ---- Q prologue: q_hat = RoPE(RMSNorm(q) w_q), scaled by log2(e)/sqrt(D), fp16; lane (l32, hi) holds dims
  // 16t + 8hi .. +7 of its row for k-step t
  half8 qf[8];
  {
    const uint16_t* qrow = a.q + (((int64_t)b * a.S + ic) * a.Hq + hq) * kHeadDim;
    float f[8][8];
    float ss = 0.f;
#pragma unroll
    for (int t = 0; t < 8; t++) {
      unpack8(*reinterpret_cast<const uint4*>(qrow + 16 * t + 8 * hi), f[t]);
#pragma unroll
      for (int e = 0; e < 8; e++) ss += f[t][e] * f[t][e];
    }
    ss = xor32_sum(ss);
    const float inv = rsqrtf(ss * (1.0f / kHeadDim) + a.eps);
#pragma unroll
    for (int t = 0; t < 8; t++) {
      float w[8];
      unpack8(*reinterpret_cast<const uint4*>(a.qw + 16 * t + 8 * hi), w);
#pragma unroll
      for (int e = 0; e < 8; e++) f[t][e] = f[t][e] * inv * w[e];
      rope8(f[t], 16 * t + 8 * hi, qpos, a.rot_pairs, a.inv_freq_rev);
#pragma unroll
      for (int e = 0; e < 8; e++) qf[t][e] = (_Float16)(f[t][e] * a.q_scale);
    }
  }

  floatx16 acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int j = 0; j < 16; j++) acc_o[db][j] = 0.f;
  // running max (log2 units, kept negated in a whole accumulator block that starts each score chain) and sum
  float m_run = 0.f, l_run = 0.f;
  bool m_set = false;
  floatx16 negm;
#pragma unroll
  for (int j = 0; j < 16; j++) negm[j] = 0.f;
  floatx16 sacc[2];
  half8 pf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int j = 0; j < 16; j++) sacc[kb][j] = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++) pf[kb][h2] = (half8){};

  // ---- direct loads: wave w copies the 1 KB LDS blocks 2w, 2w+1 of a K tile (key rows 4j..4j+3 each) and of a V^T
  // tile (dim rows 8j..8j+7 each), in the swizzled images above
  const uint32_t plane_bytes = (uint32_t)a.S_kpad * kHeadDim * 2;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.kt + (int64_t)unit * a.S_kpad * kHeadDim), (short)0, (int)plane_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.vt + (int64_t)unit * kHeadDim * a.S_kpad), (short)0, (int)plane_bytes, 0x00020000);
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int jj = 0; jj < 2; jj++) {
    const int j = 2 * wave + jj;
    const int kr = 4 * j + (lane >> 4);
    koff[jj] = (uint32_t)kr * (kHeadDim * 2) + 16u * (uint32_t)((lane & 15) ^ (kr & 15));
    const int vr = 8 * j + (lane >> 3);
    voff[jj] = (uint32_t)vr * (uint32_t)a.S_kpad * 2u + 16u * (uint32_t)((lane & 7) ^ ((vr >> 1) & 7));
  }
  auto issue_k = [&](int n, int buf) {   // K of tile t_lo + n into K buffer buf
    uint16_t* dst = smem + buf * kTileHalves;
    const uint32_t ks = (uint32_t)(t_lo + n) * kBN * kHeadDim * 2;
#pragma unroll
    for (int jj = 0; jj < 2; jj++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dst + (2 * wave + jj) * 512), 16, (int)koff[jj],
                                               (int)ks, 0, 0);
  };
  auto issue_v = [&](int n, int buf) {   // V^T of tile t_lo + n into V buffer buf
    uint16_t* dst = smem + (3 + buf) * kTileHalves;
    const uint32_t vs = (uint32_t)(t_lo + n) * kBN * 2;
#pragma unroll
    for (int jj = 0; jj < 2; jj++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dst + (2 * wave + jj) * 512), 16, (int)voff[jj],
                                               (int)vs, 0, 0);
  };

  // operand fragment addresses within a tile: V^T row 32db + l32, chunk 4kb + 2h2 + hi (fp16 elements, per lane);
  // K row 32hf + l32, chunk 2t8 + hi at chunk position (2t8 + hi) ^ (l32 mod 16), whose byte offset
  // l32 * 256 + 16 * ((2t8 + hi) ^ (l32 mod 16)) is kx ^ (32 t8) with kx the t8 = 0 offset (bits 5..7 hold t8 ^ ...)
  // (vfo includes the V^T region's base, 3 tiles in, so every fragment's immediate offset stays below 64 KB)
  int vfo[4];
#pragma unroll
  for (int c = 0; c < 4; c++) vfo[c] = 3 * kTileHalves + l32 * kBN + 8 * ((2 * c + hi) ^ ((l32 >> 1) & 7));
  const uint32_t kx = (uint32_t)l32 * (kHeadDim * 2) + 16u * (uint32_t)(hi ^ (l32 & 15));

  auto live = [&](int n) {   // this wave's queries see a key of tile n (relative index)
    const int kt = a.kbase + (t_lo + n) * kBN;
    if (kt > whi) return false;
    if (GATED && kt + kBN - 1 < wlo - a.window + 1) return false;
    return true;
  };

  // operand fragment f of an MFMA phase with K buffer KB and V buffer VB: 0..15 V^T (kb = f/8, h2 = (f/4)%2, db =
  // f%4), 16..31 K (t8 = (f-16)/2, half (f-16)%2)
  auto frag = [&](auto KBc, auto VBc, int f) -> half8 {
    constexpr int KB = decltype(KBc)::value, VB = decltype(VBc)::value;
    if (f < 16) {
      const int kb = f >> 3, h2 = (f >> 2) & 1, db = f & 3;
      return *reinterpret_cast<const half8*>(smem + VB * kTileHalves + db * 32 * kBN + vfo[2 * kb + h2]);
    }
    const int g = f - 16, t8 = g >> 1, hf = g & 1;
    const uint32_t kb_bytes = kx ^ (32u * (uint32_t)t8);
    return *reinterpret_cast<const half8*>(reinterpret_cast<const unsigned char*>(smem) +
                                           (KB * kTileHalves + hf * 32 * kHeadDim) * 2 + kb_bytes);
  };
  // the first four fragments of the next MFMA phase, read ahead of it
  half8 win[8];
  auto prefetch = [&](auto KBc, auto VBc) {
#pragma unroll
    for (int f = 0; f < 4; f++) win[f] = frag(KBc, VBc, f);
  };
  // MFMA phase: P V^T of the previous tile (V buffer VB), then S^T = K Q^T of this one (K buffer KB), both always
  // (P is zero where the previous tile showed this wave nothing; scores past the last tile are never used).  The
  // window holds the first four fragments on entry and takes the next four at once.
  auto mfma_phase = [&](auto KBc, auto VBc) {
#pragma unroll
    for (int f = 4; f < 8; f++) win[f] = frag(KBc, VBc, f);
#pragma unroll
    for (int f = 0; f < 32; f++) {
      const half8 op = win[f & 7];
      if (f + 8 < 32) win[(f + 8) & 7] = frag(KBc, VBc, f + 8);
      if (f < 16) {
        const int kb = f >> 3, h2 = (f >> 2) & 1, db = f & 3;
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op, pf[kb][h2], acc_o[db], 0, 0, 0);
      } else {
        const int g = f - 16, t8 = g >> 1, hf = g & 1;
        sacc[hf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op, qf[t8], t8 == 0 ? negm : sacc[hf], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // softmax phase of tile m: scores (relative to -m) -> P (fp16) and the row statistics.  The exponentials come
  // first; their sum exceeds 256 whenever a score exceeds m + 8, and only then (or before m is set) the tile's max
  // is taken, m raised and the exponentials redone.
  auto softmax_phase = [&](int m) {
    if (m >= n_tiles || !live(m)) {
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) pf[kb][h2] = (half8){};
      return;
    }
    const int kt = a.kbase + (t_lo + m) * kBN;
    if (kt + kBN - 1 > wlo || (GATED && kt < whi - a.window + 1)) {
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int key = kt + kb * 32 + 8 * (j >> 2) + 4 * hi + (j & 3);
          if ((unsigned)(qpos - key) >= lim) sacc[kb][j] = -INFINITY;
        }
    }
    auto exps = [&]() {
      half2 hs[2] = {half2{}, half2{}};
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
          uint32_t wp[4];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const int j = 8 * h2 + 2 * e;
            wp[e] = pack_f16(__builtin_amdgcn_exp2f(sacc[kb][j]), __builtin_amdgcn_exp2f(sacc[kb][j + 1]));
            hs[e & 1] = hs[e & 1] + __builtin_bit_cast(half2, wp[e]);   // packed fp16 sums of the rounded P
          }
          pf[kb][h2] = __builtin_bit_cast(half8, make_uint4(wp[0], wp[1], wp[2], wp[3]));
        }
      const half2 h = hs[0] + hs[1];
      return xor32_sum((float)h.x + (float)h.y);
    };
    float lt = exps();
    if (__any(!m_set || !(lt <= 256.0f))) {
      float mx0 = sacc[0][0], mx1 = sacc[1][0];
#pragma unroll
      for (int j = 1; j < 15; j += 2) {
        mx0 = fmaxf(fmaxf(mx0, sacc[0][j]), sacc[0][j + 1]);
        mx1 = fmaxf(fmaxf(mx1, sacc[1][j]), sacc[1][j + 1]);
      }
      float mx = fmaxf(fmaxf(mx0, sacc[0][15]), fmaxf(mx1, sacc[1][15]));
      mx = xor32_max(mx);
      const bool need = m_set ? mx > 8.0f : mx > -INFINITY;
      if (__any(need)) {
        const float sh = need ? mx : 0.0f;
        const float alpha = m_set ? __builtin_amdgcn_exp2f(-sh) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
          for (int j = 0; j < 16; j++) acc_o[db][j] *= alpha;
        m_run += sh;
        m_set = m_set || need;
#pragma unroll
        for (int j = 0; j < 16; j++) negm[j] = -m_run;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
          for (int j = 0; j < 16; j++) sacc[kb][j] -= sh;
        lt = exps();
      }
    }
    // lt is the sum over both lane halves; each half adds half of it back in the epilogue's final exchange
    l_run += 0.5f * lt;
  };

  // ---- prologue: K(0), K(1) and V(0) in LDS for everyone; V buffers 1 and 2 cleared (LDS starts with arbitrary
  // bits: M(0) multiplies V buffer 2 by its zero P, and a buffer no tile reaches is multiplied by zero P too, where
  // 0 * inf would be NaN)
  issue_k(0, 0);
  if (1 < n_tiles) issue_k(1, 1);
  issue_v(0, 0);
  {
    uint4* v12 = reinterpret_cast<uint4*>(smem + 4 * kTileHalves);
#pragma unroll
    for (int x = 0; x < 4; x++) v12[tid + 512 * x] = make_uint4(0u, 0u, 0u, 0u);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  const int n = n_tiles;
  // a phase boundary: this wave's LDS reads are done (lgkmcnt 0), then the work-group barrier; the memory clobber
  // keeps the compiler from moving LDS accesses across it, the scheduling barriers keep every instruction of a phase
  // inside it.  (__syncthreads() would also wait for the tile loads in flight.)
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto wait_tiles = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  };
  // the loads of phase 2m: K(m+2) into K buffer (m+2) mod 3, V(m+1) into V buffer (m+1) mod 3
  auto issue = [&](int m, auto K2c, auto V1c) {
    if (m + 2 < n) issue_k(m + 2, decltype(K2c)::value);
    if (m + 1 < n) issue_v(m + 1, decltype(V1c)::value);
  };
  // ---- phases.  Group 0 runs M(0) V(0) M(1) V(1) ... M(np), group 1 the same one phase later, np = the smallest
  // count >= n with np mod 3 = 1 (up to two empty tiles: no loads, zero P).  M(m) uses K buffer m mod 3 and V buffer
  // (m-1) mod 3; V(m) ends by reading M(m+1)'s first fragments.  Each group meets 2 np + 2 barriers.
  const int np = n + (4 - n % 3) % 3;
  prefetch(C0{}, C2{});
  if (group == 0) {
    issue(0, C2{}, C1{});
    mfma_phase(C0{}, C2{});
    barrier();
    softmax_phase(0);
    prefetch(C1{}, C0{});
    wait_tiles();
    barrier();
    for (int m = 1; m < np; m += 3) {
      issue(m, C0{}, C2{});
      mfma_phase(C1{}, C0{});
      barrier();
      softmax_phase(m);
      prefetch(C2{}, C1{});
      wait_tiles();
      barrier();
      issue(m + 1, C1{}, C0{});
      mfma_phase(C2{}, C1{});
      barrier();
      softmax_phase(m + 1);
      prefetch(C0{}, C2{});
      wait_tiles();
      barrier();
      issue(m + 2, C2{}, C1{});
      mfma_phase(C0{}, C2{});
      barrier();
      softmax_phase(m + 2);
      prefetch(C1{}, C0{});
      wait_tiles();
      barrier();
    }
    mfma_phase(C1{}, C0{});
    barrier();
    barrier();
  } else {
    issue(0, C2{}, C1{});
    barrier();
    mfma_phase(C0{}, C2{});
    wait_tiles();
    barrier();
    issue(1, C0{}, C2{});
    softmax_phase(0);
    prefetch(C1{}, C0{});
    barrier();
    for (int m = 1; m < np; m += 3) {
      mfma_phase(C1{}, C0{});
      wait_tiles();
      barrier();
      issue(m + 1, C1{}, C0{});
      softmax_phase(m);
      prefetch(C2{}, C1{});
      barrier();
      mfma_phase(C2{}, C1{});
      wait_tiles();
      barrier();
      issue(m + 2, C2{}, C1{});
      softmax_phase(m + 1);
      prefetch(C0{}, C2{});
      barrier();
      mfma_phase(C0{}, C2{});
      wait_tiles();
      barrier();
      issue(m + 3, C0{}, C2{});
      softmax_phase(m + 2);
      prefetch(C1{}, C0{});
      barrier();
    }
    mfma_phase(C1{}, C0{});
    barrier();
  }

  // ---- epilogue: O / l staged in LDS as fp32 rows, then 16 lanes per 256-byte bf16 output row (times sigmoid(g)
  // for a gated layer)
  l_run = xor32_sum(l_run);
  const float inv_l = 1.0f / l_run;
  if (a.lse && hi == 0 && qvalid)
    a.lse[((int64_t)b * a.Hq + hq) * a.S + i] = (m_run + __log2f(l_run)) * 0.6931471805599453f;
  float* Os = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int jq = 0; jq < 4; jq++) {
      const int d = db * 32 + 8 * jq + 4 * hi;
      float4 o;
      o.x = acc_o[db][4 * jq] * inv_l;
      o.y = acc_o[db][4 * jq + 1] * inv_l;
      o.z = acc_o[db][4 * jq + 2] * inv_l;
      o.w = acc_o[db][4 * jq + 3] * inv_l;
      *reinterpret_cast<float4*>(&Os[r * kOsStride + d]) = o;
    }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int c = tid + 512 * k;
    const int orow = c >> 4, oc = c & 15;
    const int ipos = i0 + orow % P2;
    if (ipos < a.S) {
      const int64_t goff = (((int64_t)b * a.S + ipos) * a.Hq + kvh * a.G + orow / P2) * kHeadDim + 8 * oc;
      const float4 o0 = *reinterpret_cast<const float4*>(&Os[orow * kOsStride + 8 * oc]);
      const float4 o1 = *reinterpret_cast<const float4*>(&Os[orow * kOsStride + 8 * oc + 4]);
      float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
      if (GATED) {
        float gv[8];
        unpack8(*reinterpret_cast<const uint4*>(a.gate + goff), gv);
#pragma unroll
        for (int e = 0; e < 8; e++)
          o[e] *= __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv[e] * kLog2e));
      }
      *reinterpret_cast<uint4*>(a.out + goff) = pack8(o);
    }
  }
}

}  // namespace

hipError_t launch_kv_stage(const StageArgs& a, hipStream_t st) {
  // the staged rows cover kbase .. pos0+S-1 in whole tiles; the prefix (< pos0) needs a cache to read
  const int64_t staged = (int64_t)a.pos0 + a.S - a.kbase;
  if (a.S < 1 || a.S_kpad % kBN || a.kbase < 0 || a.kbase > a.pos0 || staged > a.S_kpad || a.S_kpad - staged >= kBN ||
      (a.kbase < a.pos0 && (!a.ck || !a.cv || a.slots < 1)) || (a.ring && a.pos0 - a.kbase >= a.slots))
    return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.B * a.Hkv * (a.S_kpad / kBN);
  hipLaunchKernelGGL(kv_stage_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_pp(const TileAttnArgs& a, bool gated, hipStream_t st) {
  // a.P is half the work-group's positions here: 256 query rows = G heads x 2P positions
  const int64_t staged = (int64_t)a.pos0 + a.S - a.kbase;
  const int64_t first_key = gated ? std::max<int64_t>(0, (int64_t)a.pos0 - a.window + 1) : 0;
  if (a.S < 1 || a.S_kpad % kBN || a.kbase < 0 || a.kbase > first_key || staged > a.S_kpad || a.G * a.P != 128 ||
      a.n_units != a.B * a.Hkv || a.n_qtiles != (a.S + 2 * a.P - 1) / (2 * a.P) || (gated && (a.window < 1 || !a.gate)))
    return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.n_units * a.n_qtiles;
  if (gated)
    hipLaunchKernelGGL(attn_pp_kernel<true>, dim3((unsigned)blocks), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL(attn_pp_kernel<false>, dim3((unsigned)blocks), dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ring_write(const RingWriteArgs& a, hipStream_t st) {
  if (a.n < 1 || a.n > a.S || a.n > a.W) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)a.B * a.Hkv * a.n;
  hipLaunchKernelGGL(ring_write_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace zg
