// Prefill kernels of the ZGCM-1 attention core for gfx950 (CDNA4, wave64, MFMA).
//
//   kv_prologue_kernel  k_hat = RoPE(RMSNorm(k) * w_k) of a chunk, computed once and rounded to bf16 (the
//                       KV-cache format); written as bf16 to the KV cache or, converted exactly, as fp16
//                       to the workspace; v copied alongside when needed.
//   attn_prefill_kernel flash-style attention of 128 query rows (one KV group) per work-group against
//                       64-key tiles staged in LDS.  The Q prologue (RMSNorm * w_q, partial RoPE, softmax
//                       scale) is fused into the Q load; QK^T and PV run on v_mfma_f32_32x32x16_f16 with
//                       fp32 accumulation and fp32 online softmax.  GATED=true is the gated sliding-window
//                       layer (band of W keys, tiles outside skipped, sigmoid(gate) in the epilogue),
//                       GATED=false the global causal layer.
//   ring_write_kernel   after an SWA chunk, its last min(S, W) keys/values go to ring slot pos mod W.
//
// Method (ZGCM-1 paper summaries: onedev.kr "How it works"; jaehun.me "How Gated SWA Behaves"):
// per (token, head) q_hat = RoPE(RMSNorm(q) w_q), k_hat likewise; SWA output
// softmax_{i-W < j <= i}(q_hat k_hat_j / sqrt(D)) v_j (.) sigmoid(g); global output has j <= i, no gate.
//
// Precision: I/O and the KV cache are bf16.  Inside the MFMAs q_hat, k_hat, P and v are fp16 (11
// significant bits against bf16's 8): k_hat and v are bf16 values, which fp16 holds exactly in their
// range, and q_hat and P are rounded once to fp16.  This keeps the attention error well below the bf16
// rounding of the output.
#include "common.h"
#include "launch.h"

namespace zg {
namespace {

constexpr int kBN = 64;         // keys per LDS tile
constexpr int kKsStride = 136;  // halfs per K row in LDS: 128 + 8 pad (272 B keeps 16-B lane reads conflict-free)
constexpr int kVtStride = 72;   // halfs per V^T row in LDS: 64 keys + 8 pad
constexpr int kOsStride = 132;  // floats per output row staged in LDS (epilogue): 128 + 4 pad

// ---------------------------------------------------------------------------------------------
// k_hat prologue: one 16-lane group per (b, s, kv head) row, 8 dims per lane.
__global__ void __launch_bounds__(256) kv_prologue_kernel(KvPrologueArgs a) {
  const int c = threadIdx.x & 15;
  const int64_t n_rows = (int64_t)a.B * a.S * a.Hkv;
  const int64_t row_raw = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool valid = row_raw < n_rows;
  const int64_t row = valid ? row_raw : n_rows - 1;
  const int h = (int)(row % a.Hkv);
  const int64_t s = (row / a.Hkv) % a.S;
  const int64_t b = row / ((int64_t)a.Hkv * a.S);

  float f[8];
  unpack8(*reinterpret_cast<const uint4*>(a.k + row * kHeadDim + 8 * c), f);
  norm_rope8_g16(f, a.kw, c, a.pos0 + s, a.eps, a.rot_pairs, a.inv_freq_rev);
  if (valid) {
    const int64_t off = b * a.d_sb + h * a.d_sh + s * a.d_st + 8 * c;
    const uint4 kb = pack8(f);   // the KV-cache value of k_hat (bf16, nearest-even)
    *reinterpret_cast<uint4*>(a.kdst + off) = a.dst_f16 ? bf16x8_to_f16x8(kb) : kb;
    if (a.v) {
      const uint4 vb = *reinterpret_cast<const uint4*>(a.v + row * kHeadDim + 8 * c);
      *reinterpret_cast<uint4*>(a.vdst + off) = a.dst_f16 ? bf16x8_to_f16x8(vb) : vb;
    }
  }
}

// ---------------------------------------------------------------------------------------------
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

// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t dword_of(const uint4& w, int i) {
  return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
}

// Work-group: 256 threads = 4 waves; 128 query rows = G heads x P positions of one KV head; wave w
// owns rows 32w..32w+31 (row r -> head r / P, position i0 + r % P).  The S^T = K Q^T formulation puts
// one query per lane column, so the softmax statistics of a query live in lanes l and l+32 only.
template <bool GATED, bool KA_BF16, bool VA_BF16, bool HAS_RING>
__global__ void __launch_bounds__(256, 2) attn_prefill_kernel(PrefillArgs a) {
  // one LDS block: K tiles [2][64][136] and V^T tiles [2][128][72] (fp16) during the loop, the fp32
  // output rows [128][132] in the epilogue
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kBN * kKsStride + 2 * kHeadDim * kVtStride];
  static_assert(128 * kOsStride * 4 <= sizeof(smem), "epilogue staging exceeds the tile buffers");
  uint16_t (*Ks)[kBN * kKsStride] = reinterpret_cast<uint16_t (*)[kBN * kKsStride]>(smem);
  uint16_t (*Vt)[kHeadDim * kVtStride] = reinterpret_cast<uint16_t (*)[kHeadDim * kVtStride]>(smem + 2 * kBN * kKsStride);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // Block order: consecutive block ids walk the (b, kv head) units first, so with B*Hkv a multiple of 8
  // every block of one unit lands on the same XCD (blocks go round-robin over the 8 XCDs) and its K/V
  // stay in that XCD's L2.  Global layers take the longest query tiles first.
  const int unit = blockIdx.x % a.n_units;
  const int qt_rank = blockIdx.x / a.n_units;
  const int qt = GATED ? qt_rank : (a.n_qtiles - 1 - qt_rank);
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int i0 = qt * a.P;

  const int r = wave * 32 + l32;
  const int hq = kvh * a.G + r / a.P;
  const int i = i0 + r % a.P;
  const bool qvalid = i < a.S;
  const int ic = qvalid ? i : a.S - 1;
  const int64_t qpos = a.pos0 + ic;

  // wave-uniform position range of this wave's rows (clamped to the chunk)
  int pl_lo, pl_hi;
  if (a.P >= 32) { pl_lo = (wave * 32) % a.P; pl_hi = pl_lo + 31; } else { pl_lo = 0; pl_hi = a.P - 1; }
  const int64_t wlo = a.pos0 + min(i0 + pl_lo, a.S - 1);
  const int64_t whi = a.pos0 + min(i0 + pl_hi, a.S - 1);

  // key range of the work-group (absolute positions, end exclusive)
  const int64_t khi = a.pos0 + min(i0 + a.P, a.S);
  int64_t klo = 0;
  if (GATED) { klo = a.pos0 + i0 - a.window + 1; if (klo < 0) klo = 0; }
  const int t0 = (int)(klo / kBN), t1 = (int)((khi + kBN - 1) / kBN);

  // ---- Q prologue: load, RMSNorm * w_q, partial RoPE, scale by log2(e)/sqrt(D), round to fp16.
  // MFMA B operand (Q^T, K = d): lane holds q_hat[query l32][16t + 8hi .. +8] for k-step t.
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

  // SWA: fetch the gate logits of the work-group's 128 rows now, coalesced (16 lanes per 256-byte row,
  // 8 chunks of 16 bytes per thread), so their latency overlaps the whole tile loop.
  uint4 gate_pre[8];
  if (GATED) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int c = tid + 256 * k;
      const int orow = c >> 4, oc = c & 15;
      const int ipos = min(i0 + orow % a.P, a.S - 1);
      gate_pre[k] = *reinterpret_cast<const uint4*>(
          a.gate + (((int64_t)b * a.S + ipos) * a.Hq + kvh * a.G + orow / a.P) * kHeadDim + 8 * oc);
    }
  }

  floatx16 acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int j = 0; j < 16; j++) acc_o[db][j] = 0.f;
  // Running max m (log2 units) and sum l of this lane's query.  The global layer keeps -m in a whole
  // accumulator block and starts each score chain from it, so its MFMAs yield s - m directly (the SWA
  // layer, short of registers, subtracts m afterwards).  m is set by the first tile that shows the query a
  // visible key (m_set) and raised lazily after that.
  float m_run = 0.f, l_run = 0.f;
  bool m_set = false;
  floatx16 negm;
#pragma unroll
  for (int j = 0; j < 16; j++) negm[j] = 0.f;

  // ---- tile loading roles.  Rows past the key range are clamped to its last row: always initialised
  // data, whose scores the causal mask removes.
  const int kc = tid & 15, kr = tid >> 4;   // K: 16-byte chunk kc of rows kr + 16 rr
  const int vq = tid & 15, vd = tid >> 4;   // V: keys 4vq..4vq+3, dims 8vd..8vd+7
  const uint16_t* kplane = a.kA + b * a.kA_sb + kvh * a.kA_sh + 8 * kc;
  const uint16_t* vplane = a.vA + b * a.vA_sb + kvh * a.vA_sh + 8 * vd;
  const int kst = (int)a.kA_st, vst = (int)a.vA_st;
  const int apos0 = (int)a.a_pos0;
  const int klast = (int)khi - 1;
  uint4 kreg[4], vreg[4];
  const uint16_t* kplane_u = a.kA + b * a.kA_sb + kvh * a.kA_sh;   // wave-uniform plane bases
  const uint16_t* vplane_u = a.vA + b * a.vA_sb + kvh * a.vA_sh;
  int kvoff[4], vvoff[4];   // per-lane byte offsets of this thread's rows within a tile
#pragma unroll
  for (int rr = 0; rr < 4; rr++) {
    kvoff[rr] = ((kr + 16 * rr) * kst + 8 * kc) * 2;
    vvoff[rr] = ((4 * vq + rr) * vst + 8 * vd) * 2;
  }

  auto load_tile = [&](int t) {
    const int kt = t * kBN;
    if (HAS_RING && kt < apos0) {
      // part of this tile precedes the chunk: those rows come from the SWA ring (bf16, slot pos mod W)
      const uint16_t* kring = a.kR + b * a.R_sb + kvh * a.R_sh + 8 * kc;
      const uint16_t* vring = a.vR + b * a.R_sb + kvh * a.R_sh + 8 * vd;
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        const int pos = min(kt + kr + 16 * rr, klast);
        const bool ring = pos < apos0;
        const uint4 w = ring ? *reinterpret_cast<const uint4*>(kring + (pos % a.window) * kHeadDim)
                             : *reinterpret_cast<const uint4*>(kplane + (pos - apos0) * kst);
        kreg[rr] = (KA_BF16 || ring) ? bf16x8_to_f16x8(w) : w;
      }
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        const int pos = min(kt + 4 * vq + rr, klast);
        const bool ring = pos < apos0;
        const uint4 w = ring ? *reinterpret_cast<const uint4*>(vring + (pos % a.window) * kHeadDim)
                             : *reinterpret_cast<const uint4*>(vplane + (pos - apos0) * vst);
        vreg[rr] = (VA_BF16 || ring) ? bf16x8_to_f16x8(w) : w;
      }
    } else {
      // Buffer loads: the descriptor base moves with the tile (scalar), the per-lane byte offsets stay
      // constant, and rows past the key range fall outside num_records and read as zero.
      const int rows = min(kBN, klast + 1 - kt);
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kplane_u + (int64_t)(kt - apos0) * kst), (short)0, rows * kst * 2, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vplane_u + (int64_t)(kt - apos0) * vst), (short)0, rows * vst * 2, 0x00020000);
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        const uint4 w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, kvoff[rr], 0, 0));
        kreg[rr] = KA_BF16 ? bf16x8_to_f16x8(w) : w;
      }
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        const uint4 w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, vvoff[rr], 0, 0));
        vreg[rr] = VA_BF16 ? bf16x8_to_f16x8(w) : w;
      }
    }
  };
  // V^T column of key k within a tile: 16-key groups, inside a group the quads 1 and 2 swap places so
  // that the 8 keys an MFMA lane needs for one PV k-step are contiguous.
  const int vq_in = vq & 3;
  const int vcol = 16 * (vq >> 2) + 4 * (vq_in == 1 ? 2 : vq_in == 2 ? 1 : vq_in);
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int rr = 0; rr < 4; rr++) *reinterpret_cast<uint4*>(&Ks[buf][(kr + 16 * rr) * kKsStride + 8 * kc]) = kreg[rr];
    // transpose 4 keys x 8 dims: dim e of keys 0..3 -> one 8-byte LDS row segment (v_perm_b32 pairs halves)
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint2 w;
      w.x = __builtin_amdgcn_perm(dword_of(vreg[1], e >> 1), dword_of(vreg[0], e >> 1), sel);
      w.y = __builtin_amdgcn_perm(dword_of(vreg[3], e >> 1), dword_of(vreg[2], e >> 1), sel);
      *reinterpret_cast<uint2*>(&Vt[buf][(8 * vd + e) * kVtStride + vcol]) = w;
    }
  };

  const half2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  auto compute = [&](int buf, int t) {
    const int64_t kt = (int64_t)t * kBN;
    if (kt > whi) return;                                             // beyond every query of the wave
    if (GATED && kt + kBN - 1 < wlo - a.window + 1) return;           // before every window of the wave
    // S^T = K Q^T for the two 32-key halves; the two accumulator chains are interleaved so consecutive
    // MFMAs are independent.
    floatx16 sacc[2];
    const uint16_t* kfrag = &Ks[buf][l32 * kKsStride + 8 * hi];
#pragma unroll
    for (int t8 = 0; t8 < 8; t8++) {
      const half8 k0 = *reinterpret_cast<const half8*>(kfrag + 16 * t8);
      const half8 k1 = *reinterpret_cast<const half8*>(kfrag + 32 * kKsStride + 16 * t8);
      floatx16 c0 = sacc[0], c1 = sacc[1];
      if (t8 == 0) {
        if constexpr (GATED) {
#pragma unroll
          for (int j = 0; j < 16; j++) c0[j] = c1[j] = 0.f;
        } else {
          c0 = c1 = negm;
        }
      }
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, qf[t8], c0, 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1, qf[t8], c1, 0, 0, 0);
    }
    const bool full = (kt + kBN - 1 <= wlo) && (!GATED || kt >= whi - a.window + 1);
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int64_t key = kt + kb * 32 + 8 * (j >> 2) + 4 * hi + (j & 3);
          bool vis = key <= qpos;
          if (GATED) vis = vis && (qpos - key < a.window);
          if (!vis) sacc[kb][j] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int j = 0; j < 16; j += 2) mx = fmaxf(mx, fmaxf(sacc[kb][j], sacc[kb][j + 1]));
    mx = xor32_max(mx);
    // mx is the tile's max relative to m (global) or absolute (SWA).  m is raised only when the scores
    // exceed it by more than 2^8 (exact: the m used is carried along; every p stays <= 256), or set on the
    // query's first visible key.
    if constexpr (GATED) mx -= m_run;   // the global layer's sacc already holds s - m
    const bool need = m_set ? mx > 8.0f : mx > -INFINITY;
    if (__any(need)) {
      const float sh = need ? mx : 0.0f;
      const float alpha = m_set ? __builtin_amdgcn_exp2f(-sh) : 1.0f;   // l and acc are still 0 before
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int j = 0; j < 16; j++) acc_o[db][j] *= alpha;
      m_run += sh;
      m_set = m_set || need;
      if constexpr (!GATED) {
#pragma unroll
        for (int j = 0; j < 16; j++) negm[j] = -m_run;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
          for (int j = 0; j < 16; j++) sacc[kb][j] -= sh;
      }
    }
    if constexpr (GATED) {
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int j = 0; j < 16; j++) sacc[kb][j] -= m_run;
    }
    // P = exp2(s - m) rounded to fp16; the row sum adds the same rounded values (v_dot2 with ones), so
    // numerator and denominator use identical weights.
    half8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int h2 = 0; h2 < 2; h2++) {
        uint32_t wp[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int j = 8 * h2 + 2 * e;
          wp[e] = pack_f16(__builtin_amdgcn_exp2f(sacc[kb][j]), __builtin_amdgcn_exp2f(sacc[kb][j + 1]));
          l_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2, wp[e]), ones, l_run, false);
        }
        pf[kb][h2] = __builtin_bit_cast(half8, make_uint4(wp[0], wp[1], wp[2], wp[3]));
      }
    // O^T += V^T P^T: four independent accumulators (32-dim blocks) per k-step
    const uint16_t* vfrag = &Vt[buf][l32 * kVtStride + 8 * hi];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const half8 va = *reinterpret_cast<const half8*>(vfrag + db * 32 * kVtStride + kb * 32 + 16 * h2);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf[kb][h2], acc_o[db], 0, 0, 0);
        }
  };

  if (t0 < t1) {
    load_tile(t0);
    store_tile(0);
  }
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    const bool more = t + 1 < t1;
    if (more) load_tile(t + 1);
    compute(buf, t);
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, stage the 128 rows through LDS as fp32 (the K/V buffers are free after the
  // loop's last barrier), then each thread finishes 8 consecutive dims of a row (gate for SWA, bf16
  // rounding) and 16 consecutive lanes store a whole 256-byte row.
  // O^T lane layout: acc_o[db][j] is d = 32db + 8(j/4) + 4hi + j%4 of query row r.
  l_run = xor32_sum(l_run);
  const float inv_l = 1.0f / l_run;
  // training: the log-sum-exp of the query's scores (natural log; scores in log2 units are s log2(e))
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
    const int c = tid + 256 * k;
    const int orow = c >> 4, oc = c & 15;
    const int ipos = i0 + orow % a.P;
    if (ipos < a.S) {
      const int64_t goff = (((int64_t)b * a.S + ipos) * a.Hq + kvh * a.G + orow / a.P) * kHeadDim + 8 * oc;
      const float4 o0 = *reinterpret_cast<const float4*>(&Os[orow * kOsStride + 8 * oc]);
      const float4 o1 = *reinterpret_cast<const float4*>(&Os[orow * kOsStride + 8 * oc + 4]);
      float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
      if (GATED) {
        float g[8];
        unpack8(gate_pre[k], g);
#pragma unroll
        for (int e = 0; e < 8; e++) o[e] *= 1.0f / (1.0f + __expf(-g[e]));
      }
      *reinterpret_cast<uint4*>(a.out + goff) = pack8(o);
    }
  }
}

}  // namespace

hipError_t launch_kv_prologue(const KvPrologueArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.S * a.Hkv;
  const int64_t blocks = (rows + 15) / 16;
  hipLaunchKernelGGL(kv_prologue_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ring_write(const RingWriteArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Hkv * a.n;
  const int64_t blocks = (rows + 15) / 16;
  hipLaunchKernelGGL(ring_write_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const PrefillArgs& a, hipStream_t st) {
  const int64_t blocks = (int64_t)a.n_units * a.n_qtiles;
  const dim3 grid((unsigned)blocks), block(256);
  if (a.gate) {
    // gated SWA: chunk keys come from the fp16 workspace, values from the bf16 input
    if (a.ka_bf16 || !a.va_bf16) return hipErrorInvalidValue;
    if (a.kR)
      hipLaunchKernelGGL((attn_prefill_kernel<true, false, true, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((attn_prefill_kernel<true, false, true, false>), grid, block, 0, st, a);
  } else if (a.ka_bf16 && a.va_bf16) {
    hipLaunchKernelGGL((attn_prefill_kernel<false, true, true, false>), grid, block, 0, st, a);    // from the KV cache
  } else if (!a.ka_bf16 && !a.va_bf16) {
    hipLaunchKernelGGL((attn_prefill_kernel<false, false, false, false>), grid, block, 0, st, a);  // from the workspace
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace zg
