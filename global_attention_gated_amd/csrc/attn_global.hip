// Global causal prefill of the ZGCM-1 attention core for gfx950 (CDNA4, wave64, MFMA): the layer without a
// cache (one-shot prefill and the training forward).
//
//   kv_tiles_kernel     k_hat = RoPE(RMSNorm(k) w_k), rounded to bf16 (the KV-cache value) and held as fp16, and
//                       v^T as fp16, written once per layer in the layout that the attention kernel copies into
//                       LDS unchanged.
//   attn_global_kernel  flash-style causal attention of 128 query rows (G heads x P positions of one KV head) per
//                       work-group against 64-key tiles.  Each tile goes from the workspace straight into LDS
//                       (buffer loads with LDS as the destination: no registers, no LDS write instructions), 16 KB
//                       of keys and 16 KB of transposed values, double-buffered.  A direct load writes 16 bytes
//                       per lane at consecutive LDS addresses; the lanes choose their source chunks so that the LDS
//                       rows come out XOR-swizzled, which keeps the MFMA operand reads free of bank conflicts
//                       without padding.
//
// Method (ZGCM-1 paper summaries: onedev.kr "How it works"): per (token, head) q_hat = RoPE(RMSNorm(q) w_q), k_hat
// likewise; the global output is softmax_{j <= i}(q_hat k_hat_j / sqrt(D)) v_j.
//
// Precision as the other prefill kernels: k_hat and v are bf16 values held exactly in fp16, q_hat and P are
// rounded once to fp16, the MFMAs accumulate in fp32, and the online softmax runs in fp32.
#include "common.h"
#include "launch.h"

namespace zg {
namespace {

constexpr int kBN = 64;                          // keys per tile
constexpr int kTileHalves = kBN * kHeadDim;      // 8192 fp16 = 16 KB: one K tile, or one V^T tile
constexpr int kOsStride = 132;                   // floats per output row staged in LDS (epilogue): 128 + 4 pad
constexpr int kSmemBytes = 128 * kOsStride * 4;  // 67,584 B: the epilogue staging; the tile loop uses 64 KB of it
static_assert(4 * kTileHalves * 2 <= kSmemBytes, "tile buffers exceed the LDS block");
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);   // s_waitcnt vmcnt(0), other counters not waited for

typedef __attribute__((address_space(3))) void lds_void;

// ------------------------------------------------------------------------------------------------ prologue
// One work-group per (sequence, KV head, 64-key tile).
__global__ void __launch_bounds__(256) kv_tiles_kernel(KvTilesArgs a) {
  const int tid = threadIdx.x;
  const int n_tiles = a.S_pad / kBN;
  const int unit = blockIdx.x / n_tiles, tile = blockIdx.x % n_tiles;
  const int b = unit / a.Hkv, h = unit % a.Hkv;
  const int kt = tile * kBN;
  const int64_t row_b = (int64_t)b * a.S;   // input row of (b, s, h): (row_b + s) * Hkv + h
  // k_hat: a 16-lane group per key row (rows g, g + 16, g + 32, g + 48), 8 dims per lane; padding rows are zero
  {
    const int c = tid & 15, g = tid >> 4;
    uint16_t* dst = a.kt + ((int64_t)unit * a.S_pad + kt) * kHeadDim + 8 * c;
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      const int r = g + 16 * rr, s = kt + r;
      const int sc = s < a.S ? s : a.S - 1;
      float f[8];
      unpack8(*reinterpret_cast<const uint4*>(a.k + ((row_b + sc) * a.Hkv + h) * kHeadDim + 8 * c), f);
      norm_rope8_g16(f, a.kw, c, sc, a.eps, a.rot_pairs, a.inv_freq_rev);
      const uint4 w = s < a.S ? bf16x8_to_f16x8(pack8(f)) : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(dst + (int64_t)r * kHeadDim) = w;
    }
  }
  // v^T: thread (vq, vd) turns keys 4vq..4vq+3 x dims 8vd..8vd+7 into 8 dim rows of 4 keys (v_perm pairs the
  // 16-bit halves); the 4 keys go to quad slot perm(vq mod 4) of their 16-key group, perm = (0, 2, 1, 3)
  {
    const int vq = tid & 15, vd = tid >> 4;
    uint32_t w[4][4];
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      const int s = kt + 4 * vq + rr;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (s < a.S)
        x = bf16x8_to_f16x8(*reinterpret_cast<const uint4*>(a.v + ((row_b + s) * a.Hkv + h) * kHeadDim + 8 * vd));
      w[rr][0] = x.x; w[rr][1] = x.y; w[rr][2] = x.z; w[rr][3] = x.w;
    }
    const int qin = vq & 3;
    const int col = 16 * (vq >> 2) + 4 * (qin == 1 ? 2 : qin == 2 ? 1 : qin);
    uint16_t* dst = a.vt + ((int64_t)unit * kHeadDim + 8 * vd) * a.S_pad + kt + col;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint2 o;
      o.x = __builtin_amdgcn_perm(w[1][e >> 1], w[0][e >> 1], sel);
      o.y = __builtin_amdgcn_perm(w[3][e >> 1], w[2][e >> 1], sel);
      *reinterpret_cast<uint2*>(dst + (int64_t)e * a.S_pad) = o;
    }
  }
}

// ------------------------------------------------------------------------------------------------ attention
// Work-group: 256 threads = 4 waves; 128 query rows = G heads x P positions of one KV head; wave w owns rows
// 32w..32w+31 (row r -> head r / P, position i0 + r % P).  S^T = K Q^T puts one query per lane column, so the
// softmax statistics of a query live in lanes l and l + 32 only.
//
// LDS tile images (fp16, dense):
//   K   [64 keys][128 dims]: 16-byte chunk c (dims 8c..8c+7) of key row r sits at chunk position c ^ (r mod 16)
//   V^T [128 dims][64 keys]: chunk c (8 stored keys) of dim row r sits at chunk position c ^ ((r / 2) mod 8)
// The MFMA A-operand reads take one chunk from each of 16 consecutive rows per LDS cycle group; the swizzles
// spread those 16 chunks over all 64 banks.
__global__ void __launch_bounds__(256, 2) attn_global_kernel(GlobalArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kSmemBytes / 2];
  uint16_t* const Ks = smem;                     // [2] K tiles
  uint16_t* const Vt = smem + 2 * kTileHalves;   // [2] V^T tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // Block order: consecutive block ids walk the (b, kv head) units first, so with B*Hkv a multiple of 8 every
  // block of one unit lands on the same XCD (blocks go round-robin over the 8 XCDs) and its keys and values stay
  // in that XCD's L2; the longest query tiles go first.
  const int unit = blockIdx.x % a.n_units;
  const int qt = a.n_qtiles - 1 - (int)(blockIdx.x / a.n_units);
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int i0 = qt * a.P;

  const int r = wave * 32 + l32;
  const int hq = kvh * a.G + r / a.P;
  const int i = i0 + r % a.P;
  const bool qvalid = i < a.S;
  const int qpos = qvalid ? i : a.S - 1;

  // wave-uniform position range of this wave's rows (clamped to the sequence)
  int pl_lo, pl_hi;
  if (a.P >= 32) { pl_lo = (wave * 32) % a.P; pl_hi = pl_lo + 31; } else { pl_lo = 0; pl_hi = a.P - 1; }
  const int wlo = min(i0 + pl_lo, a.S - 1);
  const int whi = min(i0 + pl_hi, a.S - 1);
  const int khi = min(i0 + a.P, a.S);             // keys 0 .. khi-1 are visible to some row of the work-group
  const int n_tiles = (khi + kBN - 1) / kBN;

  // ---- Q prologue: load, RMSNorm * w_q, partial RoPE, scale by log2(e)/sqrt(D), round to fp16.
  // MFMA B operand (Q^T, K = d): lane holds q_hat[query l32][16t + 8hi .. +8] for k-step t.
  half8 qf[8];
  {
    const uint16_t* qrow = a.q + (((int64_t)b * a.S + qpos) * a.Hq + hq) * kHeadDim;
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
  // Running max m (log2 units) and sum l of this lane's query.  -m fills a whole accumulator block and starts
  // each score chain, so the MFMAs yield s - m directly.  m is set by the first tile that shows the query a
  // visible key (m_set) and raised lazily after that.
  float m_run = 0.f, l_run = 0.f;
  bool m_set = false;
  floatx16 negm;
#pragma unroll
  for (int j = 0; j < 16; j++) negm[j] = 0.f;

  // ---- direct loads: wave w copies the 1 KB LDS blocks 4w..4w+3 of the K tile (key rows 4j..4j+3 each) and of
  // the V^T tile (dim rows 8j..8j+7 each).  Byte offsets within the planes, constant over the tiles; the tile
  // moves the scalar offset.  Every tile lies inside the padded planes, so no load is out of range.
  const uint32_t plane_bytes = (uint32_t)a.S_pad * kHeadDim * 2;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.kt + (int64_t)unit * a.S_pad * kHeadDim), (short)0, (int)plane_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.vt + (int64_t)unit * kHeadDim * a.S_pad), (short)0, (int)plane_bytes, 0x00020000);
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int jj = 0; jj < 4; jj++) {
    const int j = 4 * wave + jj;
    const int kr = 4 * j + (lane >> 4);            // key row that this lane's 16 bytes fill
    koff[jj] = (uint32_t)kr * (kHeadDim * 2) + 16u * (uint32_t)((lane & 15) ^ (kr & 15));
    const int vr = 8 * j + (lane >> 3);            // dim row
    voff[jj] = (uint32_t)vr * (uint32_t)a.S_pad * 2u + 16u * (uint32_t)((lane & 7) ^ ((vr >> 1) & 7));
  }
  auto issue_tile = [&](int t, int buf) {
    const uint32_t ks = (uint32_t)t * kBN * kHeadDim * 2, vs = (uint32_t)t * kBN * 2;
#pragma unroll
    for (int jj = 0; jj < 4; jj++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(Ks + buf * kTileHalves + (4 * wave + jj) * 512), 16,
                                               (int)koff[jj], (int)ks, 0, 0);
#pragma unroll
    for (int jj = 0; jj < 4; jj++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(Vt + buf * kTileHalves + (4 * wave + jj) * 512), 16,
                                               (int)voff[jj], (int)vs, 0, 0);
  };

  // MFMA A-operand reads (fp16 element offsets within a tile): K row 32kb + l32, chunk 2t8 + hi; V^T row
  // 32db + l32, chunk 4kb + 2h2 + hi (the 8 stored keys that P's C registers 8h2..8h2+7 of block kb hold).
  int kfo[8], vfo[4];
#pragma unroll
  for (int t8 = 0; t8 < 8; t8++) kfo[t8] = l32 * kHeadDim + 8 * ((2 * t8 + hi) ^ (l32 & 15));
#pragma unroll
  for (int c = 0; c < 4; c++) vfo[c] = l32 * kBN + 8 * ((2 * c + hi) ^ ((l32 >> 1) & 7));

  const half2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  auto compute = [&](int buf, int t) {
    const int kt = t * kBN;
    if (kt > whi) return;   // beyond every query of the wave
    const uint16_t* kb_ = Ks + buf * kTileHalves;
    const uint16_t* vb_ = Vt + buf * kTileHalves;
    // S^T = K Q^T for the two 32-key halves; the two accumulator chains are interleaved so consecutive MFMAs are
    // independent, and both start from -m.  All 16 K fragments are read first (the scheduler would otherwise put
    // each read right before its MFMA and expose the LDS latency), and the same registers then take the 16 V^T
    // fragments of the PV product, read while the softmax runs.
    half8 op[16];
#pragma unroll
    for (int t8 = 0; t8 < 8; t8++) {
      op[2 * t8] = *reinterpret_cast<const half8*>(kb_ + kfo[t8]);
      op[2 * t8 + 1] = *reinterpret_cast<const half8*>(kb_ + 32 * kHeadDim + kfo[t8]);
    }
    __builtin_amdgcn_sched_barrier(0);
    floatx16 sacc[2];
#pragma unroll
    for (int t8 = 0; t8 < 8; t8++) {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op[2 * t8], qf[t8], t8 == 0 ? negm : sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op[2 * t8 + 1], qf[t8], t8 == 0 ? negm : sacc[1], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
        for (int db = 0; db < 4; db++)
          op[8 * kb + 4 * h2 + db] = *reinterpret_cast<const half8*>(vb_ + db * 32 * kBN + vfo[2 * kb + h2]);
    if (kt + kBN - 1 > wlo) {   // the diagonal cuts this tile for some row of the wave
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int key = kt + kb * 32 + 8 * (j >> 2) + 4 * hi + (j & 3);
          if (key > qpos) sacc[kb][j] = -INFINITY;
        }
    }
    // row max: two chains of three-input maxima (v_max3), one per 32-key half
    float mx0 = sacc[0][0], mx1 = sacc[1][0];
#pragma unroll
    for (int j = 1; j < 15; j += 2) {
      mx0 = fmaxf(fmaxf(mx0, sacc[0][j]), sacc[0][j + 1]);
      mx1 = fmaxf(fmaxf(mx1, sacc[1][j]), sacc[1][j + 1]);
    }
    float mx = fmaxf(fmaxf(mx0, sacc[0][15]), fmaxf(mx1, sacc[1][15]));
    mx = xor32_max(mx);
    // mx is the tile's max relative to m.  m is raised only when the scores exceed it by more than 2^8 (exact:
    // the m used is carried along; every p stays <= 256), or set on the query's first visible key.
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
#pragma unroll
      for (int j = 0; j < 16; j++) negm[j] = -m_run;
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int j = 0; j < 16; j++) sacc[kb][j] -= sh;
    }
    // P = exp2(s - m) rounded to fp16; the row sum adds the same rounded values (v_dot2 with ones), so numerator
    // and denominator use identical weights.
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
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
        for (int db = 0; db < 4; db++)
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op[8 * kb + 4 * h2 + db], pf[kb][h2], acc_o[db], 0, 0, 0);
  };

  // One step: start the next tile's copy into the other buffer (free: every wave passed the barrier after its
  // last use), compute this one, then wait for this wave's copies and meet the other waves, after which the next
  // tile is complete in LDS.  The loop runs two steps per pass so each step's buffer is a constant.
  auto step = [&](int t, int buf) {
    if (t + 1 < n_tiles) issue_tile(t + 1, buf ^ 1);
    compute(buf, t);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };
  issue_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, 0);
    if (t + 1 < n_tiles) step(t + 1, 1);
  }

  // ---- epilogue: normalise, stage the 128 rows through LDS as fp32 (the tile buffers are free after the loop's
  // last barrier), then each thread rounds 8 consecutive dims of a row to bf16 and 16 consecutive lanes store a
  // whole 256-byte row.  O^T lane layout: acc_o[db][j] is d = 32db + 8(j/4) + 4hi + j%4 of query row r.
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
      const float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
      *reinterpret_cast<uint4*>(a.out + goff) = pack8(o);
    }
  }
}

}  // namespace

hipError_t launch_kv_tiles(const KvTilesArgs& a, hipStream_t st) {
  if (a.S < 1 || a.S_pad % kBN || a.S_pad < a.S || a.S_pad - a.S >= kBN) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.B * a.Hkv * (a.S_pad / kBN);
  hipLaunchKernelGGL(kv_tiles_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_global(const GlobalArgs& a, hipStream_t st) {
  if (a.S < 1 || a.S_pad % kBN || a.S_pad < a.S || a.G * a.P != 128 || a.n_units != a.B * a.Hkv ||
      a.n_qtiles != (a.S + a.P - 1) / a.P)
    return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.n_units * a.n_qtiles;
  hipLaunchKernelGGL(attn_global_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace zg
