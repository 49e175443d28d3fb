// Streaming gated sliding-window attention (SWA) prefill for gfx950 (CDNA4, wave64, MFMA).
//
// Method (ZGCM-1 paper summaries: onedev.kr "How it works"; jaehun.me "How Gated SWA Behaves"):
//   q_hat = RoPE(RMSNorm(q) w_q), k_hat likewise, per (token, head);
//   out_i = softmax_{i-W < j <= i}(q_hat_i . k_hat_j / sqrt(D)) v_j  (.)  sigmoid(g_i).
//
// Design.  An SWA layer reads q, gate and writes out (8 KiB per token each) and reads k, v (2 KiB per token
// each): it is bound by HBM, not by the MFMAs (about 73 flop per byte).  A tile-per-work-group kernel pays
// several dependent HBM round trips per work-group for a few tiles of work; this kernel instead streams:
//   - one work-group of 4 waves owns a run of consecutive positions of one (sequence, KV head) and walks it
//     in steps of 32 positions; the 128 rows of a step are the 4 query heads of the group (GQA group 4) x 32
//     positions, one head per wave and one query per lane column (S^T = K Q^T, O^T = V^T P^T on
//     v_mfma_f32_32x32x16_f16);
//   - the keys of the window live in a 5-slot LDS ring of 32-key tiles (a 32-position step with W <= 128
//     sees at most 5 tiles); each step adds one tile;
//   - while a step computes, the next step's q rows (straight into LDS, global_load_lds) and next key/value
//     tile are already in flight, and the step's gate tile streams into LDS as well, so HBM latency hides
//     behind the MFMAs and no registers hold data in flight beyond one key/value tile;
//   - k_hat = RoPE(RMSNorm(k) w_k) is computed in the tile loader (16 lanes per key row), rounded to bf16
//     as in the KV cache and stored as fp16, so the layer needs no separate key pass;
//   - the epilogue applies sigmoid(gate) in the MFMA output layout from the LDS gate tile, writes the bf16
//     result back in place, and 16 lanes store each 256-byte output row.
// The LDS tiles use XOR-swizzled 16-byte chunks instead of padding: reads of one chunk by 16 lanes of 16
// different rows hit 16 different bank groups.
//
// Precision as in the tile kernel: q_hat and P rounded to fp16, k_hat and v exact in fp16, fp32
// accumulation, running max raised lazily by more than 2^8 only.
#include "common.h"
#include "launch.h"

namespace zg {
namespace {

constexpr int kTK = 32;        // keys per ring tile
constexpr int kRing = 5;       // ring slots
constexpr int kStep = 32;      // positions per step
constexpr int kGroup = 4;      // query heads per KV head handled here

// LDS geometry (bytes)
constexpr int kKTile = kTK * 256;        // 32 key rows x 16 chunks of 16 B
constexpr int kVTile = kHeadDim * 64;    // 128 dim rows x 4 chunks of 8 keys
constexpr int kGO = 128 * 256;           // 128 rows x 16 chunks (gate in, output out)
constexpr int kQS = 128 * 256;           // 128 q rows of the next step; wave w owns rows 32w..32w+31

__device__ __forceinline__ int k_off(int slot, int key, int chunk) {       // chunk 0..15 of key row
  return slot * kKTile + key * 256 + ((chunk ^ (key & 15)) << 4);
}
__device__ __forceinline__ int vt_off(int slot, int dim, int chunk) {      // chunk 0..3 (8 keys) of dim row
  return slot * kVTile + dim * 64 + ((chunk ^ ((dim >> 2) & 3)) << 4);
}
__device__ __forceinline__ int go_off(int row, int chunk) {                // chunk 0..15 of a 256-byte row
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}

// V^T column of key k (0..31) in a tile: within each 16-key group the quads 1 and 2 swap places, so the 8
// keys an MFMA lane needs for one PV k-step (lane half hi holds S^T rows 4hi..4hi+3 and 8+4hi..8+4hi+3)
// are contiguous.
__device__ __forceinline__ int vt_col(int k) {
  const int q = (k >> 2) & 3;
  return (k & 16) + 4 * (q == 1 ? 2 : q == 2 ? 1 : q) + (k & 3);
}

__device__ __forceinline__ uint32_t dw(const uint4& w, int i) { return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w; }

// Chunks 2t + hi (t = 0..7) of row r of a swizzled 256-byte-row LDS buffer that this wave filled with
// global_load_lds, in one asm block that also waits for the reads.  Written out because the compiler,
// seeing LDS reads after loads into LDS, would otherwise wait for every memory operation in flight
// (including the previous step's output stores); the caller has waited for the loads that filled the row.
__device__ __forceinline__ void read_row8(const unsigned char* buf, int r, int hi, uint4 (&out)[8]) {
  uint32_t ad[8];
#pragma unroll
  for (int t = 0; t < 8; t++)
    ad[t] = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(buf + go_off(r, 2 * t + hi));
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]), "=&v"(out[5]), "=&v"(out[6]),
        "=&v"(out[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
      : "memory");
}

// Work-group barrier that orders LDS only: this wave's LDS reads and writes complete (lgkmcnt 0), then
// s_barrier; the memory clobber keeps the compiler from moving memory accesses across it.  __syncthreads()
// (and any fence over LDS, since global_load_lds writes LDS through the vector-memory path) would also wait
// for every global load in flight and drain the next step's prefetches at each barrier.  LDS filled by
// global_load_lds is covered by explicit vm-counter waits before the barriers that publish it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Launch bounds ask for two work-groups' worth of registers per SIMD (256 VGPRs, no AGPRs) even though the
// LDS allows one work-group per CU: the MFMAs then keep their accumulators in VGPRs next to the softmax.
__global__ void __launch_bounds__(256, 2) __attribute__((amdgpu_num_vgpr(256))) attn_swa_stream_kernel(SwaStreamArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char Ks[kRing * kKTile];
  __shared__ __attribute__((aligned(16))) unsigned char Vt[kRing * kVTile];
  __shared__ __attribute__((aligned(16))) unsigned char GO[kGO];
  __shared__ __attribute__((aligned(16))) unsigned char QS[kQS];
  __shared__ __attribute__((aligned(16))) uint16_t Wn[2 * kHeadDim];   // w_q, w_k
  __shared__ double Fr[kMaxRotPairs];                                   // RoPE inv_freq_rev

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // consecutive work-groups walk the (sequence, KV head) units first: with B*Hkv a multiple of 8, all runs
  // of one unit land on one XCD, whose L2 then serves the tiles two neighbouring runs share
  const int unit = blockIdx.x % a.n_units;
  const int run = blockIdx.x / a.n_units;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int p_start = run * a.run;
  if (p_start >= a.S) return;
  const int p_end = min(p_start + a.run, a.S);
  const int n_steps = (p_end - p_start + kStep - 1) / kStep;
  const int n_tiles = (a.S + kTK - 1) / kTK;
  const int jmax = min(kRing - 1, (a.window + kTK - 2) / kTK);   // oldest ring tile a step can need

  const int64_t rowHq = (int64_t)a.Hq * kHeadDim;      // elements per token of q / gate / out
  const int64_t rowHkv = (int64_t)a.Hkv * kHeadDim;    // elements per token of k / v
  const uint16_t* qb = a.q + (int64_t)b * a.S * rowHq + (int64_t)(kvh * kGroup) * kHeadDim;
  const uint16_t* gb = a.gate + (int64_t)b * a.S * rowHq + (int64_t)(kvh * kGroup) * kHeadDim;
  uint16_t* ob = a.out + (int64_t)b * a.S * rowHq + (int64_t)(kvh * kGroup) * kHeadDim;
  const uint16_t* kb = a.k + (int64_t)b * a.S * rowHkv + (int64_t)kvh * kHeadDim;
  const uint16_t* vb = a.v + (int64_t)b * a.S * rowHkv + (int64_t)kvh * kHeadDim;

  // ---- key / value tile loader.  K: thread = (key rows lr and lr+16, 16-byte chunk lc), the 16 lanes of one
  // key row are one DPP row, which the k_hat prologue reduces over.  V: thread = (adjacent keys 2lr, 2lr+1,
  // dims 8lc..8lc+7), so each V^T row gets both keys in one 4-byte store.
  const int lr = tid >> 4, lc = tid & 15;
  uint4 kraw[2], vraw[2];
  auto load_kv = [&](int tile) {
    const int t0 = tile * kTK;
    const int rows = min(kTK, a.S - t0);
    const int nbytes = (int)(((rows - 1) * rowHkv + kHeadDim) * 2);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kb + (int64_t)t0 * rowHkv), (short)0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vb + (int64_t)t0 * rowHkv), (short)0, nbytes, 0x00020000);
    // rows past the sequence end fall outside the descriptors and read as zero
#pragma unroll
    for (int rr = 0; rr < 2; rr++) {
      kraw[rr] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rk, (int)(((lr + 16 * rr) * rowHkv + 8 * lc) * 2), 0, 0));
      vraw[rr] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rv, (int)(((2 * lr + rr) * rowHkv + 8 * lc) * 2), 0, 0));
    }
  };
  auto store_kv = [&](int tile) {
    const int slot = tile % kRing;
    float wk[8];
    unpack8(*reinterpret_cast<const uint4*>(Wn + kHeadDim + 8 * lc), wk);
#pragma unroll
    for (int rr = 0; rr < 2; rr++) {
      const int key = lr + 16 * rr;
      float f[8];
      unpack8(kraw[rr], f);
      norm_rope8_g16_w(f, wk, lc, (int64_t)tile * kTK + key, a.eps, a.rot_pairs, Fr);
      // the KV-cache value of k_hat (bf16, nearest-even), held exactly as fp16 for the MFMA
      *reinterpret_cast<uint4*>(Ks + k_off(slot, key, lc)) = bf16x8_to_f16x8(pack8(f));
    }
    // v: dim 8lc+e of keys 2lr, 2lr+1 -> one 4-byte store into V^T row 8lc+e
    const uint4 v0 = bf16x8_to_f16x8(vraw[0]), v1 = bf16x8_to_f16x8(vraw[1]);
    const int col = vt_col(2 * lr);
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t w = __builtin_amdgcn_perm(dw(v1, e >> 1), dw(v0, e >> 1), sel);
      *reinterpret_cast<uint32_t*>(Vt + vt_off(slot, 8 * lc + e, col >> 3) + (col & 7) * 2) = w;
    }
  };

  // ---- q rows and gate rows of a step -> QS / GO, straight from HBM (buffer loads with LDS as the destination,
  // 64 lanes x 16 B per instruction).  Wave w loads the 32 rows of its own head kvh*4 + w: lane l of instruction
  // k fills row 32w + 4k + l/16 (position i0 + 4k + l/16), chunk position l%16, which holds the row's chunk
  // (l%16) ^ (row%16).  Rows 0..15 and 16..31 of the step go through two descriptors whose ranges end with the
  // sequence (rows past it read as zero; their outputs are computed but not stored), so the per-lane byte
  // offsets are the same for both halves and for every step: 4 registers for the whole kernel.
  uint32_t qg_off[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int rr = 4 * k + (lane >> 4);                   // position within the half step, 0..15
    const int c = (lane & 15) ^ rr;
    qg_off[k] = (uint32_t)(((int64_t)rr * rowHq + wave * kHeadDim + 8 * c) * 2);
  }
  auto half_rows = [&](const uint16_t* base, int p0) {    // positions p0 .. p0+15, clipped to the sequence
    const int nvalid = min(kStep / 2, a.S - p0);
    const int bytes = nvalid > 0 ? (int)(((int64_t)(nvalid - 1) * rowHq + kGroup * kHeadDim) * 2) : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)min(p0, a.S - 1) * rowHq), (short)0, bytes,
                                             0x00020000);
  };
  auto load_rows = [&](const uint16_t* base, unsigned char* dst, int i0) {
    const __amdgpu_buffer_rsrc_t r0 = half_rows(base, i0), r1 = half_rows(base, i0 + kStep / 2);
#pragma unroll
    for (int k = 0; k < 8; k++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(k < 4 ? r0 : r1,
                                               (__attribute__((address_space(3))) void*)(dst + (32 * wave + 4 * k) * 256),
                                               16, (int)qg_off[k & 3], 0, 0, 0);
  };
  auto load_q = [&](int i0) { load_rows(qb, QS, i0); };
  auto load_gate = [&](int i0) { load_rows(gb, GO, i0); };

  // ---- the norm weights and RoPE frequencies, once, into LDS (global loads issued later would wait behind
  // the streaming loads: the vector-memory counter retires in order)
  // the ring starts as zeros: the slots of tiles before position 0 are read (and masked) by the first steps
  for (int x = tid; x < kRing * kKTile / 16; x += 256) reinterpret_cast<uint4*>(Ks)[x] = make_uint4(0u, 0u, 0u, 0u);
  for (int x = tid; x < kRing * kVTile / 16; x += 256) reinterpret_cast<uint4*>(Vt)[x] = make_uint4(0u, 0u, 0u, 0u);
  if (tid < 32) reinterpret_cast<uint4*>(Wn)[tid] = *reinterpret_cast<const uint4*>((tid < 16 ? a.qw : a.kw) + 8 * (tid & 15));
  if (tid < kMaxRotPairs) Fr[tid] = a.inv_freq_rev[tid];
  lds_barrier();

  // ---- prologue: the first step's window tiles, then its q rows
  {
    const int T0 = p_start / kTK;
    for (int j = jmax; j >= 0; j--) {
      const int tile = T0 - j;
      if (tile < 0) continue;
      load_kv(tile);
      store_kv(tile);
    }
  }
  load_q(p_start);

  const half2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  for (int c = 0; c < n_steps; c++) {
    const int i0 = p_start + c * kStep;
    const int T = i0 / kTK;
    const int i = i0 + l32;
    const int ic = min(i, a.S - 1);
    // this wave's q rows have landed; the previous step's 8 output stores, issued after them, may still be
    // in flight (the vm counter counts stores too, in order)
    if (c == 0) __builtin_amdgcn_s_waitcnt(0);
    else __builtin_amdgcn_s_waitcnt(8 | (7 << 4) | (15 << 8));
    lds_barrier();                 // the previous step's ring store is visible and its GO reads are done

    // ---- q_hat of this step: RMSNorm * w_q, partial RoPE, scale by log2(e)/sqrt(D), round to fp16
    // (MFMA B operand: lane holds q_hat[query l32][16t+8hi..+8])
    half8 qf[8];
    {
      const int r = 32 * wave + l32;
      uint4 qr[8];
      read_row8(QS, r, hi, qr);
      float f[8][8];
      float ss = 0.f;
#pragma unroll
      for (int t = 0; t < 8; t++) {
        unpack8(qr[t], f[t]);
#pragma unroll
        for (int e = 0; e < 8; e++) ss += f[t][e] * f[t][e];
      }
      ss = xor32_sum(ss);
      const float inv = rsqrtf(ss * (1.0f / kHeadDim) + a.eps);
#pragma unroll
      for (int t = 0; t < 8; t++) {
        float w[8];
        unpack8(*reinterpret_cast<const uint4*>(Wn + 16 * t + 8 * hi), w);
#pragma unroll
        for (int e = 0; e < 8; e++) f[t][e] = f[t][e] * inv * w[e];
        rope8(f[t], 16 * t + 8 * hi, ic, a.rot_pairs, Fr);
#pragma unroll
        for (int e = 0; e < 8; e++) qf[t][e] = (_Float16)(f[t][e] * a.q_scale);
      }
    }
    // this step's gate tile, the next key/value tile and the next step's q rows (into QS: this wave has
    // consumed its rows above), in that order, all in flight during this step's compute
    const bool more = c + 1 < n_steps;
    const bool next_tile = more && T + 1 < n_tiles;
    load_gate(i0);
    if (next_tile) load_kv(T + 1);
    if (more) load_q(i0 + kStep);

    // ---- attention over the whole window of the step at once: its 32 queries see keys of the ring tiles
    // T-4 .. T only, so all their scores fit in registers and one exact max per query replaces the online
    // rescaling.  The five score chains are independent (S^T = K Q^T per tile, interleaved over the k-steps).
    // Tiles before the window or before position 0 are masked out (their slots hold older keys or zeros).
    int slot_k[kRing], slot_v[kRing];
#pragma unroll
    for (int j = 0; j < kRing; j++) {
      const int sl = (T - (kRing - 1) + j + kRing) % kRing;   // ring slot of tile T-4+j (T-4 >= -4)
      slot_k[j] = sl * kKTile;
      slot_v[j] = sl * kVTile;
    }
    floatx16 sacc[kRing];
#pragma unroll
    for (int j = 0; j < kRing; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) sacc[j][e] = 0.f;
#pragma unroll
    for (int t8 = 0; t8 < 8; t8++)
#pragma unroll
      for (int j = 0; j < kRing; j++) {
        const half8 kf = *reinterpret_cast<const half8*>(Ks + slot_k[j] + k_off(0, l32, 2 * t8 + hi));
        sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[t8], sacc[j], 0, 0, 0);
      }
    // mask: key visible iff 0 <= i - key < min(W, i + 1) (one unsigned compare); tiles wholly inside every
    // window of the step skip it
    {
      const unsigned lim = (unsigned)min(a.window, i + 1);
#pragma unroll
      for (int j = 0; j < kRing; j++) {
        const int kt = (T - (kRing - 1) + j) * kTK;
        if (!(kt >= 0 && kt + kTK - 1 <= i0 && kt >= i0 + kStep - a.window)) {
#pragma unroll
          for (int e = 0; e < 16; e++) {
            const int key = kt + 8 * (e >> 2) + 4 * hi + (e & 3);
            if ((unsigned)(i - key) >= lim) sacc[j][e] = -INFINITY;
          }
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kRing; j++)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(sacc[j][e], sacc[j][e + 1]));
    mx = xor32_max(mx);   // finite: every query sees its own key
    // P = exp2(s - m) rounded to fp16; the row sum adds the same rounded values.  O^T = V^T P^T (lane: dim
    // l32 of block db; keys 16h2 + 8hi .. +8 of the tile)
    floatx16 acc_o[4];
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc_o[db][e] = 0.f;
    float l_run = 0.f;
#pragma unroll
    for (int j = 0; j < kRing; j++)
#pragma unroll
      for (int h2 = 0; h2 < 2; h2++) {
        uint32_t wp[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int x = 8 * h2 + 2 * e;
          wp[e] = pack_f16(__builtin_amdgcn_exp2f(sacc[j][x] - mx), __builtin_amdgcn_exp2f(sacc[j][x + 1] - mx));
          l_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2, wp[e]), ones, l_run, false);
        }
        const half8 pf = __builtin_bit_cast(half8, make_uint4(wp[0], wp[1], wp[2], wp[3]));
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const half8 va = *reinterpret_cast<const half8*>(Vt + slot_v[j] + vt_off(0, 32 * db + l32, 2 * h2 + hi));
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf, acc_o[db], 0, 0, 0);
        }
      }

    // ---- epilogue.  acc_o[db][j] is dim d = 32db + 8(j/4) + 4hi + j%4 of row r = 32w + l32.
    const float inv_l = 1.0f / xor32_sum(l_run);
    // this wave's gate chunks have landed in GO: they were issued before the next key/value tile (4 loads)
    // and the next step's q rows (8 loads), which may stay in flight (vm counter in order; the immediate
    // packs vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8, here left at their maxima)
    if (next_tile) __builtin_amdgcn_s_waitcnt(12 | (7 << 4) | (15 << 8));
    else if (more) __builtin_amdgcn_s_waitcnt(8 | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    lds_barrier();                   // ... and every wave's; all waves are past the ring reads
    if (next_tile) store_kv(T + 1);    // into the slot of tile T-4, which no later step reads
    {
      const int r = 32 * wave + l32;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int jq = 0; jq < 4; jq++) {
          const int d = 32 * db + 8 * jq + 4 * hi;
          unsigned char* p = GO + go_off(r, d >> 3) + (d & 7) * 2;
          const uint2 g = *reinterpret_cast<const uint2*>(p);
          const float gv[4] = {bf16lo(g.x), bf16hi(g.x), bf16lo(g.y), bf16hi(g.y)};
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; e++)   // sigmoid(g) = 1 / (1 + e^-g): v_exp and v_rcp, exact at g = +-inf
            o[e] = acc_o[db][4 * jq + e] * inv_l * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[e]));
          *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
        }
    }
    lds_barrier();
    // coalesced store, 16 lanes per 256-byte row, through a descriptor over this step's valid positions:
    // rows past the run's end fall outside it and are dropped, so every step issues exactly 8 stores
    {
      const int nvalid = min(kStep, p_end - i0);
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(ob + (int64_t)i0 * rowHq), (short)0, (int)(nvalid * rowHq * 2), 0x00020000);
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const int cc = tid + 256 * k;
        const int row = cc >> 4, ch = cc & 15;
        const int off = (int)(((row & 31) * rowHq + (row >> 5) * kHeadDim + 8 * ch) * 2);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((__vector_size__(4 * sizeof(int)))) int,
                                                                  *reinterpret_cast<const uint4*>(GO + go_off(row, ch))),
                                               ro, off, 0, 0);
      }
    }
  }
}

}  // namespace

int swa_stream_run_length(int S, int n_units) {
  // about one work-group per CU (256 CUs; the LDS ring, gate tile and 4 waves take one CU each)
  const int64_t per = ((int64_t)S * n_units + 255) / 256;
  int run = (int)((per + kStep - 1) / kStep) * kStep;
  return run < kStep ? kStep : run;
}

hipError_t launch_swa_stream(const SwaStreamArgs& a, hipStream_t st) {
  if (a.G != kGroup || a.window < 1 || a.window > kTK * (kRing - 1) || a.run % kStep) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.n_units * ((a.S + a.run - 1) / a.run);
  hipLaunchKernelGGL(attn_swa_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace zg
