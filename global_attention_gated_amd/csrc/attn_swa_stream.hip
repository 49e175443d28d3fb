// Streaming gated sliding-window attention (SWA) prefill for gfx950 (CDNA4, wave64, MFMA).
//
// Method (ZGCM-1 paper summaries: onedev.kr "How it works"; jaehun.me "How Gated SWA Behaves"):
//   q_hat = RoPE(RMSNorm(q) w_q), k_hat likewise, per (token, head);
//   out_i = softmax_{i-W < j <= i}(q_hat_i . k_hat_j / sqrt(D)) v_j  (.)  sigmoid(g_i).
//
// Design.  An SWA layer reads q, gate and writes out (8 KiB per token each) and reads k, v (2 KiB per token
// each): it is bound by HBM, not by the MFMAs (about 73 flop per byte).  A tile-per-work-group kernel pays
// several dependent HBM round trips per work-group for a few tiles of work; this kernel instead streams:
//   - one work-group of 8 waves owns a run of consecutive positions of one (sequence, KV head) and walks it
//     in steps of 32 positions; the 128 rows of a step are the 4 query heads of the group (GQA group 4) x 32
//     positions, 16 rows per wave (wave w: head w/2, positions 16(w%2) .. +15), one query per lane column
//     (S^T = K Q^T, O^T = V^T P^T on v_mfma_f32_16x16x32_f16).  Two waves per SIMD overlap one another's
//     softmax, memory waits and MFMAs; the LDS (ring, gate and q tiles: 144 KiB) allows one work-group per CU;
//   - the keys of the window live in a 5-slot LDS ring of 32-key tiles (a 32-position step with W <= 128
//     sees at most 5 tiles); each step adds one tile.  The whole window of a step is scored at once (ten
//     independent 16-key score chains per wave) and normalised with one exact max per query;
//   - while a step computes, the next step's q rows and the step's gate rows (straight into LDS with buffer
//     loads, each wave its own 16 rows) and the next key/value tile are in flight, so HBM latency hides
//     behind the compute and no registers hold data in flight beyond one key/value row per thread;
//   - k_hat = RoPE(RMSNorm(k) w_k) is computed in the tile loader (16 lanes per key row), rounded to bf16
//     as in the KV cache and stored as fp16, so the layer needs no separate key pass;
//   - the epilogue applies sigmoid(gate) in the MFMA output layout from the LDS gate rows, writes the bf16
//     result back in place, and 16 lanes store each 256-byte output row.
// The LDS tiles use XOR-swizzled 16-byte chunks instead of padding: reads of one chunk by 16 lanes of 16
// different rows hit 16 different bank groups.
//
// Precision as in the tile kernel: q_hat and P rounded to fp16, k_hat and v exact in fp16, fp32
// accumulation and softmax.
#include "common.h"
#include "launch.h"

namespace zg {
namespace {

constexpr int kTK = 32;        // keys per ring tile
constexpr int kRing = 5;       // ring slots
constexpr int kStep = 32;      // positions per step
constexpr int kGroup = 4;      // query heads per KV head handled here
constexpr int kThreads = 512;  // 8 waves
constexpr int kBlocks = 2 * kRing;   // 16-key score blocks of a step's window

typedef float floatx4 __attribute__((ext_vector_type(4)));

// LDS geometry (bytes)
constexpr int kKTile = kTK * 256;        // 32 key rows x 16 chunks of 16 B
constexpr int kVTile = kHeadDim * 64;    // 128 dim rows x 4 chunks of 8 keys
constexpr int kGO = 128 * 256;           // 128 rows x 16 chunks (gate in, output out)
constexpr int kQS = 128 * 256;           // 128 q rows of the next step; wave w owns rows 16w..16w+15

__device__ __forceinline__ int k_off(int slot, int key, int chunk) {       // chunk 0..15 of key row
  return slot * kKTile + key * 256 + ((chunk ^ (key & 15)) << 4);
}
__device__ __forceinline__ int vt_off(int slot, int dim, int chunk) {      // chunk 0..3 (8 keys) of dim row
  return slot * kVTile + dim * 64 + ((chunk ^ ((dim >> 2) & 3)) << 4);
}
__device__ __forceinline__ int go_off(int row, int chunk) {                // chunk 0..15 of a 256-byte row
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}

// Stored position of key k (0..31) in a V^T tile row.  A PV MFMA k-step covers the 32 keys of one tile; lane
// group g (lanes 16g..16g+15) holds P for keys 4g..4g+3 (score block 0 of the tile) and 16+4g..16+4g+3 (block
// 1), so those 8 keys are stored contiguously at 8g: key 16h + 4g + e sits at 8g + 4h + e.
__device__ __forceinline__ int vt_col(int k) {
  return 8 * ((k >> 2) & 3) + 4 * (k >> 4) + (k & 3);
}

// Chunks 4t + g (t = 0..3) of row r of a swizzled 256-byte-row LDS buffer that this wave filled with buffer
// loads into LDS, in one asm block that also waits for the reads.  Written out because the compiler, seeing LDS
// reads after loads into LDS, would otherwise wait for every memory operation in flight (including the
// previous step's output stores); the caller has waited for the loads that filled the row.
__device__ __forceinline__ void read_row4(const unsigned char* buf, int r, int g, uint4 (&out)[4]) {
  uint32_t ad[4];
#pragma unroll
  for (int t = 0; t < 4; t++)
    ad[t] = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(buf + go_off(r, 4 * t + g));
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
}

// Work-group barrier that orders LDS only: this wave's LDS reads and writes complete (lgkmcnt 0), then
// s_barrier; the memory clobber keeps the compiler from moving memory accesses across it.  __syncthreads()
// (and any fence over LDS, since loads into LDS go through the vector-memory path) would also wait for every
// global load in flight and drain the next step's prefetches at each barrier.  LDS filled by loads into LDS is
// covered by explicit vm-counter waits before the barriers that publish it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt with vmcnt = n (0..15) and the other counters not waited for (the immediate packs vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8)
#define ZG_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((n) | (7 << 4) | (15 << 8))

__global__ void __launch_bounds__(kThreads, 1) attn_swa_stream_kernel(SwaStreamArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char Ks[kRing * kKTile];
  __shared__ __attribute__((aligned(16))) unsigned char Vt[kRing * kVTile];
  __shared__ __attribute__((aligned(16))) unsigned char GO[kGO];
  __shared__ __attribute__((aligned(16))) unsigned char QS[kQS];
  __shared__ __attribute__((aligned(16))) uint16_t Wn[2 * kHeadDim];   // w_q, w_k
  __shared__ double Fr[kMaxRotPairs];                                   // RoPE inv_freq_rev

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: descriptors, LDS bases
  const int l16 = lane & 15, g = lane >> 4;
  const int head = wave >> 1, half = wave & 1;   // this wave's head and half step
  const int qrow = 16 * wave + l16;              // this lane's query row in QS / GO: 32 head + position

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

  // ---- key / value tile loader: thread = (key row lr, 16-byte chunk lc).  The 16 lanes of one key row are one
  // DPP row, which the k_hat prologue reduces over.  Tiles at or past the sequence end (and the tile after a
  // run's last step) read as zero through an empty descriptor, so every step issues the same loads.
  const int lr = tid >> 4, lc = tid & 15;
  uint4 kraw, vraw;
  auto load_kv = [&](int tile) {
    const int t0 = tile * kTK;
    const int rows = max(0, min(kTK, a.S - t0));
    const int nbytes = rows > 0 ? (int)(((rows - 1) * rowHkv + kHeadDim) * 2) : 0;
    const int64_t base = (int64_t)min(t0, a.S - 1) * rowHkv;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kb + base), (short)0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vb + base), (short)0, nbytes, 0x00020000);
    const int off = (int)((lr * rowHkv + 8 * lc) * 2);
    kraw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
    vraw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
  };
  auto store_kv = [&](int tile) {
    const int slot = tile % kRing;
    float wk[8], f[8];
    unpack8(*reinterpret_cast<const uint4*>(Wn + kHeadDim + 8 * lc), wk);
    unpack8(kraw, f);
    norm_rope8_g16_w(f, wk, lc, (int64_t)tile * kTK + lr, a.eps, a.rot_pairs, Fr);
    // the KV-cache value of k_hat (bf16, nearest-even), held exactly as fp16 for the MFMA
    *reinterpret_cast<uint4*>(Ks + k_off(slot, lr, lc)) = bf16x8_to_f16x8(pack8(f));
    // v: dim 8lc+e of key lr -> V^T row 8lc+e, stored column vt_col(lr)
    const uint4 v8 = bf16x8_to_f16x8(vraw);
    const uint32_t vw[4] = {v8.x, v8.y, v8.z, v8.w};
    const int col = vt_col(lr);
#pragma unroll
    for (int e = 0; e < 8; e++)
      *reinterpret_cast<uint16_t*>(Vt + vt_off(slot, 8 * lc + e, col >> 3) + (col & 7) * 2) =
          (uint16_t)(vw[e >> 1] >> (16 * (e & 1)));
  };

  // ---- q rows and gate rows of a step -> QS / GO, straight from HBM (buffer loads with LDS as the destination,
  // 64 lanes x 16 B per instruction).  Wave w loads its own 16 rows: lane l of instruction k fills row
  // 16w + 4k + l/16 (position 16(w%2) + 4k + l/16 of the step, head w/2), chunk position l%16, which holds the
  // row's chunk (l%16) ^ (row%16).  The descriptor covers the wave's 16 positions and ends with the sequence
  // (rows past it read as zero; their outputs are computed but not stored), so the per-lane byte offsets hold
  // for every step: 4 registers for the whole kernel.
  uint32_t qg_off[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int rr = 4 * k + (lane >> 4);                   // position within the wave's 16, = row % 16
    const int c = (lane & 15) ^ rr;
    qg_off[k] = (uint32_t)(((int64_t)rr * rowHq + head * kHeadDim + 8 * c) * 2);
  }
  auto load_rows = [&](const uint16_t* base, unsigned char* dst, int i0, bool live) {
    const int p0 = i0 + 16 * half;
    const int nvalid = live ? min(16, a.S - p0) : 0;
    const int bytes = nvalid > 0 ? (int)(((int64_t)(nvalid - 1) * rowHq + kGroup * kHeadDim) * 2) : 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (int64_t)min(p0, a.S - 1) * rowHq), (short)0, bytes, 0x00020000);
#pragma unroll
    for (int k = 0; k < 4; k++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + (16 * wave + 4 * k) * 256),
                                               16, (int)qg_off[k], 0, 0, 0);
  };

  // ---- the norm weights and RoPE frequencies, once, into LDS (global loads issued later would wait behind
  // the streaming loads: the vector-memory counter retires in order); the ring starts as zeros: the slots of
  // tiles before position 0 are read (and masked) by the first steps
  for (int x = tid; x < kRing * kKTile / 16; x += kThreads) reinterpret_cast<uint4*>(Ks)[x] = make_uint4(0u, 0u, 0u, 0u);
  for (int x = tid; x < kRing * kVTile / 16; x += kThreads) reinterpret_cast<uint4*>(Vt)[x] = make_uint4(0u, 0u, 0u, 0u);
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
  load_rows(qb, QS, p_start, true);
  // w_q for this lane's 32 dims (chunks 4t + g), once
  float wq[4][8];
#pragma unroll
  for (int t = 0; t < 4; t++) unpack8(*reinterpret_cast<const uint4*>(Wn + 8 * (4 * t + g)), wq[t]);
  // RoPE of the lane's query rows in chunks 4t + g, t = 0, 1 (pairs 4(4t + g) + m: every pair below 32), carried
  // along the steps: the lane's position advances by one step's 32 positions, so each pair's (cos, sin) advances
  // by a fixed rotation.  Pairs at or past rot_pairs stay at (1, 0).  Rows past the sequence end follow the same
  // progression; their outputs are not stored.
  float rc[2][4], rs[2][4], dc[2][4], dsn[2][4];
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int pi = 4 * (4 * t + g) + m;
      rc[t][m] = 1.0f; rs[t][m] = 0.0f; dc[t][m] = 1.0f; dsn[t][m] = 0.0f;
      if (pi < a.rot_pairs) {
        rope_cs((int64_t)p_start + 16 * half + l16, Fr[pi], rc[t][m], rs[t][m]);
        rope_cs(kStep, Fr[pi], dc[t][m], dsn[t][m]);
      }
    }

  // MFMA operand offsets within a tile (bytes): K row 16kh + l16, chunk 4t + g (t = 0..3); V^T row 16db + l16,
  // chunk g (stored keys 8g..8g+7)
  const half2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  for (int c = 0; c < n_steps; c++) {
    const int i0 = p_start + c * kStep;
    const int T = i0 / kTK;
    const int i = i0 + 16 * half + l16;           // this lane's query position
    const int qlo = i0 + 16 * half;               // the wave's positions qlo .. qlo+15
    // this wave's q rows have landed; the previous step's 4 output stores, issued after them, may still be in
    // flight (the vm counter counts stores too, in order)
    if (c == 0) ZG_WAIT_VM(0);
    else ZG_WAIT_VM(4);
    lds_barrier();                 // the previous step's ring store is visible and its GO reads are done

    // ---- q_hat of this step: RMSNorm * w_q, partial RoPE, scale by log2(e)/sqrt(D), round to fp16
    // (MFMA B operand of k-step t: lane holds q_hat[query l16][8(4t + g) .. +8])
    half8 qf[4];
    {
      uint4 qr[4];
      read_row4(QS, qrow, g, qr);
      float f[4][8];
      float ss = 0.f;
#pragma unroll
      for (int t = 0; t < 4; t++) {
        unpack8(qr[t], f[t]);
#pragma unroll
        for (int e = 0; e < 8; e++) ss += f[t][e] * f[t][e];
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float inv = rsqrtf(ss * (1.0f / kHeadDim) + a.eps) * a.q_scale;
#pragma unroll
      for (int t = 0; t < 4; t++) {
#pragma unroll
        for (int e = 0; e < 8; e++) f[t][e] = f[t][e] * inv * wq[t][e];
        if (t < 2) {
#pragma unroll
          for (int m = 0; m < 4; m++) {
            const float x0 = f[t][2 * m], x1 = f[t][2 * m + 1];
            f[t][2 * m] = x0 * rc[t][m] - x1 * rs[t][m];
            f[t][2 * m + 1] = x0 * rs[t][m] + x1 * rc[t][m];
            const float c1 = rc[t][m] * dc[t][m] - rs[t][m] * dsn[t][m];
            rs[t][m] = rs[t][m] * dc[t][m] + rc[t][m] * dsn[t][m];
            rc[t][m] = c1;
          }
        } else {
          rope8(f[t], 8 * (4 * t + g), min(i, a.S - 1), a.rot_pairs, Fr);
        }
#pragma unroll
        for (int e = 0; e < 8; e++) qf[t][e] = (_Float16)f[t][e];
      }
    }
    // this step's gate rows, the next key/value tile and the next step's q rows (into QS: this wave has consumed
    // its rows above), in that order, all in flight during this step's compute; past the run's last step the
    // loads are empty, so the counts stay the same
    const bool more = c + 1 < n_steps;
    load_rows(gb, GO, i0, true);
    load_kv(more ? T + 1 : n_tiles);
    load_rows(qb, QS, i0 + kStep, more);

    // ---- the whole window of the step: score blocks of 16 keys, block kb = 2j + kh covering keys
    // 32(T - 4 + j) + 16kh .. +15 (tiles before position 0 sit in zero-filled slots and are masked)
    int slot_k[kRing], slot_v[kRing];
#pragma unroll
    for (int j = 0; j < kRing; j++) {
      const int sl = (T - (kRing - 1) + j + kRing) % kRing;   // ring slot of tile T-4+j (T-4 >= -4)
      slot_k[j] = sl * kKTile;
      slot_v[j] = sl * kVTile;
    }
    floatx4 sacc[kBlocks];
#pragma unroll
    for (int kb = 0; kb < kBlocks; kb++) sacc[kb] = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; t++)
#pragma unroll
      for (int kb = 0; kb < kBlocks; kb++) {
        const half8 kf = *reinterpret_cast<const half8*>(Ks + slot_k[kb >> 1] + k_off(0, 16 * (kb & 1) + l16, 4 * t + g));
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[t], sacc[kb], 0, 0, 0);
      }
    // mask: key visible iff 0 <= i - key < min(W, i + 1) (one unsigned compare); blocks wholly inside every
    // window of the wave's 16 queries skip it.  C layout: lane (l16, g) holds keys 4g .. 4g+3 of the block.
    {
      const unsigned lim = (unsigned)min(a.window, i + 1);
#pragma unroll
      for (int kb = 0; kb < kBlocks; kb++) {
        const int kt = (T - (kRing - 1)) * kTK + 16 * kb;
        if (!(kt >= 0 && kt + 15 <= qlo && kt >= qlo + 16 - a.window)) {
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const int key = kt + 4 * g + e;
            if ((unsigned)(i - key) >= lim) sacc[kb][e] = -INFINITY;
          }
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kBlocks; kb++) mx = fmaxf(mx, fmaxf(fmaxf(sacc[kb][0], sacc[kb][1]), fmaxf(sacc[kb][2], sacc[kb][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));   // finite: every query sees its own key
    // P = exp2(s - m) rounded to fp16; the row sum adds the same rounded values.  O^T = V^T P^T, one k-step per
    // tile: lane (l16, g) supplies P for keys 4g..4g+3 and 16+4g..16+4g+3 of the tile (= stored keys 8g..8g+7)
    floatx4 acc_o[8];
#pragma unroll
    for (int db = 0; db < 8; db++) acc_o[db] = (floatx4){0.f, 0.f, 0.f, 0.f};
    float l_run = 0.f;
#pragma unroll
    for (int j = 0; j < kRing; j++) {
      uint32_t wp[4];
#pragma unroll
      for (int e = 0; e < 2; e++) {
        wp[e] = pack_f16(__builtin_amdgcn_exp2f(sacc[2 * j][2 * e] - mx), __builtin_amdgcn_exp2f(sacc[2 * j][2 * e + 1] - mx));
        wp[2 + e] = pack_f16(__builtin_amdgcn_exp2f(sacc[2 * j + 1][2 * e] - mx),
                             __builtin_amdgcn_exp2f(sacc[2 * j + 1][2 * e + 1] - mx));
      }
#pragma unroll
      for (int e = 0; e < 4; e++) l_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2, wp[e]), ones, l_run, false);
      const half8 pf = __builtin_bit_cast(half8, make_uint4(wp[0], wp[1], wp[2], wp[3]));
#pragma unroll
      for (int db = 0; db < 8; db++) {
        const half8 va = *reinterpret_cast<const half8*>(Vt + slot_v[j] + vt_off(0, 16 * db + l16, g));
        acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pf, acc_o[db], 0, 0, 0);
      }
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    const float inv_l = 1.0f / l_run;
    // training: the log-sum-exp of the query's scores (natural log; scores in log2 units are s log2(e))
    if (a.lse && g == 0 && i < p_end)
      a.lse[((int64_t)b * a.Hq + kvh * kGroup + head) * a.S + i] = (mx + __log2f(l_run)) * 0.6931471805599453f;

    // ---- epilogue.  acc_o[db][e] is dim d = 16db + 4g + e of this lane's query row.
    // This wave's gate rows have landed in GO: they were issued before the next key/value tile (2 loads) and
    // the next step's q rows (4 loads), which may stay in flight.
    ZG_WAIT_VM(6);
    lds_barrier();                   // ... and every wave's; all waves are past the ring reads
    if (more) {
      ZG_WAIT_VM(4);                 // the next key/value tile (the next step's q rows may stay in flight)
      store_kv(T + 1);               // into the slot of tile T-4, which no later step reads
    }
#pragma unroll
    for (int db = 0; db < 8; db++) {
      const int d = 16 * db + 4 * g;
      unsigned char* p = GO + go_off(qrow, d >> 3) + (d & 7) * 2;
      const uint2 gw = *reinterpret_cast<const uint2*>(p);
      const float gv[4] = {bf16lo(gw.x), bf16hi(gw.x), bf16lo(gw.y), bf16hi(gw.y)};
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; e++)   // sigmoid(g) = 1 / (1 + e^-g): v_exp and v_rcp, exact at g = +-inf
        o[e] = acc_o[db][e] * __builtin_amdgcn_rcpf(__builtin_fmaf(l_run, __expf(-gv[e]), l_run));
      *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
    }
    lds_barrier();
    // coalesced store, 16 lanes per 256-byte row, through a descriptor over this step's valid positions:
    // rows past the run's end fall outside it and are dropped, so every step issues exactly 4 stores
    {
      const int nvalid = min(kStep, p_end - i0);
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(ob + (int64_t)i0 * rowHq), (short)0, (int)(nvalid * rowHq * 2), 0x00020000);
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int cc = tid + kThreads * k;
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
  // about one work-group per CU (256 CUs; the LDS ring, gate and q tiles of 8 waves take one CU each)
  const int64_t per = ((int64_t)S * n_units + 255) / 256;
  int run = (int)((per + kStep - 1) / kStep) * kStep;
  return run < kStep ? kStep : run;
}

hipError_t launch_swa_stream(const SwaStreamArgs& a, hipStream_t st) {
  if (a.G != kGroup || a.window < 1 || a.window > kTK * (kRing - 1) || a.run % kStep) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.n_units * ((a.S + a.run - 1) / a.run);
  hipLaunchKernelGGL(attn_swa_stream_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace zg
