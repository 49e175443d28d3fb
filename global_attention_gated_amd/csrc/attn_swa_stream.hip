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
//     positions, 16 rows per wave (wave w: head w%4, positions 16(w/4) .. +15), one query per lane column
//     (S^T = K Q^T, O^T = V^T P^T on v_mfma_f32_16x16x32_f16); the LDS (ring, gate and q rows: 160 KiB) allows
//     one work-group per CU;
//   - the two wave groups (waves 0-3 and 4-7; waves w and w+4 share a SIMD) run half a step apart: a step of a
//     group is a compute phase (the window's scores, softmax, PV) and an output phase (half of the next ring tile,
//     gate, output rows, and the next step's q_hat), and one group's compute phase runs beside the other's output
//     phase, one work-group barrier between phases;
//   - the keys of the window live in a 6-slot LDS ring of 32-key tiles: a 32-position step with W <= 128 reads
//     5 tiles, and the next tile is written (one half by each group) while they are read.  The whole window of
//     a step is scored at once (ten independent 16-key score chains per wave) and normalised with one exact max
//     per query;
//   - each wave's q rows and gate rows go straight from HBM into its own LDS rows with buffer loads whose
//     destination is LDS, one step ahead, and the raw key/value rows of the next ring half into registers one
//     step ahead; no wave reads another wave's rows, so only the ring needs the barriers;
//   - k_hat = RoPE(RMSNorm(k) w_k) is computed in the ring loader (16 lanes per key row), rounded to bf16
//     as in the KV cache and stored as fp16, so the layer needs no separate key pass;
//   - the queries' RoPE (pairs of the first 64 dims; more rotary dims take the tile kernel) is carried along the
//     steps as a fixed rotation per step; a run has at most 256 steps, so the carried value is at most 256 fp32
//     rotations from the exact angle (relative error ~3e-5, against 2^-12 for q_hat's fp16 rounding);
//   - a chunk that continues a cached sequence (pos0 > 0) works in absolute positions (RoPE, mask), and the run's
//     first window takes the keys before the chunk from the layer's ring (k_hat already, bf16);
//   - the epilogue applies sigmoid(gate) in the MFMA output layout from the LDS gate rows, writes the bf16
//     result back in place, and 16 lanes store each 256-byte output row of the wave.
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
constexpr int kWinTiles = 5;   // ring tiles a 32-position step with W <= 128 reads (T-4 .. T)
constexpr int kRing = 6;       // ring slots: the window's 5 tiles and the next tile, written while they are read
constexpr int kStep = 32;      // positions per step
constexpr int kGroup = 4;      // query heads per KV head handled here
constexpr int kThreads = 512;  // 8 waves
constexpr int kBlocks = 2 * kWinTiles;   // 16-key score blocks of a step's window
constexpr int kMaxRunSteps = 256;        // steps per work-group at most (bounds the carried RoPE rotation)

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

// CACHED: a chunk at pos0 > 0 whose window starts in the layer's ring; the cache-less kernel compiles without any of it.
template <bool CACHED>
__global__ void __launch_bounds__(kThreads, 1) attn_swa_stream_kernel(SwaStreamArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char Ks[kRing * kKTile];
  __shared__ __attribute__((aligned(16))) unsigned char Vt[kRing * kVTile];
  __shared__ __attribute__((aligned(16))) unsigned char GO[kGO];
  __shared__ __attribute__((aligned(16))) unsigned char QS[kQS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: descriptors, LDS bases
  const int grp = wave >> 2;      // wave group: 0 takes positions 0..15 of every step, 1 positions 16..31
  const int head = wave & 3;      // this wave's query head within the KV head's group
  const int half = grp;
  const int l16 = lane & 15, g = lane >> 4;
  const int qrow = 16 * wave + l16;              // this lane's query row in QS / GO (16 rows per wave)

  // consecutive work-groups walk the (sequence, KV head) units first: with B*Hkv a multiple of 8, all runs
  // of one unit land on one XCD, whose L2 then serves the tiles two neighbouring runs share
  const int unit = blockIdx.x % a.n_units;
  const int run = blockIdx.x / a.n_units;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int p_start = run * a.run;
  if (p_start >= a.S) return;
  const int p_end = min(p_start + a.run, a.S);
  const int n_steps = (p_end - p_start + kStep - 1) / kStep;
  const int jmax = min(kWinTiles - 1, (a.window + kTK - 2) / kTK);   // oldest window tile a step can need

  const int64_t rowHq = (int64_t)a.Hq * kHeadDim;      // elements per token of q / gate / out
  const int64_t rowHkv = (int64_t)a.Hkv * kHeadDim;    // elements per token of k / v
  const uint16_t* qb = a.q + (int64_t)b * a.S * rowHq + (int64_t)(kvh * kGroup) * kHeadDim;
  const uint16_t* gb = a.gate + (int64_t)b * a.S * rowHq + (int64_t)(kvh * kGroup) * kHeadDim;
  uint16_t* ob = a.out + (int64_t)b * a.S * rowHq + (int64_t)(kvh * kGroup) * kHeadDim;
  const uint16_t* kb = a.k + (int64_t)b * a.S * rowHkv + (int64_t)kvh * kHeadDim;
  const uint16_t* vb = a.v + (int64_t)b * a.S * rowHkv + (int64_t)kvh * kHeadDim;

  // ---- constants held in registers (the LDS is taken whole by the ring and the row buffers): this thread's w_k
  // chunk and the RoPE frequencies of its key pairs 4lc .. 4lc+3 (the key loader: chunk lc = tid % 16 of a key row),
  // and this lane's w_q chunks 4t + g
  const int lc = tid & 15;
  const uint4 wk_raw = *reinterpret_cast<const uint4*>(a.kw + 8 * lc);
  double frk[4];
#pragma unroll
  for (int m = 0; m < 4; m++) frk[m] = 4 * lc + m < a.rot_pairs ? a.inv_freq_rev[4 * lc + m] : 0.0;
  float wq[4][8];
#pragma unroll
  for (int t = 0; t < 4; t++) unpack8(*reinterpret_cast<const uint4*>(a.qw + 8 * (4 * t + g)), wq[t]);

  // ---- key / value rows: thread (key row lr, 16-byte chunk lc); the 16 lanes of one key row are one DPP row,
  // which the k_hat prologue reduces over.  Rows at or past the sequence end read as zero through the descriptor.
  uint4 kraw, vraw;
  auto load_kv = [&](int tile, int lr, bool live = true) {   // live = false: an empty load (keeps the counts)
    const int t0 = tile * kTK;
    const int rows = live ? max(0, min(kTK, a.S - t0)) : 0;
    const int nbytes = rows > 0 ? (int)(((rows - 1) * rowHkv + kHeadDim) * 2) : 0;
    const int64_t base = (int64_t)min(max(t0, 0), a.S - 1) * rowHkv;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kb + base), (short)0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vb + base), (short)0, nbytes, 0x00020000);
    const int off = (int)((lr * rowHkv + 8 * lc) * 2);
    kraw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kCpolNT));
    vraw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kCpolNT));
  };
  // store_kv(tile, lr, cached): row lr of a tile into its ring slot.  Cached tiles (before the chunk) hold k_hat
  // already (the cache ring's bf16 values), the chunk's own tiles raw k, whose k_hat is computed here at the key's
  // absolute position (the same arithmetic as every other k_hat of the library)
  const int64_t pos0 = CACHED ? (int64_t)a.pos0 : 0;
  auto store_kv = [&](int tile, int lr, bool cached) {
    const int slot = (tile + kRing) % kRing;   // tile >= -4
    if (cached) {
      *reinterpret_cast<uint4*>(Ks + k_off(slot, lr, lc)) = bf16x8_to_f16x8(kraw);
    } else {
      float wk[8], f[8];
      unpack8(wk_raw, wk);
      unpack8(kraw, f);
      norm_rope8_g16_f(f, wk, lc, pos0 + (int64_t)tile * kTK + lr, a.eps, a.rot_pairs, [&](int i) { return frk[i & 3]; });
      // the KV-cache value of k_hat (bf16, nearest-even), held exactly as fp16 for the MFMA
      *reinterpret_cast<uint4*>(Ks + k_off(slot, lr, lc)) = bf16x8_to_f16x8(pack8(f));
    }
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
  // 16w + 4k + l/16 (position 16 half + 4k + l/16 of the step), chunk position l%16, which holds the row's chunk
  // (l%16) ^ (row%16).  The descriptor covers the wave's 16 positions and ends with the sequence (rows past it read
  // as zero; their outputs are computed but not stored), so the per-lane byte offsets hold for every step.
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
                                               16, (int)qg_off[k], 0, 0, kCpolNT);
  };

  // ---- the ring starts as zeros: the slots of tiles before position 0 are read (and masked) by the first steps
  for (int x = tid; x < kRing * kKTile / 16; x += kThreads) reinterpret_cast<uint4*>(Ks)[x] = make_uint4(0u, 0u, 0u, 0u);
  for (int x = tid; x < kRing * kVTile / 16; x += kThreads) reinterpret_cast<uint4*>(Vt)[x] = make_uint4(0u, 0u, 0u, 0u);
  lds_barrier();

  // ---- prologue: the first step's window tiles (all threads, one row chunk each).  Tiles before the chunk
  // (tile < 0) hold the positions before pos0: from the cache's ring when there is one (slot p mod W of the
  // sequence's KV head; positions below 0 stay zero), otherwise zero (and masked).
  const int T0 = p_start / kTK;
  {
    const int lr = tid >> 4;
    for (int j = jmax; j >= 0; j--) {
      const int tile = T0 - j;
      if (tile < 0) {
        if constexpr (CACHED) {
          const int64_t p = pos0 + (int64_t)tile * kTK + lr;
          kraw = vraw = make_uint4(0u, 0u, 0u, 0u);
          if (p >= 0) {
            const int64_t row = (((int64_t)b * a.Hkv + kvh) * a.window + p % a.window) * kHeadDim + 8 * lc;
            kraw = *reinterpret_cast<const uint4*>(a.ck + row);
            vraw = *reinterpret_cast<const uint4*>(a.cv + row);
          }
          store_kv(tile, lr, true);
        }
        continue;
      }
      load_kv(tile, lr);
      store_kv(tile, lr, false);
    }
  }
  // the ring tile a group writes in its next output phase, and its key rows: group 0 rows 16..31 of tile T + 1,
  // group 1 rows 0..15 of tile T + 2 (T = the step's tile; see the schedule below)
  const int hr = 16 * (1 - grp) + ((tid & 255) >> 4);
  load_rows(qb, QS, p_start, true);
  load_rows(gb, GO, p_start, true);
  load_kv(T0 + 1, hr, n_steps > 1);

  // RoPE of the lane's query rows in chunks 4t + g, t = 0, 1 (pairs 4(4t + g) + m: every pair below 32; the kernel
  // takes rot_pairs <= 32), carried along the steps: the lane's position advances by one step's 32 positions, so
  // each pair's (cos, sin) advances by a fixed rotation.  A run has at most kMaxRunSteps steps, so the carried value
  // is at most that many fp32 rotations away from the exact angle.  Pairs at or past rot_pairs stay at (1, 0).  Rows
  // past the sequence end follow the same progression; their outputs are not stored.
  float rc[2][4], rs[2][4], dc[2][4], dsn[2][4];
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int pi = 4 * (4 * t + g) + m;
      rc[t][m] = 1.0f; rs[t][m] = 0.0f; dc[t][m] = 1.0f; dsn[t][m] = 0.0f;
      if (pi < a.rot_pairs) {
        const double fr = a.inv_freq_rev[pi];
        rope_cs(pos0 + p_start + 16 * half + l16, fr, rc[t][m], rs[t][m]);
        rope_cs(kStep, fr, dc[t][m], dsn[t][m]);
      }
    }
  ZG_WAIT_VM(0);
  lds_barrier();

  // ---- q_hat of a step (MFMA B operand of k-step t: lane holds q_hat[query l16][8(4t + g) .. +8]), from the
  // lane's raw chunks 4t + g: RMSNorm * w_q, rope(f, t) on chunks t = 0, 1, scale by log2(e)/sqrt(D), round to fp16.
  // It is computed in the output phase before the step's compute phase, which then starts with its MFMAs.
  half8 qf[4];
  auto q_hat = [&](const uint4 (&qr)[4], auto rope) {
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
      rope(f[t], t);
#pragma unroll
      for (int e = 0; e < 8; e++) qf[t][e] = (_Float16)f[t][e];
    }
  };
  // the next step's q_hat from this wave's q rows in LDS, with the carried rotation (then advanced by a step)
  auto next_q = [&]() {
    uint4 qr[4];
    read_row4(QS, qrow, g, qr);
    q_hat(qr, [&](float* f, int t) {
      if (t < 2) {
#pragma unroll
        for (int m = 0; m < 4; m++) {
          const float x0 = f[2 * m], x1 = f[2 * m + 1];
          f[2 * m] = x0 * rc[t][m] - x1 * rs[t][m];
          f[2 * m + 1] = x0 * rs[t][m] + x1 * rc[t][m];
          const float c1 = rc[t][m] * dc[t][m] - rs[t][m] * dsn[t][m];
          rs[t][m] = rs[t][m] * dc[t][m] + rc[t][m] * dsn[t][m];
          rc[t][m] = c1;
        }
      }
    });
  };
  next_q();   // step 0 (its q rows landed with the prologue's loads)

  // ---- the two wave groups run half a step apart.  Each step of a group is a compute phase M (the window's scores,
  // softmax, PV: MFMA work and its dependent VALU) and an output phase V (half a ring tile, gate, output rows, and
  // the next step's q_hat: VALU work);
  // group 1 starts with an output phase of its own (the first ring half), so one group's M runs beside the other's V
  // on every SIMD (wave w and w + 4 share one), one work-group barrier between phases:
  //   interval 2c:     group 0: M(c)                         group 1: V(c-1), ring rows 0..15 of tile T(c)+1
  //   interval 2c + 1: group 0: V(c), ring rows 16..31 of T(c)+1   group 1: M(c)
  // M(c) reads tiles T(c)-4 .. T(c); tile T(c)+1 goes to the slot of T(c)-5, which no phase in flight reads (6 slots);
  // both halves of it are written before either group's M(c+1).
  // Per wave and step, the vector-memory operations in issue order: M: q rows of the next step (4 loads into LDS);
  // V: output rows (4 stores), gate rows of the next step (4 loads into LDS), the next ring half (2 loads), then the
  // wait for the q rows.  Rows and
  // tiles past a run's end use empty descriptors, so every step issues the same operations and the waits below are
  // fixed counts (the vm counter retires loads and stores in order).
  floatx4 acc_o[8];
  float l_run = 0.f;
  if (grp == 1) {
    if (n_steps > 1) store_kv(T0 + 1, hr, false);
    load_kv(T0 + 2, hr, n_steps > 2);
    lds_barrier();
  }
  for (int c = 0; c < n_steps; c++) {
    const int i0 = p_start + c * kStep;
    const int T = i0 / kTK;
    const int i = i0 + 16 * half + l16;           // this lane's query position
    const int qlo = i0 + 16 * half;               // the wave's positions qlo .. qlo+15
    const bool more = c + 1 < n_steps;
    // ================= M(c) =================
    // the compute phase is the critical one: on a SIMD this wave's instructions issue ahead of the other group's
    // output-phase wave while it is in M
    __builtin_amdgcn_s_setprio(1);
    // q_hat of this step is in qf (computed at the end of the previous output phase, or in the prologue); this
    // wave's q rows in LDS have been read, so the next step's go there
    load_rows(qb, QS, i0 + kStep, more);
    // ---- the whole window of the step: score blocks of 16 keys, block kb = 2j + kh covering keys
    // 32(T - 4 + j) + 16kh .. +15 (tiles before position 0 sit in zero-filled slots and are masked)
    int slot_k[kWinTiles], slot_v[kWinTiles];
#pragma unroll
    for (int j = 0; j < kWinTiles; j++) {
      const int sl = (T - (kWinTiles - 1) + j + kRing) % kRing;   // ring slot of tile T-4+j (T-4 >= -4)
      slot_k[j] = sl * kKTile;
      slot_v[j] = sl * kVTile;
    }
    floatx4 sacc[kBlocks];
#pragma unroll
    for (int kb = 0; kb < kBlocks; kb++) sacc[kb] = (floatx4){0.f, 0.f, 0.f, 0.f};
    // score MFMA f = kBlocks t + kb takes its K fragment from a window read 4 MFMAs ahead (the scheduling barriers
    // keep that order: left alone, the compiler reads each fragment right before its MFMA and waits for it there)
    constexpr int kWinS = 4;
    auto kfrag = [&](int f) {
      const int t = f / kBlocks, kb = f % kBlocks;
      return *reinterpret_cast<const half8*>(Ks + slot_k[kb >> 1] + k_off(0, 16 * (kb & 1) + l16, 4 * t + g));
    };
    half8 kwin[kWinS];
#pragma unroll
    for (int f = 0; f < kWinS; f++) kwin[f] = kfrag(f);
#pragma unroll
    for (int f = 0; f < 4 * kBlocks; f++) {
      const half8 kf = kwin[f % kWinS];
      if (f + kWinS < 4 * kBlocks) kwin[f % kWinS] = kfrag(f + kWinS);
      sacc[f % kBlocks] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[f / kBlocks], sacc[f % kBlocks], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // mask: key visible iff 0 <= i - key < min(W, pos0 + i + 1) (one unsigned compare; positions are chunk-local,
    // the bound keeps keys at absolute positions >= 0); blocks wholly inside every
    // window of the wave's 16 queries skip it.  C layout: lane (l16, g) holds keys 4g .. 4g+3 of the block.
    {
      const unsigned lim = CACHED ? (unsigned)min((int64_t)a.window, pos0 + i + 1) : (unsigned)min(a.window, i + 1);
#pragma unroll
      for (int kb = 0; kb < kBlocks; kb++) {
        const int kt = (T - (kWinTiles - 1)) * kTK + 16 * kb;
        if (!(kt >= (CACHED ? -(int)pos0 : 0) && kt + 15 <= qlo && kt >= qlo + 16 - a.window)) {
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
    const half2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int db = 0; db < 8; db++) acc_o[db] = (floatx4){0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
#pragma unroll
    for (int j = 0; j < kWinTiles; j++) {
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
    // training: the log-sum-exp of the query's scores (natural log; scores in log2 units are s log2(e))
    if (a.lse && g == 0 && i < p_end)
      a.lse[((int64_t)b * a.Hq + kvh * kGroup + head) * a.S + i] = (mx + __log2f(l_run)) * 0.6931471805599453f;
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();

    // ================= V(c) =================
    // this group's half of the next ring tile, from raw rows loaded in the previous V, and this wave's gate rows,
    // loaded before them (since then: 4 loads in M)
    ZG_WAIT_VM(4);
    if (c + 1 + grp < n_steps) store_kv(T + 1 + grp, hr, false);
    // ---- epilogue.  acc_o[db][e] is dim d = 16db + 4g + e of this lane's query row.
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
    // coalesced store of the wave's own 16 rows, 16 lanes per 256-byte row, through a descriptor over its valid
    // positions: rows past the run's end fall outside it and are dropped, so every step issues exactly 4 stores
    {
      const int nvalid = __builtin_amdgcn_readfirstlane(max(0, min(16, p_end - qlo)));
      const int prow = __builtin_amdgcn_readfirstlane(min(qlo, a.S - 1));
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(ob + (int64_t)prow * rowHq), (short)0, (int)(nvalid * rowHq * 2), 0x00020000);
      uint4 orow[4];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int r = 4 * k + (lane >> 4), ch = lane & 15;
        orow[k] = *reinterpret_cast<const uint4*>(GO + go_off(16 * wave + r, ch));
      }
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int r = 4 * k + (lane >> 4), ch = lane & 15;
        const int off = (int)((r * rowHq + head * kHeadDim + 8 * ch) * 2);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((__vector_size__(4 * sizeof(int)))) int, orow[k]),
                                               ro, off, 0, 0);
      }
    }
    // the next step's gate rows into the same LDS rows, once this wave's reads of them are done, and the raw rows
    // of this group's next ring half
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the LDS reads are complete (vmcnt 63, expcnt 7: not waited)
    load_rows(gb, GO, i0 + kStep, more);
    load_kv(T + 2 + grp, hr, c + 2 + grp < n_steps);   // stored in the next V if a step still needs it
    // ---- the next step's q_hat: its q rows were loaded at the start of M (since then: 4 stores, 4 + 2 loads)
    if (more) {
      ZG_WAIT_VM(10);
      next_q();
    }
    lds_barrier();
  }
  if (grp == 0) lds_barrier();
}

}  // namespace

int swa_stream_run_length(int S, int n_units) {
  // about one work-group per CU (256 CUs; the LDS ring, gate and q tiles of 8 waves take one CU each), at most
  // kMaxRunSteps steps each
  const int64_t per = ((int64_t)S * n_units + 255) / 256;
  int64_t run = (per + kStep - 1) / kStep * kStep;
  run = run < kStep ? kStep : run;
  return (int)(run > (int64_t)kStep * kMaxRunSteps ? (int64_t)kStep * kMaxRunSteps : run);
}

hipError_t launch_swa_stream(const SwaStreamArgs& a, hipStream_t st) {
  if (a.G != kGroup || a.window < 1 || a.window > kTK * (kWinTiles - 1) || a.rot_pairs > 32 || a.run % kStep ||
      a.run > kStep * kMaxRunSteps)
    return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.n_units * ((a.S + a.run - 1) / a.run);
  if (a.ck) hipLaunchKernelGGL(attn_swa_stream_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(attn_swa_stream_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace zg
