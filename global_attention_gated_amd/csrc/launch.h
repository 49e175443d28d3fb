// Internal launch interface between the C-ABI host code (zgattn_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zg {

constexpr int kMaxLayers = 64;
constexpr int kMaxDecodeBatch = 128;
constexpr int kDecodeChunk = 8192;   // keys per split-K work-group of a global decode layer

// After a gated chunk with a cache: k_hat (recomputed from k, bit-identical to the staging's) and raw v of the
// chunk's last n rows go to ring slot (position mod W).
struct RingWriteArgs {
  const uint16_t* k;         // input k [B][S][Hkv][D]
  const uint16_t* v;         // input v [B][S][Hkv][D]
  const uint16_t* kw;        // [D]
  uint16_t* kring;           // [B][Hkv][W][D]
  uint16_t* vring;
  int32_t B, S, Hkv, W, n;   // rows S-n .. S-1 of the chunk
  int64_t pos0;
  int32_t rot_pairs;
  float eps;
  double inv_freq_rev[64];
};

// Staging of the keys and values a tile-path call attends to, positions kbase .. pos0+S-1 (kbase <= pos0), in the
// layout the attention kernel copies into LDS with direct (buffer-to-LDS) loads:
//   kt: k_hat fp16 [B][Hkv][S_kpad][D]
//   vt: v^T fp16 [B][Hkv][D][S_kpad], inside each group of 16 keys the quads of 4 keys in the order 0, 2, 1, 3
// Staged row r is position kbase + r; S_kpad = the staged count rounded up to a whole 64-key tile, the padding
// rows zero.  Positions >= pos0 come from the chunk's k (k_hat computed here) and v; earlier ones from the cache
// (ck/cv, bf16 [B][Hkv][slots][D]: row p of a global layer, or ring slot p mod slots).  With dk/dv set, the chunk's
// k_hat and v are also stored in those cache rows (a global layer with a cache).
struct StageArgs {
  const uint16_t* k;     // [B][S][Hkv][D] bf16, the chunk
  const uint16_t* v;
  const uint16_t* kw;    // [D]
  const uint16_t* ck;    // cache K / V of the layer, or null when kbase == pos0
  const uint16_t* cv;
  uint16_t* dk;          // cache K / V rows for the chunk's positions, or null
  uint16_t* dv;
  int64_t slots;         // rows per (b, head) of the cache arrays
  int32_t ring;          // 1: slot = position mod slots
  uint16_t* kt;
  uint16_t* vt;
  int32_t pos0, kbase;
  int32_t B, S, S_kpad, Hkv;
  int32_t rot_pairs;
  float eps;
  double inv_freq_rev[64];
};

// Tile-path attention over the staged keys (see StageArgs): queries at pos0 .. pos0+S-1; causal when gate is null
// (global layer), else within the window and multiplied by sigmoid(gate).
struct TileAttnArgs {
  const uint16_t* q;    // [B][S][Hq][D]
  const uint16_t* gate; // [B][S][Hq][D], null for a global layer
  const uint16_t* qw;   // [D]
  uint16_t* out;        // [B][S][Hq][D]
  float* lse;           // [B][Hq][S] or null
  const uint16_t* kt;   // staged tiles
  const uint16_t* vt;
  int32_t pos0, kbase;
  int32_t B, S, S_kpad, Hq, Hkv, G, P;  // P = 128 / G: query positions per wave group (a work-group has two)
  int32_t window;       // gated layers
  int32_t rot_pairs;
  float eps;
  float q_scale;        // log2(e) / sqrt(D)
  int32_t n_units;      // B * Hkv
  int32_t n_qtiles;     // ceil(S / 2P): work-groups per (sequence, KV head)
  double inv_freq_rev[64];
};

// Streaming gated-SWA prefill without a cache (GQA group 4, window <= 128): one work-group per run of
// `run` consecutive positions (a multiple of 32) of one (b, kv head); k_hat is computed in the kernel.
struct SwaStreamArgs {
  const uint16_t* q;     // [B][S][Hq][D]
  const uint16_t* k;     // [B][S][Hkv][D] (raw k)
  const uint16_t* v;     // [B][S][Hkv][D]
  const uint16_t* gate;  // [B][S][Hq][D]
  const uint16_t* qw;    // [D]
  const uint16_t* kw;    // [D]
  uint16_t* out;         // [B][S][Hq][D]
  int32_t B, S, Hq, Hkv, G;
  int32_t window;
  int32_t rot_pairs;
  float eps;
  float q_scale;         // log2(e) / sqrt(D)
  int32_t n_units;       // B * Hkv
  int32_t run;           // positions per work-group
  float* lse;            // [B][Hq][S] natural log of each softmax denominator (training), or null
  double inv_freq_rev[64];
  // a chunk that continues a cached sequence: its positions are pos0 .. pos0+S-1, and the window's earlier keys come
  // from the layer's ring (k_hat and v, bf16, [B][Hkv][window][D], position p in slot p mod window); ck = null: none
  const uint16_t* ck;
  const uint16_t* cv;
  int32_t pos0;
};

// Device state of FP8 operands under delayed scaling: n tensors (a projection: 0 = the input x, 1 = the weight
// W), each with an amax history of H floats, the per-work-group maxima of the current call's quantisation,
// the scale in use and its inverse.
constexpr int32_t kFp8MaxBlocks = 2048;   // work-groups of one quantisation launch (8 per CU)
constexpr int32_t kFp8MaxTensors = 8;
struct Fp8State {
  float* hist;        // [n][H]
  float* partial;     // [n][kFp8MaxBlocks]
  float* scale;       // [n]
  float* scale_inv;   // [n]
  int32_t H;
  int32_t n;
};
// Work-groups of each tensor's quantisation in the current call (0 = not quantised: state left unchanged).
struct Fp8Blocks {
  int32_t n[kFp8MaxTensors];
};

// Backward of an attention layer (training), no cache, positions 0..S-1.  Sp = S rounded up to 128; the
// workspace arrays are zero past S (and nlse2 -inf), so tiles may run over the end.
struct BwdArgs {
  const uint16_t* q;      // [B][S][Hq][D] bf16
  const uint16_t* k;      // [B][S][Hkv][D]
  const uint16_t* v;      // [B][S][Hkv][D]
  const uint16_t* gate;   // [B][S][Hq][D], null for a global layer
  const uint16_t* qw;     // [D]
  const uint16_t* kw;     // [D]
  const uint16_t* out;    // [B][S][Hq][D] the forward's output
  const uint16_t* dout;   // [B][S][Hq][D]
  const float* lse;       // [B][Hq][S] natural log of the softmax denominators
  uint16_t* dq;           // [B][S][Hq][D] bf16
  uint16_t* dk;           // [B][S][Hkv][D]
  uint16_t* dv;           // [B][S][Hkv][D]
  uint16_t* dgate;        // [B][S][Hq][D], null for a global layer
  float* dqw;             // [D]
  float* dkw;             // [D]
  // workspace
  uint16_t* qh16;         // [B][Hq][Sp][D] fp16 q_hat * log2(e)/sqrt(D)
  uint16_t* qt;           // [B][Hq][D][Sp] bf16 q_hat transposed
  uint16_t* da;           // [B][Hq][Sp][D] bf16 dA
  uint16_t* dat;          // [B][Hq][D][Sp] bf16 dA transposed
  float* nlse2;           // [B][Hq][Sp] -lse * log2(e) (negated: the score accumulators start from it)
  float* ndelta;          // [B][Hq][Sp] -(dout . out) (negated: the dP accumulators start from it)
  uint16_t* kh16;         // [B][Hkv][Sp][D] fp16 k_hat (bf16 values)
  uint16_t* kt;           // [B][Hkv][D][Sp] bf16 k_hat transposed
  float* dw_part;         // [n_qblk + n_kblk][D]: per-work-group partials of dw_q (dQ kernel), then of dw_k (dK)
  int32_t n_qblk;         // work-groups of the dQ kernel: B * Hkv * ceil(S / 32)
  int32_t n_kblk;         // key blocks of the dK kernels: B * Hkv * bwd_k_blocks(S, window)
  int32_t B, S, Sp, Hq, Hkv, G;
  int32_t window;         // 0 for a global layer
  int32_t rot_pairs;
  float eps;
  float q_scale;          // log2(e) / sqrt(D)
  double inv_freq_rev[64];
};

// One entry per layer of a KV cache, in device memory.
struct LayerDesc {
  uint16_t* k;
  uint16_t* v;
  int64_t slots;     // rows per (b, h): max_tokens (global) or W (SWA)
  int32_t is_global;
  int32_t index;     // global: index among global layers (for the partials); SWA: index among SWA layers
};

struct DecodeArgs {
  const uint16_t* q;       // [L][B][Hq][D]
  const uint16_t* k;       // [L][B][Hkv][D]
  const uint16_t* v;
  const uint16_t* gate;    // [L][B][Hq][D]
  const uint16_t* qw;      // [L][D]
  const uint16_t* kw;
  uint16_t* out;           // [L][B][Hq][D]
  const LayerDesc* layers; // device [L]
  const int32_t* glob_ids; // device [n_global]: 0-based layer numbers of the global layers
  const int32_t* swa_ids;  // device [n_swa]
  float* part_m;           // [n_global][B][Hkv][max_chunks][G]
  float* part_l;
  float* part_acc;         // [n_global][B][Hkv][max_chunks][G][D]
  int32_t L, B, Hq, Hkv, G, W;
  int32_t n_global, n_swa, max_chunks;
  int32_t rot_pairs;
  float eps;
  float q_scale;
  double inv_freq_rev[64];
  int64_t pos[kMaxDecodeBatch];
};

hipError_t launch_ring_write(const RingWriteArgs& a, hipStream_t st);
hipError_t launch_kv_stage(const StageArgs& a, hipStream_t st);
hipError_t launch_attn_pp(const TileAttnArgs& a, bool gated, hipStream_t st);
hipError_t launch_swa_stream(const SwaStreamArgs& a, hipStream_t st);
int32_t fp8_quantize_blocks(int64_t n);   // work-groups launch_fp8_quantize uses for n values
hipError_t launch_fp8_quantize(const uint16_t* x, uint8_t* q, int64_t n, const float* scale, float* partial,
                               hipStream_t st);
hipError_t launch_bwd_dw_zero(float* dqw, float* dkw, hipStream_t st);   // D = 128 floats each
hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_kv(const BwdArgs& a, hipStream_t st);
// key blocks (dw_k partials per (sequence, KV head)) of the key-centric backward: 256 keys (causal) or 128 (window)
int bwd_k_blocks(int32_t S, int32_t window);
hipError_t launch_bwd_q(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dw_reduce(const BwdArgs& a, hipStream_t st);
hipError_t launch_fp8_finalize(const Fp8State& s, int32_t idx, const Fp8Blocks& nb, hipStream_t st);
int swa_stream_run_length(int S, int n_units);
hipError_t launch_decode_append(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_swa(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_global(const DecodeArgs& a, int32_t chunks_needed, hipStream_t st);
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t st);

}  // namespace zg
