/*
 * zgattn.h -- C ABI of the MI355X (gfx950) attention core of the ZGCM-1 hybrid backbone:
 * gated sliding-window attention (SWA) layers interleaved 5:1 with ungated global causal layers,
 * GQA heads, QK-RMSNorm and partial RoPE, prefill and single-token decode against a KV cache.
 *
 * The operation (ZGCM-1 paper summaries: onedev.kr "How it works"; jaehun.me "New Approach" and
 * "How Gated SWA Behaves"):
 *   q_hat = RoPE_R(RMSNorm(q) * w_q),  k_hat = RoPE_R(RMSNorm(k) * w_k)     per (token, head), over D
 *   gated SWA layer:  out = softmax_{j in (i-W, i]}(q_hat . k_hat_j / sqrt(D)) v_j  (.)  sigmoid(gate)
 *   global layer:     out = softmax_{j <= i}(q_hat . k_hat_j / sqrt(D)) v_j           (no gate)
 *   query head h reads KV head h / (Hq / Hkv).  RMSNorm: x * w / sqrt(mean(x^2) + eps).
 *   RoPE_R rotates pairs (2i, 2i+1), 2i+1 < R, of a row at absolute position p by p * base^(-2i/R);
 *   dims >= R are unchanged.  The window W counts the query itself.
 * The projections around this core (q/k/v/g_proj before, o_proj after) are not part of this library:
 * the gate argument is the precomputed g_proj(h) logits.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as pointers to 16-bit bf16 bit patterns in DEVICE memory, contiguous,
 *     16-byte aligned, in the stated layout (row-major, last index fastest).  Host pointers are marked.
 *   - Only D == 128 is implemented (ZG_EUNSUPPORTED otherwise); Hq must be a multiple of Hkv and
 *     128 must be a multiple of Hq / Hkv; rotary_dims must be even and <= D.
 *   - Every call validates its arguments on the host first; on a non-zero status nothing has been
 *     enqueued and zg_last_error() (thread-local) describes the failure.  On ZG_OK the work is only
 *     enqueued on `stream` (a hipStream_t passed as void*; NULL = the default stream): outputs are
 *     ready after the stream reaches that point, and kernel faults surface at the caller's next
 *     synchronisation.  No C++ exception crosses this ABI.
 *   - The caller owns every q/k/v/gate/weight/out/workspace buffer; the library never frees them and
 *     keeps no reference to them after the enqueued work completes.  The KV cache is library-owned.
 *   - Calls that share a KV cache or a workspace must be ordered on one stream (or synchronised by
 *     the caller); the library does not lock.
 *   - Value range.  Inside the prefill MFMAs, k_hat and v are held in fp16 (exact for bf16 values of magnitude
 *     2^-14 .. 65504): a value beyond +-65504 is clamped to +-65504 (never infinite), so results are exact for
 *     |v| <= 65504 and a larger value only changes the outputs of the queries that attend to it (as if it were
 *     +-65504), never those of other queries.  |k_hat_d| <= sqrt(D) |w_k,d| by the RMSNorm, so keys stay in range
 *     for |w_k| <= 5790; q_hat * log2(e)/sqrt(D) for |w_q| <= 45000.  Decode and the backward read v in bf16 and
 *     are exact over bf16's whole range.  NaN inputs are outside the contract.
 */
#ifndef ZGATTN_H
#define ZGATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum zg_status {
  ZG_OK = 0,
  ZG_EINVAL = 1,       /* malformed argument: null pointer, bad size, misalignment, inconsistent shape */
  ZG_EUNSUPPORTED = 2, /* well-formed but not implemented (D != 128, GQA group not dividing 128, ...) */
  ZG_ERANGE = 3,       /* position / capacity / workspace size out of range */
  ZG_ENOMEM = 4,       /* device allocation failed */
  ZG_EHIP = 5          /* a HIP runtime call failed (launch error, ...) */
};

/* Opaque, library-owned KV cache. */
typedef struct zg_kv_cache zg_kv_cache;

/* Shape of a KV cache.  Layers are numbered 1..n_layers; the global ones are listed in global_layers
 * (HOST array of n_global distinct 1-based layer numbers, e.g. {6,12,18,24,30} for the 32-layer 5:1
 * schedule of the pages).  Every other layer is a gated-SWA layer that keeps a `window`-slot ring. */
typedef struct {
  int32_t n_layers;
  const int32_t* global_layers; /* HOST, may be NULL when n_global == 0 */
  int32_t n_global;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;  /* must be 128 */
  int32_t window;    /* SWA window W (the pages: 128) */
  int64_t max_tokens; /* capacity of each global layer: positions 0 .. max_tokens-1 */
} zg_cache_desc;

/* Device layout of the cache (all bf16, K and V in separate arrays per layer):
 *   global layer: K[b][kv_head][max_tokens][D], V the same; row p holds position p.
 *   SWA layer:    K[b][kv_head][window][D],     V the same; slot p mod W holds position p
 *                 (the last W positions; slots whose position would be negative are unused).
 * K rows hold k_hat (after RMSNorm and RoPE, rounded to nearest-even bf16); V rows hold v unchanged.
 * The cache also keeps, on the host, the current length (next position) of every (layer, sequence).
 *
 * KV-cache footprint as the pages count it (onedev.kr "How it works"; jaehun.me "Why the KV Cache
 * Shrinks by 6.4x"): 2 (K,V) x Hkv x D x 2 bytes per position per layer, every position in a global
 * layer and at most W positions in an SWA layer. */

/* Allocate and zero a cache (one device allocation, on the current HIP device; all lengths 0).
 * *out receives the handle; *bytes_out (nullable) the device bytes allocated.
 * Errors: EINVAL (bad descriptor), EUNSUPPORTED (head_dim != 128), ENOMEM. */
int kv_cache_alloc(const zg_cache_desc* desc, zg_kv_cache** out, uint64_t* bytes_out);

/* Release a cache (synchronises the device first).  NULL is accepted. */
int kv_cache_free(zg_kv_cache* cache);

/* Host-only closed form: cache bytes for `tokens` positions of every sequence in desc->batch,
 * sum over layers of 2*Hkv*D*2*batch*(global ? tokens : min(tokens, window)).  0 on a bad descriptor. */
uint64_t kv_cache_footprint_bytes(const zg_cache_desc* desc, int64_t tokens);

/* Device pointers to layer `layer`'s K and V arrays (layout above) and their slot count per (b, head)
 * (max_tokens or window).  For filling a cache with precomputed contents, and for tests. */
int kv_cache_layer_view(const zg_kv_cache* cache, int32_t layer, void** k, void** v, int64_t* slots);

/* Current length (number of positions written) of sequence b in layer `layer`. */
int kv_cache_length(const zg_kv_cache* cache, int32_t layer, int32_t b, int64_t* len);

/* Set that length (after filling the arrays through kv_cache_layer_view).  ERANGE if len < 0 or,
 * for a global layer, len > max_tokens. */
int kv_cache_set_length(zg_kv_cache* cache, int32_t layer, int32_t b, int64_t len);

/* Device workspace bytes that swa_prefill / global_prefill need for a chunk of S tokens at absolute positions
 * pos0 .. pos0+S-1 (pos0 > 0 only with a cache).  The call stages the keys its queries see, positions kbase ..
 * pos0+S-1 (kbase = 0 for a global layer, max(0, pos0 - window + 1) for a gated one: window 0 means global), as
 * fp16 k_hat and transposed v in whole 64-key tiles: 2 * B*Hkv*K_pad*D 16-bit elements, K_pad = pos0+S-kbase
 * rounded up to a multiple of 64.  0 when S == 0 or an argument is negative. */
uint64_t prefill_workspace_bytes_at(int32_t B, int32_t S, int32_t Hkv, int32_t D, int64_t pos0, int32_t window);
/* The same for a call without a cache (pos0 = 0): prefill_workspace_bytes_at(B, S, Hkv, D, 0, 0). */
uint64_t prefill_workspace_bytes(int32_t B, int32_t S, int32_t Hkv, int32_t D);

/* Gated sliding-window attention layer, prefill of S new tokens per sequence at absolute positions
 * pos0 .. pos0+S-1 (onedev.kr "How it works": GatedSWA(h) = o_proj(A_SWA(q,k,v) (.) sigmoid(g_proj(h))),
 * 128-token window; jaehun.me "How Gated SWA Behaves").
 *   q, gate, out: [B][S][Hq][D]; k, v: [B][S][Hkv][D]; q_norm_w, k_norm_w: [D]   (device bf16)
 *   window: W >= 1; rotary_dims: R; rope_base: RoPE base; eps: RMSNorm epsilon.
 *   cache (nullable): with a cache, keys at positions pos0-W+1 .. pos0-1 are read from layer `layer`'s
 *     ring, whose length must equal pos0, and the chunk's last min(S, W) positions are written into
 *     the ring (length becomes pos0+S).  Without a cache pos0 must be 0.
 *   workspace: device buffer of at least prefill_workspace_bytes_at(B, S, Hkv, D, pos0 (0 without a cache), window)
 *     bytes, 16-byte aligned (the streaming kernel of the common case, GQA group 4, W <= 128 and rotary_dims <= 64,
 *     with or without a cache, does not touch it).
 * S == 0 or B == 0 is a no-op.  Errors: EINVAL, EUNSUPPORTED, ERANGE, EHIP. */
int swa_prefill(const void* q, const void* k, const void* v, const void* gate, const void* q_norm_w,
                const void* k_norm_w, void* out, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                int32_t window, int32_t rotary_dims, double rope_base, float eps, int64_t pos0,
                zg_kv_cache* cache, int32_t layer, void* workspace, uint64_t workspace_bytes, void* stream);

/* Ungated global causal attention layer, prefill (onedev.kr "How it works": the global layers see the
 * whole context without the gate).  Arguments as swa_prefill without gate and window.
 *   cache (nullable): with a cache, layer `layer` must be a global layer of the cache whose length
 *     equals pos0 (positions 0..pos0-1 are read from it: chunked prefill), pos0+S <= max_tokens, and the
 *     chunk's k_hat and v are written at rows pos0 .. pos0+S-1.  Without a cache pos0 must be 0.
 *   workspace: at least prefill_workspace_bytes_at(B, S, Hkv, D, pos0 (0 without a cache), 0) bytes: with a cache
 *     every earlier position is staged, so the workspace grows with the context (1 GiB at 262,144 positions for
 *     B = 1, Hkv = 8). */
int global_prefill(const void* q, const void* k, const void* v, const void* q_norm_w, const void* k_norm_w,
                   void* out, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t rotary_dims,
                   double rope_base, float eps, int64_t pos0, zg_kv_cache* cache, int32_t layer,
                   void* workspace, uint64_t workspace_bytes, void* stream);

/* One decode step of every layer of the cache (onedev.kr "How it works": the 5:1 hybrid of gated-SWA and global
 * layers; jaehun.me "Why the KV Cache Shrinks by 6.4x": an SWA layer keeps only the last W keys, a global layer
 * every key, so decoding reads a W-slot ring per SWA layer and the whole cache per global layer).
 * Each sequence b adds one token at absolute position
 * positions[b] (HOST array [B]; must equal the cache length of every layer for that sequence).
 *   q, gate, out: [L][B][Hq][D]; k, v: [L][B][Hkv][D]; q_norm_w, k_norm_w: [L][D]   (device bf16)
 *   with L = the cache's n_layers, B = its batch.  gate rows of global layers are ignored.
 * Per layer the new k_hat and v are appended first (SWA: ring slot p mod W; global: row p), then the
 * token attends over the cache (itself included): SWA layers over positions p-W+1..p with the gate,
 * global layers over 0..p without it.  The layers' inputs are all given, so the layers are computed
 * concurrently.  Every length advances by one.  Errors: EINVAL, EUNSUPPORTED, ERANGE (a position that
 * differs from the cache length or reaches max_tokens), EHIP. */
int hybrid_decode_step(const void* q, const void* k, const void* v, const void* gate, const void* q_norm_w,
                       const void* k_norm_w, void* out, const int64_t* positions, int32_t Hq,
                       int32_t rotary_dims, double rope_base, float eps, zg_kv_cache* cache, void* stream);

/* ---- For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): global_prefill without a workspace argument.  The keys are staged in a scratch array that the library
 * holds on each GPU it runs on (global_prefill_noalloc_max_bytes() = 64 MiB per GPU, until the process ends; enough
 * for 8 KV heads x 16,384 positions); the call allocates nothing.  A call whose staging needs more
 * (prefill_workspace_bytes_at(B, S, Hkv, D, pos0, 0) above the maximum) returns ERANGE.  Every call on one GPU
 * shares that GPU's array, so calls that overlap on one GPU (different streams, or other threads) race: order them
 * on one stream.  Arguments and other errors as global_prefill. */
uint64_t global_prefill_noalloc_max_bytes(void);
int global_prefill_noalloc(const void* q, const void* k, const void* v, const void* q_norm_w, const void* k_norm_w,
                           void* out, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t rotary_dims,
                           double rope_base, float eps, int64_t pos0, zg_kv_cache* cache, int32_t layer, void* stream);

/* ---- Training: forward with log-sum-exp, and the backward of an attention layer (no cache, positions 0..S-1).
 * The forward is swa_prefill / global_prefill that also writes, per (sequence, query head, position), the natural
 * log of its softmax denominator: lse_i = log sum_j exp(s_ij), s_ij = q_hat_i . k_hat_j / sqrt(D) over the visible
 * keys.  lse [B][Hq][S] device fp32.  Other arguments and errors as swa_prefill (workspace of
 * prefill_workspace_bytes). */
int swa_prefill_train(const void* q, const void* k, const void* v, const void* gate, const void* q_norm_w,
                      const void* k_norm_w, void* out, float* lse, int32_t B, int32_t S, int32_t Hq, int32_t Hkv,
                      int32_t D, int32_t window, int32_t rotary_dims, double rope_base, float eps, void* workspace,
                      uint64_t workspace_bytes, void* stream);
int global_prefill_train(const void* q, const void* k, const void* v, const void* q_norm_w, const void* k_norm_w,
                         void* out, float* lse, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t rotary_dims, double rope_base, float eps, void* workspace, uint64_t workspace_bytes,
                         void* stream);

/* Workspace bytes of the backward: staged q_hat (fp16 and transposed bf16), dA = dout (.) sigmoid(g) (bf16, also
 * transposed), per-row Delta = dout . out and lse, k_hat (fp16 and transposed bf16), with S rounded up to 128, and
 * the per-work-group partial sums of the norm-weight gradients. */
uint64_t backward_workspace_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D);

/* Gradients of a gated-SWA layer's output (onedev.kr "How it works": A_SWA(q,k,v) (.) sigmoid(g), with the
 * QK-RMSNorm and partial RoPE of jaehun.me "How Gated SWA Behaves") with respect to its inputs, given dout = dL/dout.
 *   inputs as swa_prefill_train, plus out [B][S][Hq][D] and lse [B][Hq][S] from it, and dout [B][S][Hq][D];
 *   outputs dq [B][S][Hq][D], dk, dv [B][S][Hkv][D], dgate [B][S][Hq][D] (device bf16, written) and
 *   dq_norm_w, dk_norm_w [D] (device fp32, written: sums over every token and head).
 * Chain rule: dA = dout (.) sigmoid(g); dgate = dout (.) out (.) (1 - sigmoid(g)); Delta_i = dout_i . out_i;
 * ds_ij = p_ij (dA_i . v_j - Delta_i); dq_hat = ds k_hat / sqrt(D); dk_hat = ds^T q_hat / sqrt(D) and
 * dv = p^T dA summed over the query heads of a KV head; then through RoPE and RMSNorm.  The bf16 rounding of
 * k_hat passes its gradient through unchanged.  Score products in fp16 (as the forward), gradient products in
 * bf16, fp32 accumulation.  D = 128 and GQA group 4 only.
 * Errors: EINVAL, EUNSUPPORTED, ERANGE (workspace, size), EHIP. */
int swa_prefill_backward(const void* q, const void* k, const void* v, const void* gate, const void* q_norm_w,
                         const void* k_norm_w, const void* out, const float* lse, const void* dout, void* dq, void* dk,
                         void* dv, void* dgate, float* dq_norm_w, float* dk_norm_w, int32_t B, int32_t S, int32_t Hq,
                         int32_t Hkv, int32_t D, int32_t window, int32_t rotary_dims, double rope_base, float eps,
                         void* workspace, uint64_t workspace_bytes, void* stream);
/* The global layer's backward: as swa_prefill_backward without the gate (dA = dout) and the window. */
int global_prefill_backward(const void* q, const void* k, const void* v, const void* q_norm_w, const void* k_norm_w,
                            const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            float* dq_norm_w, float* dk_norm_w, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                            int32_t rotary_dims, double rope_base, float eps, void* workspace, uint64_t workspace_bytes,
                            void* stream);

/* ---- Projections around the core (onedev.kr "How it works": GatedSWA(h) = o_proj(A_SWA(q,k,v) (.)
 * sigmoid(g_proj(h))), with q/k/v/g projections of the hidden state h).  Plain GEMMs on hipBLASLt. */

/* y = x . W^T, a linear layer's forward: x [T][K], W [N][K] (out_features x in_features), y [T][N], device
 * bf16, fp32 accumulation, result rounded to bf16.  The library keeps one hipBLASLt handle, a 64 MiB
 * workspace and a cached plan per (T, K, N) per device, created on first use.  T == 0 is a no-op.
 * Errors: EINVAL (shape, null, alignment), EHIP (hipBLASLt failure, message names the status). */
int linear_bf16(const void* x, const void* w, void* y, int64_t T, int32_t K, int32_t N, void* stream);

/* ---- FP8 projections with delayed scaling (onedev.kr "What differs": FP8 matmuls, E4M3 in the forward pass,
 * delayed scaling over a 1,024-step amax history).  E4M3 is the OCP format: largest finite value 448,
 * 3 mantissa bits, subnormals down to 2^-9.  A state keeps, for the input x and the weight W, an amax
 * history of `history` calls and the scale in use, s = 448 / max(history) (1 while the history is zero).
 * Each call quantises x and W with the current scales (code = E4M3(v * s), nearest-even, saturating at +-448),
 * runs the GEMM on the codes with fp32 accumulation and multiplies by 1/(s_x s_w), then records this call's
 * max |x| and max |W| in the histories and derives the next scales: the scales lag the data by one call. */
typedef struct zg_fp8_linear zg_fp8_linear;

/* Allocate a state for y[T][N] = x[T][K] . W[N][K]^T on the current device: histories zero, scales 1.
 * K must be a multiple of 8.  Errors: EINVAL, EUNSUPPORTED, ENOMEM, EHIP. */
int fp8_linear_alloc(int32_t K, int32_t N, int32_t history, zg_fp8_linear** out);
/* Release a state (synchronises the device first).  NULL is accepted. */
int fp8_linear_free(zg_fp8_linear* state);
/* The scales the next call will use, {s_x, s_w} (HOST float[2]); synchronises the device. */
int fp8_linear_scales(const zg_fp8_linear* state, float* scales_out);
/* Workspace bytes of linear_fp8_delayed: the E4M3 codes of x (T*K bytes), then those of W (N*K bytes), each
 * starting on a 256-byte boundary.  After a call the workspace holds both code arrays. */
uint64_t fp8_linear_workspace_bytes(int64_t T, int32_t K, int32_t N);
/* One FP8 projection: x [T][K], W [N][K], y [T][N] device bf16; state as allocated for (K, N).  Calls that
 * share a state must be ordered on one stream.  T == 0 is a no-op (the state does not advance).
 * Errors: EINVAL (shape or device mismatch, null, alignment), ERANGE (workspace), EHIP. */
int linear_fp8_delayed(const void* x, const void* w, void* y, int64_t T, int32_t K, int32_t N, zg_fp8_linear* state,
                       void* workspace, uint64_t workspace_bytes, void* stream);

/* Workspace bytes for gated_swa_layer / global_layer on B x S tokens without a cache: the bf16 activations q, g, o
 * [T][Hq*D] and k, v [T][Hkv*D] (T = B*S), 256-byte aligned, followed by the attention's workspace, which takes the
 * rest of the buffer: prefill_workspace_bytes(B, S, Hkv, D) here; with a cache at pos0 > 0, pass
 * layer_workspace_bytes - prefill_workspace_bytes(B, S, Hkv, D) + prefill_workspace_bytes_at(B, S, Hkv, D, pos0,
 * window) bytes (window 0 for a global layer). */
uint64_t layer_workspace_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D);

/* A gated-SWA attention layer from the hidden state: q = h W_q^T, k = h W_k^T, v = h W_v^T, g = h W_g^T, then
 * swa_prefill (QK-RMSNorm, partial RoPE, windowed attention, sigmoid(g) gate), then y = o W_o^T.
 *   h [B][S][d_model]; W_q, W_g [Hq*D][d_model]; W_k, W_v [Hkv*D][d_model]; W_o [d_model][Hq*D];
 *   q_norm_w, k_norm_w [D]; y [B][S][d_model]   (device bf16).  The head layout of q/k/v/g/o is that of
 *   swa_prefill ([token][head][D]).  Other arguments as swa_prefill; workspace of layer_workspace_bytes.
 * Every argument (the attention's included) is validated before anything is enqueued.
 * Errors: as linear_bf16 and swa_prefill. */
int gated_swa_layer(const void* h, const void* w_q, const void* w_k, const void* w_v, const void* w_g, const void* w_o,
                    const void* q_norm_w, const void* k_norm_w, void* y, int32_t B, int32_t S, int32_t d_model,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t window, int32_t rotary_dims, double rope_base, float eps,
                    int64_t pos0, zg_kv_cache* cache, int32_t layer, void* workspace, uint64_t workspace_bytes,
                    void* stream);

/* The global layer: as gated_swa_layer without the gate projection and the window (global_prefill). */
int global_layer(const void* h, const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                 const void* q_norm_w, const void* k_norm_w, void* y, int32_t B, int32_t S, int32_t d_model, int32_t Hq,
                 int32_t Hkv, int32_t D, int32_t rotary_dims, double rope_base, float eps, int64_t pos0,
                 zg_kv_cache* cache, int32_t layer, void* workspace, uint64_t workspace_bytes, void* stream);

/* ---- Whole layers with FP8 projections (onedev.kr "What differs": the matmuls run in FP8, E4M3 forward, delayed
 * scaling over a 1,024-step amax history).  A layer state holds seven delayed-scaling tensors, each with its own
 * history and scale as in zg_fp8_linear: 0 = h, 1 = W_q, 2 = W_k, 3 = W_v, 4 = W_g (unused by a global layer),
 * 5 = the attention output o, 6 = W_o.  Per call h is quantised once and feeds the four input projections, o once
 * for o_proj; every GEMM multiplies by the inverse scales of its two operands; after the call each quantised
 * tensor's max |v| enters its history and its next scale is derived (the scales lag the data by one call). */
typedef struct zg_fp8_layer zg_fp8_layer;

/* Allocate a layer state on the current device (histories zero, scales 1).  d_model and Hq*D must be multiples
 * of 8.  Errors: EINVAL, EUNSUPPORTED, ENOMEM, EHIP. */
int fp8_layer_alloc(int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D, int32_t history, zg_fp8_layer** out);
/* Release a layer state (synchronises the device first).  NULL is accepted. */
int fp8_layer_free(zg_fp8_layer* state);
/* The seven scales the next call will use (HOST float[7], tensor order above); synchronises the device. */
int fp8_layer_scales(const zg_fp8_layer* state, float* scales_out);
/* Workspace bytes of the FP8 layers without a cache: the activations of layer_workspace_bytes, then the E4M3 codes of
 * h [T][d_model], o [T][Hq*D], W_q, W_k, W_v, W_g and W_o, each starting on a 256-byte boundary, then the attention's
 * workspace, the rest of the buffer (with a cache, sized as for gated_swa_layer / global_layer). */
uint64_t fp8_layer_workspace_bytes(int32_t B, int32_t S, int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D);
/* gated_swa_layer / global_layer with every projection on E4M3 operands under the layer state `fp8` (shapes must
 * match the state's).  Calls that share a state must be ordered on one stream.  B*S == 0 is a no-op (the state
 * does not advance).  Errors: as gated_swa_layer / global_layer, and EINVAL for a null or mismatched state. */
int gated_swa_layer_fp8(const void* h, const void* w_q, const void* w_k, const void* w_v, const void* w_g,
                        const void* w_o, const void* q_norm_w, const void* k_norm_w, void* y, int32_t B, int32_t S,
                        int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D, int32_t window, int32_t rotary_dims,
                        double rope_base, float eps, int64_t pos0, zg_kv_cache* cache, int32_t layer,
                        zg_fp8_layer* fp8, void* workspace, uint64_t workspace_bytes, void* stream);
int global_layer_fp8(const void* h, const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                     const void* q_norm_w, const void* k_norm_w, void* y, int32_t B, int32_t S, int32_t d_model,
                     int32_t Hq, int32_t Hkv, int32_t D, int32_t rotary_dims, double rope_base, float eps, int64_t pos0,
                     zg_kv_cache* cache, int32_t layer, zg_fp8_layer* fp8, void* workspace, uint64_t workspace_bytes,
                     void* stream);

/* Thread-local description of the last non-OK status returned on this thread ("" if none). */
const char* zg_last_error(void);

/* Kernel timer: while enabled, every launch of the main attention kernels records a pair of HIP
 * events on the launch stream.  zg_kernel_timer_read synchronises on the recorded events and returns,
 * for the kernel family `name` ("attn_swa", "attn_global", "decode_global", "decode_swa",
 * "kv_stage", "decode_merge", "decode_append", "linear", "fp8_quantize", "bwd_prep", "bwd_kv", "bwd_q"),
 * the summed device time in ms and the launch count
 * since the last reset.  Enabling resets the counters. */
int zg_kernel_timer_enable(int32_t on);
int zg_kernel_timer_read(const char* name, double* total_ms, int64_t* launches);
/* Restrict the kernel timer to one kernel family (`name` as above), so that a timed run pays for the events of
 * that family only; NULL or "" times every family again.  Takes effect for launches made after the call. */
int zg_kernel_timer_only(const char* name);

#ifdef __cplusplus
}
#endif

#endif /* ZGATTN_H */
