// zgattn C ABI: argument validation, KV-cache ownership, launch planning.  All device work is
// enqueued on the caller's stream by the kernels in attn_prefill.hip and decode.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/zgattn.h"
#include "common.h"
#include "launch.h"
#include "linear.h"

using namespace zg;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ZG_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// base^(-2i/R) / (2 pi) in double for the pairs i < R/2 (the rotary angle in revolutions per position).
void fill_inv_freq(double* out, int rot_pairs, int rotary_dims, double base) {
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < 64; i++)
    out[i] = i < rot_pairs ? std::pow(base, -2.0 * (double)i / (double)rotary_dims) / two_pi : 0.0;
}

// ---------------------------------------------------------------------------------- kernel timer
struct TimerEntry {
  hipEvent_t start, stop;
  std::string name;
};
std::mutex g_timer_mu;
bool g_timer_on = false;
std::string g_timer_only;   // when not empty, only this kernel family is timed
std::vector<TimerEntry> g_timer_log;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_timer_pool;

struct ScopedTimer {
  bool on = false;
  TimerEntry ent;
  hipStream_t st;
  ScopedTimer(const char* name, hipStream_t s) : st(s) {
    std::lock_guard<std::mutex> lk(g_timer_mu);
    if (!g_timer_on) return;
    if (!g_timer_only.empty() && g_timer_only != name) return;
    if (g_timer_pool.empty()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
      g_timer_pool.push_back({a, b});
    }
    ent.start = g_timer_pool.back().first;
    ent.stop = g_timer_pool.back().second;
    g_timer_pool.pop_back();
    ent.name = name;
    on = hipEventRecord(ent.start, st) == hipSuccess;
  }
  ~ScopedTimer() {
    if (!on) return;
    (void)hipEventRecord(ent.stop, st);
    std::lock_guard<std::mutex> lk(g_timer_mu);
    g_timer_log.push_back(ent);
  }
};

}  // namespace

// ---------------------------------------------------------------------------------- KV cache
struct zg_kv_cache {
  zg_cache_desc desc;
  std::vector<int32_t> is_global;   // [L]
  std::vector<int32_t> glob_ids, swa_ids;
  std::vector<LayerDesc> layers;    // host copy
  std::vector<int64_t> length;      // [L][B]
  int device = 0;
  void* arena = nullptr;
  uint64_t arena_bytes = 0;
  LayerDesc* d_layers = nullptr;
  int32_t* d_glob = nullptr;
  int32_t* d_swa = nullptr;
  float* part_m = nullptr;
  float* part_l = nullptr;
  float* part_acc = nullptr;
  int32_t max_chunks = 0;
};

namespace {

int check_desc(const zg_cache_desc* d) {
  if (!d) return fail(ZG_EINVAL, "null cache descriptor");
  if (d->n_layers < 1 || d->n_layers > kMaxLayers) return fail(ZG_EINVAL, "n_layers must be in 1..%d", kMaxLayers);
  if (d->n_global < 0 || d->n_global > d->n_layers) return fail(ZG_EINVAL, "n_global out of range");
  if (d->n_global > 0 && !d->global_layers) return fail(ZG_EINVAL, "global_layers is null");
  if (d->batch < 1 || d->n_kv_heads < 1) return fail(ZG_EINVAL, "batch and n_kv_heads must be >= 1");
  if (d->window < 1) return fail(ZG_EINVAL, "window must be >= 1");
  if (d->max_tokens < 1) return fail(ZG_EINVAL, "max_tokens must be >= 1");
  std::vector<int> seen(d->n_layers + 1, 0);
  for (int i = 0; i < d->n_global; i++) {
    const int l = d->global_layers[i];
    if (l < 1 || l > d->n_layers) return fail(ZG_EINVAL, "global layer %d outside 1..%d", l, d->n_layers);
    if (seen[l]++) return fail(ZG_EINVAL, "global layer %d listed twice", l);
  }
  if (d->head_dim != kHeadDim) return fail(ZG_EUNSUPPORTED, "head_dim %d: only 128 is implemented", d->head_dim);
  return ZG_OK;
}

int check_layer(const zg_kv_cache* c, int32_t layer) {
  if (!c) return fail(ZG_EINVAL, "null cache");
  if (layer < 1 || layer > c->desc.n_layers) return fail(ZG_EINVAL, "layer %d outside 1..%d", layer, c->desc.n_layers);
  return ZG_OK;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) (void)hipSetDevice(dev);
    else prev = -1;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

}  // namespace

extern "C" uint64_t kv_cache_footprint_bytes(const zg_cache_desc* d, int64_t tokens) {
  if (check_desc(d) != ZG_OK || tokens < 0) return 0;
  std::vector<int> glob(d->n_layers + 1, 0);
  for (int i = 0; i < d->n_global; i++) glob[d->global_layers[i]] = 1;
  const uint64_t per_pos = 2ull * d->n_kv_heads * d->head_dim * 2ull;
  uint64_t total = 0;
  for (int l = 1; l <= d->n_layers; l++) {
    const int64_t n = glob[l] ? tokens : (tokens < d->window ? tokens : d->window);
    total += per_pos * (uint64_t)n;
  }
  return total * (uint64_t)d->batch;
}

extern "C" int kv_cache_alloc(const zg_cache_desc* d, zg_kv_cache** out, uint64_t* bytes_out) {
  if (!out) return fail(ZG_EINVAL, "null output handle");
  *out = nullptr;
  int rc = check_desc(d);
  if (rc) return rc;
  zg_kv_cache* c = new (std::nothrow) zg_kv_cache();
  if (!c) return fail(ZG_ENOMEM, "host allocation failed");
  c->desc = *d;
  c->desc.global_layers = nullptr;   // not retained
  c->is_global.assign(d->n_layers, 0);
  for (int i = 0; i < d->n_global; i++) c->is_global[d->global_layers[i] - 1] = 1;
  for (int l = 0; l < d->n_layers; l++) (c->is_global[l] ? c->glob_ids : c->swa_ids).push_back(l);
  c->length.assign((size_t)d->n_layers * d->batch, 0);
  if (hipGetDevice(&c->device) != hipSuccess) { delete c; return fail(ZG_EHIP, "hipGetDevice failed"); }

  // arena layout: per layer K then V, each [B][Hkv][slots][D] bf16, 256-byte aligned
  const uint64_t row = (uint64_t)kHeadDim * 2;
  uint64_t off = 0;
  std::vector<uint64_t> koff(d->n_layers), voff(d->n_layers);
  c->layers.resize(d->n_layers);
  for (int l = 0; l < d->n_layers; l++) {
    const int64_t slots = c->is_global[l] ? d->max_tokens : d->window;
    const uint64_t bytes = (uint64_t)d->batch * d->n_kv_heads * (uint64_t)slots * row;
    koff[l] = off; off += (bytes + 255) & ~255ull;
    voff[l] = off; off += (bytes + 255) & ~255ull;
    c->layers[l].slots = slots;
    c->layers[l].is_global = c->is_global[l];
  }
  int gi = 0, si = 0;
  for (int l = 0; l < d->n_layers; l++) c->layers[l].index = c->is_global[l] ? gi++ : si++;
  c->max_chunks = (int32_t)((d->max_tokens + kDecodeChunk - 1) / kDecodeChunk);
  const int G_max = 8;   // partial buffers sized for the largest supported group
  const uint64_t n_part = (uint64_t)c->glob_ids.size() * d->batch * d->n_kv_heads * c->max_chunks * G_max;
  const uint64_t part_off = off;
  off += ((n_part * 4 + 255) & ~255ull) * 2 + ((n_part * kHeadDim * 4 + 255) & ~255ull);
  const uint64_t meta_off = off;
  off += (sizeof(LayerDesc) * d->n_layers + 255) & ~255ull;
  off += 2 * ((sizeof(int32_t) * d->n_layers + 255) & ~255ull);

  hipError_t e = hipMalloc(&c->arena, off);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete c;
    return fail(ZG_ENOMEM, "hipMalloc of %llu bytes failed: %s", (unsigned long long)off, hipGetErrorString(e));
  }
  c->arena_bytes = off;
  char* base = static_cast<char*>(c->arena);
  for (int l = 0; l < d->n_layers; l++) {
    c->layers[l].k = reinterpret_cast<uint16_t*>(base + koff[l]);
    c->layers[l].v = reinterpret_cast<uint16_t*>(base + voff[l]);
  }
  c->part_m = reinterpret_cast<float*>(base + part_off);
  c->part_l = reinterpret_cast<float*>(base + part_off + ((n_part * 4 + 255) & ~255ull));
  c->part_acc = reinterpret_cast<float*>(base + part_off + 2 * ((n_part * 4 + 255) & ~255ull));
  c->d_layers = reinterpret_cast<LayerDesc*>(base + meta_off);
  c->d_glob = reinterpret_cast<int32_t*>(base + meta_off + ((sizeof(LayerDesc) * d->n_layers + 255) & ~255ull));
  c->d_swa = c->d_glob + (((sizeof(int32_t) * d->n_layers + 255) & ~255ull) / sizeof(int32_t));

  e = hipMemset(c->arena, 0, meta_off);
  if (e == hipSuccess) e = hipMemcpy(c->d_layers, c->layers.data(), sizeof(LayerDesc) * d->n_layers, hipMemcpyHostToDevice);
  if (e == hipSuccess && !c->glob_ids.empty())
    e = hipMemcpy(c->d_glob, c->glob_ids.data(), sizeof(int32_t) * c->glob_ids.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess && !c->swa_ids.empty())
    e = hipMemcpy(c->d_swa, c->swa_ids.data(), sizeof(int32_t) * c->swa_ids.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(c->arena);
    delete c;
    return hip_fail(e, "initialising the KV cache");
  }
  *out = c;
  if (bytes_out) *bytes_out = off;
  return ZG_OK;
}

extern "C" int kv_cache_free(zg_kv_cache* c) {
  if (!c) return ZG_OK;
  DeviceGuard g(c->device);
  hipError_t e = hipDeviceSynchronize();
  if (c->arena) {
    hipError_t e2 = hipFree(c->arena);
    if (e == hipSuccess) e = e2;
  }
  delete c;
  return e == hipSuccess ? ZG_OK : hip_fail(e, "kv_cache_free");
}

extern "C" int kv_cache_layer_view(const zg_kv_cache* c, int32_t layer, void** k, void** v, int64_t* slots) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  const LayerDesc& ld = c->layers[layer - 1];
  if (k) *k = ld.k;
  if (v) *v = ld.v;
  if (slots) *slots = ld.slots;
  return ZG_OK;
}

extern "C" int kv_cache_length(const zg_kv_cache* c, int32_t layer, int32_t b, int64_t* len) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  if (b < 0 || b >= c->desc.batch) return fail(ZG_EINVAL, "sequence %d outside 0..%d", b, c->desc.batch - 1);
  if (!len) return fail(ZG_EINVAL, "null output");
  *len = c->length[(size_t)(layer - 1) * c->desc.batch + b];
  return ZG_OK;
}

extern "C" int kv_cache_set_length(zg_kv_cache* c, int32_t layer, int32_t b, int64_t len) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  if (b < 0 || b >= c->desc.batch) return fail(ZG_EINVAL, "sequence %d outside 0..%d", b, c->desc.batch - 1);
  if (len < 0 || (c->is_global[layer - 1] && len > c->desc.max_tokens))
    return fail(ZG_ERANGE, "length %lld out of range", (long long)len);
  c->length[(size_t)(layer - 1) * c->desc.batch + b] = len;
  return ZG_OK;
}

namespace {
// Keys a tile-path call stages: positions kbase .. pos0+S-1, kbase = the oldest position the chunk's first query
// sees (0 for a global layer), in whole 64-key tiles.
struct StagePlan {
  int64_t kbase, staged, s_kpad;
};
StagePlan stage_plan(int64_t pos0, int64_t S, int64_t window) {
  const int64_t kbase = window > 0 ? std::max<int64_t>(0, pos0 - window + 1) : 0;
  const int64_t staged = pos0 + S - kbase;
  return {kbase, staged, (staged + 63) / 64 * 64};
}
}  // namespace

extern "C" uint64_t prefill_workspace_bytes_at(int32_t B, int32_t S, int32_t Hkv, int32_t D, int64_t pos0,
                                               int32_t window) {
  if (B < 0 || S < 0 || Hkv < 0 || D < 0 || pos0 < 0 || window < 0) return 0;
  if (S == 0) return 0;
  const StagePlan pl = stage_plan(pos0, S, window);
  return 2ull * (uint64_t)B * (uint64_t)pl.s_kpad * (uint64_t)Hkv * (uint64_t)D * 2ull;
}

extern "C" uint64_t prefill_workspace_bytes(int32_t B, int32_t S, int32_t Hkv, int32_t D) {
  return prefill_workspace_bytes_at(B, S, Hkv, D, 0, 0);
}

// ---------------------------------------------------------------------------------- prefill
namespace {

// validate_only: check every argument (the tensor pointers need only be non-null) and return without
// enqueueing anything (used by the layer entry points before they launch the projections).
// After a gated chunk with a cache has attended (stream order): its last min(S, W) keys (k_hat, recomputed at their
// absolute positions) and values into the layer's ring, slot position mod W.
int ring_write(const void* k, const void* v, const void* kw, const LayerDesc* ld, int32_t B, int32_t S, int32_t Hkv,
               int32_t window, int64_t pos0, int rot_pairs, float eps, const double* inv_freq_rev, hipStream_t st) {
  RingWriteArgs ra{};
  ra.k = static_cast<const uint16_t*>(k);
  ra.v = static_cast<const uint16_t*>(v);
  ra.kw = static_cast<const uint16_t*>(kw);
  ra.kring = ld->k; ra.vring = ld->v;
  ra.B = B; ra.S = S; ra.Hkv = Hkv; ra.W = window; ra.n = S < window ? S : window; ra.pos0 = pos0;
  ra.rot_pairs = rot_pairs; ra.eps = eps;
  std::memcpy(ra.inv_freq_rev, inv_freq_rev, sizeof ra.inv_freq_rev);
  hipError_t e = launch_ring_write(ra, st);
  if (e != hipSuccess) return hip_fail(e, "ring write launch");
  return ZG_OK;
}

int prefill_common(bool gated, const void* q, const void* k, const void* v, const void* gate, const void* qw,
                   const void* kw, void* out, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                   int32_t window, int32_t R, double base, float eps, int64_t pos0, zg_kv_cache* cache,
                   int32_t layer, void* ws, uint64_t ws_bytes, void* stream, bool validate_only = false,
                   float* lse = nullptr, const char* fn_name = nullptr) {
  const char* fn = fn_name ? fn_name : (gated ? "swa_prefill" : "global_prefill");
  if (B < 0 || S < 0) return fail(ZG_EINVAL, "%s: negative B or S", fn);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(ZG_EINVAL, "%s: Hq (%d) must be a positive multiple of Hkv (%d)", fn, Hq, Hkv);
  if (D != kHeadDim) return fail(ZG_EUNSUPPORTED, "%s: head dim %d, only 128 is implemented", fn, D);
  const int G = Hq / Hkv;
  if (128 % G) return fail(ZG_EUNSUPPORTED, "%s: GQA group %d must divide 128", fn, G);
  if (gated && window < 1) return fail(ZG_EINVAL, "%s: window must be >= 1", fn);
  if (R < 0 || R > D || (R & 1)) return fail(ZG_EINVAL, "%s: rotary_dims %d must be even and in 0..%d", fn, R, D);
  if (!(base > 0.0) || !std::isfinite(base)) return fail(ZG_EINVAL, "%s: rope_base must be positive and finite", fn);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(ZG_EINVAL, "%s: eps must be finite and >= 0", fn);
  if (pos0 < 0) return fail(ZG_EINVAL, "%s: pos0 must be >= 0", fn);
  if (!cache && pos0 != 0) return fail(ZG_EINVAL, "%s: pos0 > 0 needs a cache holding the earlier positions", fn);
  if ((int64_t)B * S * Hq >= (1ll << 40)) return fail(ZG_ERANGE, "%s: problem too large", fn);
  // the kernels index positions and per-(b, head) rows with 32-bit integers
  if (pos0 + S >= (1ll << 31) || (int64_t)S * Hkv * D >= (1ll << 31))
    return fail(ZG_ERANGE, "%s: positions or chunk beyond the 32-bit row range", fn);
  if (cache) {
    int rc = check_layer(cache, layer);
    if (rc) return rc;
    if (cache->desc.batch != B) return fail(ZG_EINVAL, "%s: cache batch %d != B %d", fn, cache->desc.batch, B);
    if (cache->desc.n_kv_heads != Hkv) return fail(ZG_EINVAL, "%s: cache has %d KV heads, not %d", fn, cache->desc.n_kv_heads, Hkv);
    const bool lg = cache->is_global[layer - 1] != 0;
    if (lg == gated) return fail(ZG_EINVAL, "%s: layer %d of the cache is a %s layer", fn, layer, lg ? "global" : "gated-SWA");
    if (gated && cache->desc.window != window) return fail(ZG_EINVAL, "%s: window %d != cache window %d", fn, window, cache->desc.window);
    for (int b = 0; b < B; b++)
      if (cache->length[(size_t)(layer - 1) * B + b] != pos0)
        return fail(ZG_ERANGE, "%s: cache length of sequence %d is %lld, pos0 is %lld", fn, b,
                    (long long)cache->length[(size_t)(layer - 1) * B + b], (long long)pos0);
    if (!gated && pos0 + S > cache->desc.max_tokens)
      return fail(ZG_ERANGE, "%s: positions up to %lld exceed the cache capacity %lld", fn, (long long)(pos0 + S),
                  (long long)cache->desc.max_tokens);
  }
  if (B == 0 || S == 0) return ZG_OK;
  if (!q || !k || !v || !qw || !kw || !out || (gated && !gate)) return fail(ZG_EINVAL, "%s: null tensor pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(qw) || !aligned16(kw) || !aligned16(out) ||
      (gated && !aligned16(gate)))
    return fail(ZG_EINVAL, "%s: tensors must be 16-byte aligned", fn);
  if (!ws) return fail(ZG_EINVAL, "%s: workspace required", fn);
  if (!aligned16(ws)) return fail(ZG_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  const uint64_t ws_need = prefill_workspace_bytes_at(B, S, Hkv, D, cache ? pos0 : 0, gated ? window : 0);
  if (ws_bytes < ws_need)
    return fail(ZG_ERANGE, "%s: workspace of %llu bytes < %llu needed", fn, (unsigned long long)ws_bytes,
                (unsigned long long)ws_need);
  if (cache) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != cache->device)
      return fail(ZG_EINVAL, "%s: the cache lives on device %d, the current device is %d", fn, cache->device, cur);
  }

  if (validate_only) return ZG_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int rot_pairs = R / 2;
  if (lse && cache) return fail(ZG_EINVAL, "%s: the training forward takes no cache", fn);
  if (gated && G == 4 && window <= 128 && rot_pairs <= 32) {
    // streaming SWA kernel: k_hat computed in its tile loader, no workspace pass; with a cache, the window's keys
    // before the chunk come from the layer's ring, and the chunk's last keys go to the ring afterwards (it carries
    // the queries' RoPE for the pairs of the first 64 dims; more rotary dims take the tile path)
    const LayerDesc* ld = cache ? &cache->layers[layer - 1] : nullptr;
    SwaStreamArgs sa{};
    sa.q = static_cast<const uint16_t*>(q);
    sa.k = static_cast<const uint16_t*>(k);
    sa.v = static_cast<const uint16_t*>(v);
    sa.gate = static_cast<const uint16_t*>(gate);
    sa.qw = static_cast<const uint16_t*>(qw);
    sa.kw = static_cast<const uint16_t*>(kw);
    sa.out = static_cast<uint16_t*>(out);
    sa.B = B; sa.S = S; sa.Hq = Hq; sa.Hkv = Hkv; sa.G = G;
    sa.window = window;
    sa.rot_pairs = rot_pairs;
    sa.eps = eps;
    sa.q_scale = (float)(1.4426950408889634 / std::sqrt((double)D));
    sa.n_units = B * Hkv;
    sa.run = swa_stream_run_length(S, sa.n_units);
    sa.lse = lse;
    sa.pos0 = (int32_t)(cache ? pos0 : 0);
    if (cache && pos0 > 0) { sa.ck = ld->k; sa.cv = ld->v; }
    fill_inv_freq(sa.inv_freq_rev, rot_pairs, R, base);
    {
      ScopedTimer tm("attn_swa", st);
      hipError_t e = launch_swa_stream(sa, st);
      if (e != hipSuccess) return hip_fail(e, "attention launch");
    }
    if (cache) {
      const int rc = ring_write(k, v, kw, ld, B, S, Hkv, window, pos0, rot_pairs, eps, sa.inv_freq_rev, st);
      if (rc) return rc;
      for (int b = 0; b < B; b++) cache->length[(size_t)(layer - 1) * B + b] = pos0 + S;
    }
    return ZG_OK;
  }
  // tile path: stage the keys the chunk sees (its own, and with a cache the earlier positions from the cache) as
  // fp16 tiles in the workspace, then the tile kernel
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  const LayerDesc* ld = cache ? &cache->layers[layer - 1] : nullptr;
  const StagePlan pl = stage_plan(cache ? pos0 : 0, S, gated ? window : 0);
  StageArgs sa{};
  sa.k = k16;
  sa.v = v16;
  sa.kw = static_cast<const uint16_t*>(kw);
  if (cache) {
    sa.slots = ld->slots;
    sa.ring = gated ? 1 : 0;
    if (pl.kbase < pos0) { sa.ck = ld->k; sa.cv = ld->v; }
    if (!gated) { sa.dk = ld->k; sa.dv = ld->v; }   // the chunk's rows of a global layer's cache
  }
  sa.kt = static_cast<uint16_t*>(ws);
  sa.vt = sa.kt + (int64_t)B * Hkv * pl.s_kpad * kHeadDim;
  sa.pos0 = (int32_t)(cache ? pos0 : 0);
  sa.kbase = (int32_t)pl.kbase;
  sa.B = B; sa.S = S; sa.S_kpad = (int32_t)pl.s_kpad; sa.Hkv = Hkv;
  sa.rot_pairs = rot_pairs;
  sa.eps = eps;
  fill_inv_freq(sa.inv_freq_rev, rot_pairs, R, base);
  {
    ScopedTimer tm("kv_stage", st);
    hipError_t e = launch_kv_stage(sa, st);
    if (e != hipSuccess) return hip_fail(e, "key staging launch");
  }
  TileAttnArgs ta{};
  ta.q = static_cast<const uint16_t*>(q);
  ta.gate = gated ? static_cast<const uint16_t*>(gate) : nullptr;
  ta.qw = static_cast<const uint16_t*>(qw);
  ta.out = static_cast<uint16_t*>(out);
  ta.lse = lse;
  ta.kt = sa.kt; ta.vt = sa.vt;
  ta.pos0 = sa.pos0; ta.kbase = sa.kbase;
  ta.B = B; ta.S = S; ta.S_kpad = sa.S_kpad; ta.Hq = Hq; ta.Hkv = Hkv; ta.G = G; ta.P = 128 / G;
  ta.window = gated ? window : 0;
  ta.rot_pairs = rot_pairs;
  ta.eps = eps;
  ta.q_scale = (float)(1.4426950408889634 / std::sqrt((double)D));
  ta.n_units = B * Hkv;
  std::memcpy(ta.inv_freq_rev, sa.inv_freq_rev, sizeof ta.inv_freq_rev);
  {
    ScopedTimer tm(gated ? "attn_swa" : "attn_global", st);
    ta.n_qtiles = (S + 2 * ta.P - 1) / (2 * ta.P);   // 256 query rows = G heads x 2P positions per work-group
    hipError_t e = launch_attn_pp(ta, gated, st);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
  }
  // a gated layer with a cache: the chunk's last min(S, W) positions go to the ring (the staging has read the
  // ring's earlier contents)
  if (gated && cache) {
    const int rc = ring_write(k, v, kw, ld, B, S, Hkv, window, pos0, rot_pairs, eps, sa.inv_freq_rev, st);
    if (rc) return rc;
  }
  if (cache)
    for (int b = 0; b < B; b++) cache->length[(size_t)(layer - 1) * B + b] = pos0 + S;
  return ZG_OK;
}

}  // namespace

extern "C" int swa_prefill(const void* q, const void* k, const void* v, const void* gate, const void* q_norm_w,
                           const void* k_norm_w, void* out, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                           int32_t window, int32_t rotary_dims, double rope_base, float eps, int64_t pos0,
                           zg_kv_cache* cache, int32_t layer, void* workspace, uint64_t workspace_bytes,
                           void* stream) {
  return prefill_common(true, q, k, v, gate, q_norm_w, k_norm_w, out, B, S, Hq, Hkv, D, window, rotary_dims,
                        rope_base, eps, pos0, cache, layer, workspace, workspace_bytes, stream);
}

extern "C" int global_prefill(const void* q, const void* k, const void* v, const void* q_norm_w, const void* k_norm_w,
                              void* out, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                              int32_t rotary_dims, double rope_base, float eps, int64_t pos0, zg_kv_cache* cache,
                              int32_t layer, void* workspace, uint64_t workspace_bytes, void* stream) {
  return prefill_common(false, q, k, v, nullptr, q_norm_w, k_norm_w, out, B, S, Hq, Hkv, D, 0, rotary_dims, rope_base,
                        eps, pos0, cache, layer, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------------- allocation-free global prefill
// The staging workspace of global_prefill_noalloc: one array per GPU, held until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: kernels get the device address that hipGetSymbolAddress
// returns for the current device (kept in g_scratch_dev), never the array's name.
namespace {
constexpr uint64_t kScratchBytes = 64ull << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The device address of this device's scratch array (looked up once per device, with that device current).
int scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(ZG_EUNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(ZG_EHIP, "%s: hipGetSymbolAddress of the scratch array: %s", fn, hipGetErrorString(e));
    }
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return ZG_OK;
}
}  // namespace

extern "C" uint64_t global_prefill_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int global_prefill_noalloc(const void* q, const void* k, const void* v, const void* q_norm_w,
                                      const void* k_norm_w, void* out, int32_t B, int32_t S, int32_t Hq, int32_t Hkv,
                                      int32_t D, int32_t rotary_dims, double rope_base, float eps, int64_t pos0,
                                      zg_kv_cache* cache, int32_t layer, void* stream) {
  const char* fn = "global_prefill_noalloc";
  if (B < 0 || S < 0 || Hkv < 0 || D < 0 || pos0 < 0) return fail(ZG_EINVAL, "%s: negative size or position", fn);
  const uint64_t need = prefill_workspace_bytes_at(B, S, Hkv, D, cache ? pos0 : 0, 0);
  if (need > kScratchBytes)
    return fail(ZG_ERANGE, "%s: the call stages %llu bytes of keys, more than the %llu-byte scratch array", fn,
                (unsigned long long)need, (unsigned long long)kScratchBytes);
  void* ws = nullptr;
  if (B > 0 && S > 0) {
    const int rc = scratch_address(fn, &ws);
    if (rc) return rc;
  }
  return prefill_common(false, q, k, v, nullptr, q_norm_w, k_norm_w, out, B, S, Hq, Hkv, D, 0, rotary_dims, rope_base,
                        eps, pos0, cache, layer, ws, kScratchBytes, stream, false, nullptr, fn);
}

// ---------------------------------------------------------------------------------- training: forward + backward
extern "C" int swa_prefill_train(const void* q, const void* k, const void* v, const void* gate, const void* q_norm_w,
                                 const void* k_norm_w, void* out, float* lse, int32_t B, int32_t S, int32_t Hq,
                                 int32_t Hkv, int32_t D, int32_t window, int32_t rotary_dims, double rope_base,
                                 float eps, void* workspace, uint64_t workspace_bytes, void* stream) {
  if (B > 0 && S > 0 && !lse) return fail(ZG_EINVAL, "swa_prefill_train: null lse");
  return prefill_common(true, q, k, v, gate, q_norm_w, k_norm_w, out, B, S, Hq, Hkv, D, window, rotary_dims, rope_base,
                        eps, 0, nullptr, 0, workspace, workspace_bytes, stream, false, lse, "swa_prefill_train");
}

extern "C" int global_prefill_train(const void* q, const void* k, const void* v, const void* q_norm_w,
                                    const void* k_norm_w, void* out, float* lse, int32_t B, int32_t S, int32_t Hq,
                                    int32_t Hkv, int32_t D, int32_t rotary_dims, double rope_base, float eps,
                                    void* workspace, uint64_t workspace_bytes, void* stream) {
  if (B > 0 && S > 0 && !lse) return fail(ZG_EINVAL, "global_prefill_train: null lse");
  return prefill_common(false, q, k, v, nullptr, q_norm_w, k_norm_w, out, B, S, Hq, Hkv, D, 0, rotary_dims, rope_base,
                        eps, 0, nullptr, 0, workspace, workspace_bytes, stream, false, lse, "global_prefill_train");
}

namespace {
struct BwdLayout {
  uint64_t qh16, qt, da, dat, lse2, delta, kh16, kt, dw_part, total;
};
uint64_t a256(uint64_t x) { return (x + 255) & ~255ull; }
BwdLayout bwd_layout(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D) {
  const uint64_t Sp = ((uint64_t)S + 127) / 128 * 128;
  const uint64_t q2 = (uint64_t)B * Hq * Sp * D * 2, k2 = (uint64_t)B * Hkv * Sp * D * 2;
  const uint64_t rows = (uint64_t)B * Hq * Sp * 4;
  BwdLayout l{};
  uint64_t o = 0;
  l.qh16 = o; o += a256(q2);
  l.qt = o; o += a256(q2);
  l.da = o; o += a256(q2);
  l.dat = o; o += a256(q2);
  l.lse2 = o; o += a256(rows);
  l.delta = o; o += a256(rows);
  l.kh16 = o; o += a256(k2);
  l.kt = o; o += a256(k2);
  const uint64_t n_blk = (uint64_t)B * Hkv * (((uint64_t)S + 31) / 32 + ((uint64_t)S + 127) / 128);
  l.dw_part = o; o += a256(n_blk * D * 4);
  l.total = o;
  return l;
}

int backward_common(bool gated, const void* q, const void* k, const void* v, const void* gate, const void* qw,
                    const void* kw, const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* dgate, float* dqw, float* dkw, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                    int32_t window, int32_t R, double base, float eps, void* ws, uint64_t ws_bytes, void* stream) {
  const char* fn = gated ? "swa_prefill_backward" : "global_prefill_backward";
  if (B < 0 || S < 0) return fail(ZG_EINVAL, "%s: negative B or S", fn);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(ZG_EINVAL, "%s: Hq (%d) must be a positive multiple of Hkv (%d)", fn, Hq, Hkv);
  if (D != kHeadDim) return fail(ZG_EUNSUPPORTED, "%s: head dim %d, only 128 is implemented", fn, D);
  if (Hq / Hkv != 4) return fail(ZG_EUNSUPPORTED, "%s: GQA group %d, only 4 is implemented", fn, Hq / Hkv);
  if (gated && window < 1) return fail(ZG_EINVAL, "%s: window must be >= 1", fn);
  if (R < 0 || R > D || (R & 1)) return fail(ZG_EINVAL, "%s: rotary_dims %d must be even and in 0..%d", fn, R, D);
  if (!(base > 0.0) || !std::isfinite(base)) return fail(ZG_EINVAL, "%s: rope_base must be positive and finite", fn);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(ZG_EINVAL, "%s: eps must be finite and >= 0", fn);
  if ((int64_t)S >= (1ll << 30) || (int64_t)B * Hq * (((int64_t)S + 127) / 128 * 128) * D >= (1ll << 40))
    return fail(ZG_ERANGE, "%s: problem too large", fn);
  if (!dqw || !dkw) return fail(ZG_EINVAL, "%s: null norm-weight gradient", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (B == 0 || S == 0) {   // empty: the norm-weight gradients are zero
    hipError_t e = launch_bwd_dw_zero(dqw, dkw, st);
    return e == hipSuccess ? ZG_OK : hip_fail(e, "clearing the norm-weight gradients");
  }
  if (!q || !k || !v || !qw || !kw || !out || !lse || !dout || !dq || !dk || !dv || (gated && (!gate || !dgate)))
    return fail(ZG_EINVAL, "%s: null tensor pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(qw) || !aligned16(kw) || !aligned16(out) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(lse) ||
      (gated && (!aligned16(gate) || !aligned16(dgate))))
    return fail(ZG_EINVAL, "%s: tensors must be 16-byte aligned", fn);
  const BwdLayout L = bwd_layout(B, S, Hq, Hkv, D);
  if (!ws || !aligned16(ws)) return fail(ZG_EINVAL, "%s: a 16-byte aligned workspace is required", fn);
  if (ws_bytes < L.total)
    return fail(ZG_ERANGE, "%s: workspace of %llu bytes < %llu needed", fn, (unsigned long long)ws_bytes,
                (unsigned long long)L.total);
  unsigned char* w = static_cast<unsigned char*>(ws);
  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.gate = gated ? static_cast<const uint16_t*>(gate) : nullptr;
  a.qw = static_cast<const uint16_t*>(qw);
  a.kw = static_cast<const uint16_t*>(kw);
  a.out = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.dgate = gated ? static_cast<uint16_t*>(dgate) : nullptr;
  a.dqw = dqw;
  a.dkw = dkw;
  a.qh16 = reinterpret_cast<uint16_t*>(w + L.qh16);
  a.qt = reinterpret_cast<uint16_t*>(w + L.qt);
  a.da = reinterpret_cast<uint16_t*>(w + L.da);
  a.dat = reinterpret_cast<uint16_t*>(w + L.dat);
  a.nlse2 = reinterpret_cast<float*>(w + L.lse2);
  a.ndelta = reinterpret_cast<float*>(w + L.delta);
  a.kh16 = reinterpret_cast<uint16_t*>(w + L.kh16);
  a.kt = reinterpret_cast<uint16_t*>(w + L.kt);
  a.dw_part = reinterpret_cast<float*>(w + L.dw_part);
  a.n_qblk = B * Hkv * ((S + 31) / 32);
  a.n_kblk = B * Hkv * bwd_k_blocks(S, gated ? window : 0);
  a.B = B; a.S = S; a.Sp = (S + 127) / 128 * 128; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.window = gated ? window : 0;
  a.rot_pairs = R / 2;
  a.eps = eps;
  a.q_scale = (float)(1.4426950408889634 / std::sqrt((double)D));
  fill_inv_freq(a.inv_freq_rev, R / 2, R, base);
  hipError_t e;
  {
    ScopedTimer tm("bwd_prep", st);
    e = launch_bwd_prep(a, st);
  }
  if (e != hipSuccess) return hip_fail(e, "backward prep launch");
  {
    ScopedTimer tm("bwd_kv", st);
    e = launch_bwd_kv(a, st);
  }
  if (e != hipSuccess) return hip_fail(e, "backward dK/dV launch");
  {
    ScopedTimer tm("bwd_q", st);
    e = launch_bwd_q(a, st);
  }
  if (e != hipSuccess) return hip_fail(e, "backward dQ launch");
  e = launch_bwd_dw_reduce(a, st);
  if (e != hipSuccess) return hip_fail(e, "backward dw reduction launch");
  return ZG_OK;
}
}  // namespace

extern "C" uint64_t backward_workspace_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D) {
  if (B < 0 || S < 0 || Hq < 0 || Hkv < 0 || D < 0) return 0;
  return bwd_layout(B, S, Hq, Hkv, D).total;
}

extern "C" int swa_prefill_backward(const void* q, const void* k, const void* v, const void* gate, const void* q_norm_w,
                                    const void* k_norm_w, const void* out, const float* lse, const void* dout, void* dq,
                                    void* dk, void* dv, void* dgate, float* dq_norm_w, float* dk_norm_w, int32_t B,
                                    int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t window, int32_t rotary_dims,
                                    double rope_base, float eps, void* workspace, uint64_t workspace_bytes,
                                    void* stream) {
  return backward_common(true, q, k, v, gate, q_norm_w, k_norm_w, out, lse, dout, dq, dk, dv, dgate, dq_norm_w,
                         dk_norm_w, B, S, Hq, Hkv, D, window, rotary_dims, rope_base, eps, workspace, workspace_bytes,
                         stream);
}

extern "C" int global_prefill_backward(const void* q, const void* k, const void* v, const void* q_norm_w,
                                       const void* k_norm_w, const void* out, const float* lse, const void* dout,
                                       void* dq, void* dk, void* dv, float* dq_norm_w, float* dk_norm_w, int32_t B,
                                       int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t rotary_dims,
                                       double rope_base, float eps, void* workspace, uint64_t workspace_bytes,
                                       void* stream) {
  return backward_common(false, q, k, v, nullptr, q_norm_w, k_norm_w, out, lse, dout, dq, dk, dv, nullptr, dq_norm_w,
                         dk_norm_w, B, S, Hq, Hkv, D, 0, rotary_dims, rope_base, eps, workspace, workspace_bytes,
                         stream);
}

// ---------------------------------------------------------------------------------- projections, layers
extern "C" int linear_bf16(const void* x, const void* w, void* y, int64_t T, int32_t K, int32_t N, void* stream) {
  const char* fn = "linear_bf16";
  if (T < 0 || K < 1 || N < 1) return fail(ZG_EINVAL, "%s: T must be >= 0, K and N >= 1", fn);
  if (T == 0) return ZG_OK;
  if (!x || !w || !y) return fail(ZG_EINVAL, "%s: null tensor pointer", fn);
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return fail(ZG_EINVAL, "%s: tensors must be 16-byte aligned", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  ScopedTimer tm("linear", st);
  const int s = linear_bf16_run(x, w, y, T, K, N, st);
  if (s) return fail(ZG_EHIP, "%s: hipBLASLt %s (T=%lld K=%d N=%d)", fn, blas_status_name(s), (long long)T, K, N);
  return ZG_OK;
}

// ---- FP8 projections with delayed scaling
struct zg_fp8_linear {
  int device = -1;
  int32_t K = 0, N = 0, H = 0;
  int32_t idx = 0;       // history slot of the next call
  void* mem = nullptr;   // device: hist [2][H], partial [2][kFp8MaxBlocks], scale [2], scale_inv [2]
  zg::Fp8State st{};
};

// The FP8 state of a whole layer: tensors 0 = h, 1..4 = W_q, W_k, W_v, W_g, 5 = the attention output o,
// 6 = W_o (W_g unused by a global layer).
enum { kF8H = 0, kF8Wq = 1, kF8Wk = 2, kF8Wv = 3, kF8Wg = 4, kF8O = 5, kF8Wo = 6, kF8LayerTensors = 7 };
struct zg_fp8_layer {
  int device = -1;
  int32_t d_model = 0, Hq = 0, Hkv = 0, D = 0, H = 0;
  int32_t idx = 0;
  void* mem = nullptr;   // device: hist [7][H], partial [7][kFp8MaxBlocks], scale [7], scale_inv [7]
  zg::Fp8State st{};
};

namespace {
// Device memory for n tensors' delayed-scaling state: histories zero, scales and their inverses one.
int fp8_state_alloc(const char* fn, int32_t n, int32_t history, void** mem, zg::Fp8State* st) {
  const size_t P = (size_t)n * ((size_t)history + (size_t)zg::kFp8MaxBlocks);   // floats before the scales
  const size_t bytes = (P + 2 * (size_t)n) * 4;
  if (hipMalloc(mem, bytes) != hipSuccess) { *mem = nullptr; return fail(ZG_ENOMEM, "%s: device allocation failed", fn); }
  float* base = static_cast<float*>(*mem);
  st->hist = base;
  st->partial = base + (size_t)n * history;
  st->scale = base + P;
  st->scale_inv = base + P + n;
  st->H = history;
  st->n = n;
  std::vector<float> init(P + 2 * (size_t)n, 0.0f);
  for (size_t i = P; i < init.size(); i++) init[i] = 1.0f;
  if (hipMemcpy(*mem, init.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(*mem);
    *mem = nullptr;
    return fail(ZG_EHIP, "%s: initialising the state failed", fn);
  }
  return ZG_OK;
}
}  // namespace

namespace {
uint64_t align256(uint64_t x) { return (x + 255) & ~255ull; }
uint64_t layer_activation_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D) {
  const uint64_t T = (uint64_t)B * (uint64_t)S;
  return align256(T * (3ull * Hq + 2ull * Hkv) * (uint64_t)D * 2ull);   // q, g, o and k, v (bf16)
}
}  // namespace

extern "C" uint64_t layer_workspace_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D) {
  if (B < 0 || S < 0 || Hq < 0 || Hkv < 0 || D < 0) return 0;
  return layer_activation_bytes(B, S, Hq, Hkv, D) + prefill_workspace_bytes(B, S, Hkv, D);
}

extern "C" uint64_t fp8_layer_workspace_bytes(int32_t B, int32_t S, int32_t d_model, int32_t Hq, int32_t Hkv,
                                              int32_t D) {
  if (B < 0 || S < 0 || d_model < 0 || Hq < 0 || Hkv < 0 || D < 0) return 0;
  const uint64_t T = (uint64_t)B * (uint64_t)S, dm = (uint64_t)d_model, qd = (uint64_t)Hq * D, kd = (uint64_t)Hkv * D;
  return layer_workspace_bytes(B, S, Hq, Hkv, D) + align256(T * dm) + align256(T * qd) + 2 * align256(qd * dm) +
         2 * align256(kd * dm) + align256(dm * qd);
}

namespace {
// q/k/v(/g) = h W^T, the attention core, y = o W_o^T.  With f8, every projection runs on E4M3 operands under
// delayed scaling (h quantised once for the four input projections, o once for o_proj).
int layer_common(bool gated, const void* h, const void* w_q, const void* w_k, const void* w_v, const void* w_g,
                 const void* w_o, const void* qw, const void* kw, void* y, int32_t B, int32_t S, int32_t d_model,
                 int32_t Hq, int32_t Hkv, int32_t D, int32_t window, int32_t R, double base, float eps, int64_t pos0,
                 zg_kv_cache* cache, int32_t layer, zg_fp8_layer* f8, void* ws, uint64_t ws_bytes, void* stream) {
  const char* fn = f8 ? (gated ? "gated_swa_layer_fp8" : "global_layer_fp8") : (gated ? "gated_swa_layer" : "global_layer");
  if (d_model < 1) return fail(ZG_EINVAL, "%s: d_model must be >= 1", fn);
  if (B < 0 || S < 0 || Hq < 1 || Hkv < 1 || D < 1) return fail(ZG_EINVAL, "%s: bad shape", fn);
  if (f8) {
    if (f8->d_model != d_model || f8->Hq != Hq || f8->Hkv != Hkv || f8->D != D)
      return fail(ZG_EINVAL, "%s: shape (d_model=%d, Hq=%d, Hkv=%d, D=%d) does not match the FP8 state (%d, %d, %d, %d)",
                  fn, d_model, Hq, Hkv, D, f8->d_model, f8->Hq, f8->Hkv, f8->D);
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != f8->device)
      return fail(ZG_EINVAL, "%s: the FP8 state lives on device %d, the current device is %d", fn, f8->device, cur);
  }
  if (B == 0 || S == 0) return ZG_OK;
  if (!h || !w_q || !w_k || !w_v || !w_o || !y || (gated && !w_g)) return fail(ZG_EINVAL, "%s: null tensor pointer", fn);
  if (!aligned16(h) || !aligned16(w_q) || !aligned16(w_k) || !aligned16(w_v) || !aligned16(w_o) || !aligned16(y) ||
      (gated && !aligned16(w_g)))
    return fail(ZG_EINVAL, "%s: tensors must be 16-byte aligned", fn);
  if (!ws || !aligned16(ws)) return fail(ZG_EINVAL, "%s: a 16-byte aligned workspace is required", fn);
  // layout: the activations q [T][Hq*D], k, v [T][Hkv*D], g, o [T][Hq*D]; (FP8) the E4M3 codes of h, o, W_q, W_k,
  // W_v, W_g and W_o; then the attention's workspace, which takes the rest (with a cache at pos0 > 0 the attention
  // stages the earlier positions too, so it needs more than without)
  const uint64_t act = layer_activation_bytes(B, S, Hq, Hkv, D);
  const uint64_t codes = f8 ? fp8_layer_workspace_bytes(B, S, d_model, Hq, Hkv, D) - layer_workspace_bytes(B, S, Hq, Hkv, D) : 0;
  const uint64_t attn_need = prefill_workspace_bytes_at(B, S, Hkv, D, cache ? pos0 : 0, gated ? window : 0);
  const uint64_t need = act + codes + attn_need;
  if (ws_bytes < need)
    return fail(ZG_ERANGE, "%s: workspace of %llu bytes < %llu needed", fn, (unsigned long long)ws_bytes,
                (unsigned long long)need);
  const int64_t T = (int64_t)B * S;
  uint16_t* q = static_cast<uint16_t*>(ws);
  uint16_t* k = q + T * Hq * D;
  uint16_t* v = k + T * Hkv * D;
  uint16_t* g = v + T * Hkv * D;
  uint16_t* o = g + T * Hq * D;
  void* aws = static_cast<unsigned char*>(ws) + act + codes;
  const uint64_t aws_bytes = ws_bytes - act - codes;
  // the attention's arguments first, so a bad one enqueues nothing
  int rc = prefill_common(gated, q, k, v, gated ? g : nullptr, qw, kw, o, B, S, Hq, Hkv, D, window, R, base, eps, pos0,
                          cache, layer, aws, aws_bytes, stream, /*validate_only=*/true);
  if (rc) return rc;
  if (!f8) {
    if ((rc = linear_bf16(h, w_q, q, T, d_model, Hq * D, stream))) return rc;
    if ((rc = linear_bf16(h, w_k, k, T, d_model, Hkv * D, stream))) return rc;
    if ((rc = linear_bf16(h, w_v, v, T, d_model, Hkv * D, stream))) return rc;
    if (gated && (rc = linear_bf16(h, w_g, g, T, d_model, Hq * D, stream))) return rc;
    rc = prefill_common(gated, q, k, v, gated ? g : nullptr, qw, kw, o, B, S, Hq, Hkv, D, window, R, base, eps, pos0,
                        cache, layer, aws, aws_bytes, stream);
    if (rc) return rc;
    return linear_bf16(o, w_o, y, T, Hq * D, d_model, stream);
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t dm = d_model, qd = (int64_t)Hq * D, kd = (int64_t)Hkv * D;
  uint8_t* hc = static_cast<uint8_t*>(ws) + act;
  uint8_t* oc = hc + align256(T * dm);
  uint8_t* wc[kF8LayerTensors] = {};
  wc[kF8Wq] = oc + align256(T * qd);
  wc[kF8Wk] = wc[kF8Wq] + align256(qd * dm);
  wc[kF8Wv] = wc[kF8Wk] + align256(kd * dm);
  wc[kF8Wg] = wc[kF8Wv] + align256(kd * dm);
  wc[kF8Wo] = wc[kF8Wg] + align256(qd * dm);
  const Fp8State& fs = f8->st;
  Fp8Blocks nb{};
  auto quant = [&](int t, const void* src, uint8_t* dst, int64_t n) {
    nb.n[t] = fp8_quantize_blocks(n);
    return launch_fp8_quantize(static_cast<const uint16_t*>(src), dst, n, fs.scale + t, fs.partial + (int64_t)t * kFp8MaxBlocks, st);
  };
  auto gemm = [&](const uint8_t* xc, int tx, int tw, void* out, int32_t K, int32_t N) {
    ScopedTimer tm("linear", st);
    const int s = linear_fp8_run(xc, wc[tw], out, T, K, N, fs.scale_inv + tx, fs.scale_inv + tw, st);
    return s ? fail(ZG_EHIP, "%s: hipBLASLt %s (T=%lld K=%d N=%d)", fn, blas_status_name(s), (long long)T, K, N) : ZG_OK;
  };
  hipError_t e;
  {
    ScopedTimer tm("fp8_quantize", st);
    e = quant(kF8H, h, hc, T * dm);
    if (e == hipSuccess) e = quant(kF8Wq, w_q, wc[kF8Wq], qd * dm);
    if (e == hipSuccess) e = quant(kF8Wk, w_k, wc[kF8Wk], kd * dm);
    if (e == hipSuccess) e = quant(kF8Wv, w_v, wc[kF8Wv], kd * dm);
    if (e == hipSuccess && gated) e = quant(kF8Wg, w_g, wc[kF8Wg], qd * dm);
  }
  if (e != hipSuccess) return hip_fail(e, "fp8 quantize launch");
  if ((rc = gemm(hc, kF8H, kF8Wq, q, d_model, (int32_t)qd))) return rc;
  if ((rc = gemm(hc, kF8H, kF8Wk, k, d_model, (int32_t)kd))) return rc;
  if ((rc = gemm(hc, kF8H, kF8Wv, v, d_model, (int32_t)kd))) return rc;
  if (gated && (rc = gemm(hc, kF8H, kF8Wg, g, d_model, (int32_t)qd))) return rc;
  rc = prefill_common(gated, q, k, v, gated ? g : nullptr, qw, kw, o, B, S, Hq, Hkv, D, window, R, base, eps, pos0, cache,
                      layer, aws, aws_bytes, stream);
  if (rc) return rc;
  {
    ScopedTimer tm("fp8_quantize", st);
    e = quant(kF8O, o, oc, T * qd);
    if (e == hipSuccess) e = quant(kF8Wo, w_o, wc[kF8Wo], dm * qd);
  }
  if (e != hipSuccess) return hip_fail(e, "fp8 quantize launch");
  if ((rc = gemm(oc, kF8O, kF8Wo, y, (int32_t)qd, d_model))) return rc;
  e = launch_fp8_finalize(fs, f8->idx, nb, st);
  if (e != hipSuccess) return hip_fail(e, "fp8 finalize launch");
  f8->idx = (f8->idx + 1) % f8->H;
  return ZG_OK;
}
}  // namespace

extern "C" int fp8_layer_alloc(int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D, int32_t history,
                               zg_fp8_layer** out) {
  const char* fn = "fp8_layer_alloc";
  if (!out) return fail(ZG_EINVAL, "%s: null output handle", fn);
  *out = nullptr;
  if (d_model < 1 || Hq < 1 || Hkv < 1 || D < 1 || history < 1)
    return fail(ZG_EINVAL, "%s: d_model, Hq, Hkv, D and history must be >= 1", fn);
  if (d_model % 8 || ((int64_t)Hq * D) % 8)
    return fail(ZG_EUNSUPPORTED, "%s: d_model (%d) and Hq*D (%d) must be multiples of 8", fn, d_model, Hq * D);
  auto* f = new (std::nothrow) zg_fp8_layer();
  if (!f) return fail(ZG_ENOMEM, "%s: host allocation failed", fn);
  f->d_model = d_model; f->Hq = Hq; f->Hkv = Hkv; f->D = D; f->H = history;
  if (hipGetDevice(&f->device) != hipSuccess) { delete f; return fail(ZG_EHIP, "%s: no current device", fn); }
  if (int rc = fp8_state_alloc(fn, kF8LayerTensors, history, &f->mem, &f->st)) { delete f; return rc; }
  *out = f;
  return ZG_OK;
}

extern "C" int fp8_layer_free(zg_fp8_layer* f) {
  if (!f) return ZG_OK;
  (void)hipDeviceSynchronize();
  (void)hipFree(f->mem);
  delete f;
  return ZG_OK;
}

extern "C" int fp8_layer_scales(const zg_fp8_layer* f, float* scales_out) {
  if (!f || !scales_out) return fail(ZG_EINVAL, "fp8_layer_scales: null argument");
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(scales_out, f->st.scale, kF8LayerTensors * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(ZG_EHIP, "fp8_layer_scales: reading the device state failed");
  return ZG_OK;
}

extern "C" int fp8_linear_alloc(int32_t K, int32_t N, int32_t history, zg_fp8_linear** out) {
  const char* fn = "fp8_linear_alloc";
  if (!out) return fail(ZG_EINVAL, "%s: null output handle", fn);
  *out = nullptr;
  if (K < 1 || N < 1 || history < 1) return fail(ZG_EINVAL, "%s: K, N and history must be >= 1", fn);
  if (K % 8) return fail(ZG_EUNSUPPORTED, "%s: K = %d must be a multiple of 8", fn, K);
  auto* f = new (std::nothrow) zg_fp8_linear();
  if (!f) return fail(ZG_ENOMEM, "%s: host allocation failed", fn);
  f->K = K; f->N = N; f->H = history;
  if (hipGetDevice(&f->device) != hipSuccess) { delete f; return fail(ZG_EHIP, "%s: no current device", fn); }
  if (int rc = fp8_state_alloc(fn, 2, history, &f->mem, &f->st)) { delete f; return rc; }
  *out = f;
  return ZG_OK;
}

extern "C" int fp8_linear_free(zg_fp8_linear* f) {
  if (!f) return ZG_OK;
  (void)hipDeviceSynchronize();
  (void)hipFree(f->mem);
  delete f;
  return ZG_OK;
}

extern "C" int fp8_linear_scales(const zg_fp8_linear* f, float* scales_out) {
  if (!f || !scales_out) return fail(ZG_EINVAL, "fp8_linear_scales: null argument");
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(scales_out, f->st.scale, 2 * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(ZG_EHIP, "fp8_linear_scales: reading the device state failed");
  return ZG_OK;
}

extern "C" uint64_t fp8_linear_workspace_bytes(int64_t T, int32_t K, int32_t N) {
  if (T < 0 || K < 0 || N < 0) return 0;
  return align256((uint64_t)T * (uint64_t)K) + align256((uint64_t)N * (uint64_t)K);
}

extern "C" int linear_fp8_delayed(const void* x, const void* w, void* y, int64_t T, int32_t K, int32_t N,
                                  zg_fp8_linear* f, void* workspace, uint64_t workspace_bytes, void* stream) {
  const char* fn = "linear_fp8_delayed";
  if (!f) return fail(ZG_EINVAL, "%s: null state", fn);
  if (T < 0 || K != f->K || N != f->N) return fail(ZG_EINVAL, "%s: shape (T=%lld, K=%d, N=%d) does not match the state (K=%d, N=%d)", fn, (long long)T, K, N, f->K, f->N);
  if (T == 0) return ZG_OK;
  if (!x || !w || !y) return fail(ZG_EINVAL, "%s: null tensor pointer", fn);
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return fail(ZG_EINVAL, "%s: tensors must be 16-byte aligned", fn);
  if (!workspace || !aligned16(workspace)) return fail(ZG_EINVAL, "%s: a 16-byte aligned workspace is required", fn);
  if (workspace_bytes < fp8_linear_workspace_bytes(T, K, N))
    return fail(ZG_ERANGE, "%s: workspace of %llu bytes < %llu needed", fn, (unsigned long long)workspace_bytes,
                (unsigned long long)fp8_linear_workspace_bytes(T, K, N));
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != f->device)
    return fail(ZG_EINVAL, "%s: the state lives on device %d, the current device is %d", fn, f->device, cur);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  uint8_t* wq = xq + align256((uint64_t)T * K);
  hipError_t e;
  {
    ScopedTimer tm("fp8_quantize", st);
    e = launch_fp8_quantize(static_cast<const uint16_t*>(x), xq, T * K, f->st.scale + 0, f->st.partial, st);
    if (e == hipSuccess)
      e = launch_fp8_quantize(static_cast<const uint16_t*>(w), wq, (int64_t)N * K, f->st.scale + 1,
                              f->st.partial + zg::kFp8MaxBlocks, st);
  }
  if (e != hipSuccess) return hip_fail(e, "fp8 quantize launch");
  {
    ScopedTimer tm("linear", st);
    const int s = linear_fp8_run(xq, wq, y, T, K, N, f->st.scale_inv + 0, f->st.scale_inv + 1, st);
    if (s) return fail(ZG_EHIP, "%s: hipBLASLt %s (T=%lld K=%d N=%d)", fn, blas_status_name(s), (long long)T, K, N);
  }
  Fp8Blocks nb{};
  nb.n[0] = fp8_quantize_blocks(T * K);
  nb.n[1] = fp8_quantize_blocks((int64_t)N * K);
  e = launch_fp8_finalize(f->st, f->idx, nb, st);
  if (e != hipSuccess) return hip_fail(e, "fp8 finalize launch");
  f->idx = (f->idx + 1) % f->H;
  return ZG_OK;
}

extern "C" int gated_swa_layer(const void* h, const void* w_q, const void* w_k, const void* w_v, const void* w_g,
                               const void* w_o, const void* q_norm_w, const void* k_norm_w, void* y, int32_t B,
                               int32_t S, int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D, int32_t window,
                               int32_t rotary_dims, double rope_base, float eps, int64_t pos0, zg_kv_cache* cache,
                               int32_t layer, void* workspace, uint64_t workspace_bytes, void* stream) {
  return layer_common(true, h, w_q, w_k, w_v, w_g, w_o, q_norm_w, k_norm_w, y, B, S, d_model, Hq, Hkv, D, window,
                      rotary_dims, rope_base, eps, pos0, cache, layer, nullptr, workspace, workspace_bytes, stream);
}

extern "C" int global_layer(const void* h, const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                            const void* q_norm_w, const void* k_norm_w, void* y, int32_t B, int32_t S, int32_t d_model,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t rotary_dims, double rope_base, float eps,
                            int64_t pos0, zg_kv_cache* cache, int32_t layer, void* workspace, uint64_t workspace_bytes,
                            void* stream) {
  return layer_common(false, h, w_q, w_k, w_v, nullptr, w_o, q_norm_w, k_norm_w, y, B, S, d_model, Hq, Hkv, D, 0,
                      rotary_dims, rope_base, eps, pos0, cache, layer, nullptr, workspace, workspace_bytes, stream);
}

extern "C" int gated_swa_layer_fp8(const void* h, const void* w_q, const void* w_k, const void* w_v, const void* w_g,
                                   const void* w_o, const void* q_norm_w, const void* k_norm_w, void* y, int32_t B,
                                   int32_t S, int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D, int32_t window,
                                   int32_t rotary_dims, double rope_base, float eps, int64_t pos0, zg_kv_cache* cache,
                                   int32_t layer, zg_fp8_layer* fp8, void* workspace, uint64_t workspace_bytes,
                                   void* stream) {
  if (!fp8) return fail(ZG_EINVAL, "gated_swa_layer_fp8: null FP8 state");
  return layer_common(true, h, w_q, w_k, w_v, w_g, w_o, q_norm_w, k_norm_w, y, B, S, d_model, Hq, Hkv, D, window,
                      rotary_dims, rope_base, eps, pos0, cache, layer, fp8, workspace, workspace_bytes, stream);
}

extern "C" int global_layer_fp8(const void* h, const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                                const void* q_norm_w, const void* k_norm_w, void* y, int32_t B, int32_t S,
                                int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D, int32_t rotary_dims,
                                double rope_base, float eps, int64_t pos0, zg_kv_cache* cache, int32_t layer,
                                zg_fp8_layer* fp8, void* workspace, uint64_t workspace_bytes, void* stream) {
  if (!fp8) return fail(ZG_EINVAL, "global_layer_fp8: null FP8 state");
  return layer_common(false, h, w_q, w_k, w_v, nullptr, w_o, q_norm_w, k_norm_w, y, B, S, d_model, Hq, Hkv, D, 0,
                      rotary_dims, rope_base, eps, pos0, cache, layer, fp8, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------------- decode
extern "C" int hybrid_decode_step(const void* q, const void* k, const void* v, const void* gate, const void* q_norm_w,
                                  const void* k_norm_w, void* out, const int64_t* positions, int32_t Hq,
                                  int32_t R, double base, float eps, zg_kv_cache* cache, void* stream) {
  const char* fn = "hybrid_decode_step";
  if (!cache) return fail(ZG_EINVAL, "%s: null cache", fn);
  const zg_cache_desc& d = cache->desc;
  const int B = d.batch, Hkv = d.n_kv_heads, L = d.n_layers;
  if (Hq < 1 || Hq % Hkv) return fail(ZG_EINVAL, "%s: Hq (%d) must be a positive multiple of Hkv (%d)", fn, Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(ZG_EUNSUPPORTED, "%s: GQA group %d (1, 2, 4 or 8 implemented)", fn, G);
  if (B > kMaxDecodeBatch) return fail(ZG_EUNSUPPORTED, "%s: batch %d > %d", fn, B, kMaxDecodeBatch);
  if (R < 0 || R > kHeadDim || (R & 1)) return fail(ZG_EINVAL, "%s: rotary_dims %d must be even and in 0..128", fn, R);
  if (!(base > 0.0) || !std::isfinite(base)) return fail(ZG_EINVAL, "%s: rope_base must be positive and finite", fn);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(ZG_EINVAL, "%s: eps must be finite and >= 0", fn);
  if (!positions) return fail(ZG_EINVAL, "%s: null positions", fn);
  if (!q || !k || !v || !gate || !q_norm_w || !k_norm_w || !out) return fail(ZG_EINVAL, "%s: null tensor pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gate) || !aligned16(q_norm_w) ||
      !aligned16(k_norm_w) || !aligned16(out))
    return fail(ZG_EINVAL, "%s: tensors must be 16-byte aligned", fn);
  int64_t pmax = 0;
  for (int b = 0; b < B; b++) {
    const int64_t p = positions[b];
    if (p < 0) return fail(ZG_ERANGE, "%s: negative position for sequence %d", fn, b);
    if (p >= d.max_tokens) return fail(ZG_ERANGE, "%s: position %lld of sequence %d reaches the capacity %lld", fn,
                                       (long long)p, b, (long long)d.max_tokens);
    for (int l = 0; l < L; l++)
      if (cache->length[(size_t)l * B + b] != p)
        return fail(ZG_ERANGE, "%s: layer %d of sequence %d holds %lld positions, the new token is at %lld", fn, l + 1,
                    b, (long long)cache->length[(size_t)l * B + b], (long long)p);
    if (p > pmax) pmax = p;
  }
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != cache->device)
    return fail(ZG_EINVAL, "%s: the cache lives on device %d, the current device is %d", fn, cache->device, cur);

  hipStream_t st = static_cast<hipStream_t>(stream);
  DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.gate = static_cast<const uint16_t*>(gate);
  a.qw = static_cast<const uint16_t*>(q_norm_w);
  a.kw = static_cast<const uint16_t*>(k_norm_w);
  a.out = static_cast<uint16_t*>(out);
  a.layers = cache->d_layers;
  a.glob_ids = cache->d_glob;
  a.swa_ids = cache->d_swa;
  a.part_m = cache->part_m;
  a.part_l = cache->part_l;
  a.part_acc = cache->part_acc;
  a.L = L; a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.W = d.window;
  a.n_global = (int32_t)cache->glob_ids.size();
  a.n_swa = (int32_t)cache->swa_ids.size();
  a.max_chunks = cache->max_chunks;
  a.rot_pairs = R / 2;
  a.eps = eps;
  a.q_scale = (float)(1.4426950408889634 / std::sqrt((double)kHeadDim));
  fill_inv_freq(a.inv_freq_rev, R / 2, R, base);
  for (int b = 0; b < B; b++) a.pos[b] = positions[b];
  const int32_t chunks = (int32_t)((pmax + 1 + kDecodeChunk - 1) / kDecodeChunk);

  hipError_t e;
  {
    ScopedTimer tm("decode_append", st);
    e = launch_decode_append(a, st);
  }
  if (e != hipSuccess) return hip_fail(e, "decode append launch");
  {
    ScopedTimer tm("decode_swa", st);
    e = launch_decode_swa(a, st);
  }
  if (e != hipSuccess) return hip_fail(e, "decode SWA launch");
  if (a.n_global) {
    {
      ScopedTimer tm("decode_global", st);
      e = launch_decode_global(a, chunks, st);
    }
    if (e != hipSuccess) return hip_fail(e, "decode global launch");
    {
      ScopedTimer tm("decode_merge", st);
      e = launch_decode_merge(a, st);
    }
    if (e != hipSuccess) return hip_fail(e, "decode merge launch");
  }
  for (int l = 0; l < L; l++)
    for (int b = 0; b < B; b++) cache->length[(size_t)l * B + b] = positions[b] + 1;
  return ZG_OK;
}

extern "C" const char* zg_last_error(void) { return g_err.c_str(); }

extern "C" int zg_kernel_timer_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  for (auto& t : g_timer_log) g_timer_pool.push_back({t.start, t.stop});
  g_timer_log.clear();
  g_timer_on = on != 0;
  return ZG_OK;
}

extern "C" int zg_kernel_timer_only(const char* name) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  g_timer_only = name ? name : "";
  return ZG_OK;
}

extern "C" int zg_kernel_timer_read(const char* name, double* total_ms, int64_t* launches) {
  if (!name || !total_ms || !launches) return fail(ZG_EINVAL, "zg_kernel_timer_read: null argument");
  std::lock_guard<std::mutex> lk(g_timer_mu);
  double sum = 0.0;
  int64_t n = 0;
  for (auto& t : g_timer_log) {
    if (t.name != name) continue;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e != hipSuccess) return hip_fail(e, "zg_kernel_timer_read");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess) return hip_fail(e, "zg_kernel_timer_read");
    sum += ms;
    n++;
  }
  *total_ms = sum;
  *launches = n;
  return ZG_OK;
}
