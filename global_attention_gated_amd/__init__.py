"""Python binding of libzgattn.so: the MI355X (gfx950) attention core of the ZGCM-1 hybrid backbone.

Argument marshalling only: every step runs in the library's HIP kernels.  Tensors are torch CUDA
(ROCm) tensors of dtype bfloat16, contiguous; work is enqueued on torch's current stream.  The library
must have been built (``python -m global_attention_gated_amd.build``); importing this module raises if
it is missing.

Entry points (C ABI in include/zgattn.h):
  swa_prefill        gated sliding-window layer prefill   (A_SWA(q,k,v) (.) sigmoid(gate))
  global_prefill     ungated global causal layer prefill
  hybrid_decode_step one new token per sequence through every layer of a KVCache
  KVCache            kv_cache_alloc / kv_cache_free / footprint / layer views / lengths
  linear_bf16        y = x W^T on hipBLASLt (the projections around the core)
  gated_swa_layer    q/k/v/g projections + swa_prefill + o_proj, from the hidden state
  global_layer       q/k/v projections + global_prefill + o_proj
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ZGATTN_LIB selects another build of the same library (for A/B timing of kernel variants)
LIB_PATH = os.environ.get("ZGATTN_LIB") or os.path.join(_HERE, "libzgattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m global_attention_gated_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

ZG_OK, ZG_EINVAL, ZG_EUNSUPPORTED, ZG_ERANGE, ZG_ENOMEM, ZG_EHIP = range(6)
_STATUS = {1: "EINVAL", 2: "EUNSUPPORTED", 3: "ERANGE", 4: "ENOMEM", 5: "EHIP"}

_vp, _i32, _i64, _u64, _f32, _f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_double


class CacheDesc(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("global_layers", ctypes.POINTER(_i32)), ("n_global", _i32),
                ("batch", _i32), ("n_kv_heads", _i32), ("head_dim", _i32), ("window", _i32),
                ("max_tokens", _i64)]


_lib.kv_cache_alloc.argtypes = [ctypes.POINTER(CacheDesc), ctypes.POINTER(_vp), ctypes.POINTER(_u64)]
_lib.kv_cache_free.argtypes = [_vp]
_lib.kv_cache_footprint_bytes.argtypes = [ctypes.POINTER(CacheDesc), _i64]
_lib.kv_cache_footprint_bytes.restype = _u64
_lib.kv_cache_layer_view.argtypes = [_vp, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_i64)]
_lib.kv_cache_length.argtypes = [_vp, _i32, _i32, ctypes.POINTER(_i64)]
_lib.kv_cache_set_length.argtypes = [_vp, _i32, _i32, _i64]
_lib.prefill_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
_lib.prefill_workspace_bytes.restype = _u64
_lib.prefill_workspace_bytes_at.argtypes = [_i32, _i32, _i32, _i32, _i64, _i32]
_lib.prefill_workspace_bytes_at.restype = _u64
_lib.swa_prefill.argtypes = [_vp] * 7 + [_i32] * 7 + [_f64, _f32, _i64, _vp, _i32, _vp, _u64, _vp]
_lib.global_prefill.argtypes = [_vp] * 6 + [_i32] * 6 + [_f64, _f32, _i64, _vp, _i32, _vp, _u64, _vp]
_lib.global_prefill_noalloc.argtypes = [_vp] * 6 + [_i32] * 6 + [_f64, _f32, _i64, _vp, _i32, _vp]
_lib.global_prefill_noalloc_max_bytes.restype = _u64
_lib.hybrid_decode_step.argtypes = [_vp] * 7 + [ctypes.POINTER(_i64), _i32, _i32, _f64, _f32, _vp, _vp]
_lib.linear_bf16.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _vp]
_lib.layer_workspace_bytes.argtypes = [_i32] * 5
_lib.layer_workspace_bytes.restype = _u64
_lib.gated_swa_layer.argtypes = [_vp] * 9 + [_i32] * 8 + [_f64, _f32, _i64, _vp, _i32, _vp, _u64, _vp]
_lib.global_layer.argtypes = [_vp] * 8 + [_i32] * 7 + [_f64, _f32, _i64, _vp, _i32, _vp, _u64, _vp]
_lib.fp8_linear_alloc.argtypes = [_i32, _i32, _i32, ctypes.POINTER(_vp)]
_lib.fp8_linear_free.argtypes = [_vp]
_lib.fp8_linear_scales.argtypes = [_vp, ctypes.POINTER(_f32)]
_lib.fp8_linear_workspace_bytes.argtypes = [_i64, _i32, _i32]
_lib.fp8_linear_workspace_bytes.restype = _u64
_lib.linear_fp8_delayed.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _u64, _vp]
_lib.fp8_layer_alloc.argtypes = [_i32] * 5 + [ctypes.POINTER(_vp)]
_lib.fp8_layer_free.argtypes = [_vp]
_lib.fp8_layer_scales.argtypes = [_vp, ctypes.POINTER(_f32)]
_lib.fp8_layer_workspace_bytes.argtypes = [_i32] * 6
_lib.fp8_layer_workspace_bytes.restype = _u64
_lib.gated_swa_layer_fp8.argtypes = [_vp] * 9 + [_i32] * 8 + [_f64, _f32, _i64, _vp, _i32, _vp, _vp, _u64, _vp]
_lib.global_layer_fp8.argtypes = [_vp] * 8 + [_i32] * 7 + [_f64, _f32, _i64, _vp, _i32, _vp, _vp, _u64, _vp]
_fp = ctypes.POINTER(ctypes.c_float)
_lib.swa_prefill_train.argtypes = [_vp] * 8 + [_i32] * 7 + [_f64, _f32, _vp, _u64, _vp]
_lib.global_prefill_train.argtypes = [_vp] * 7 + [_i32] * 6 + [_f64, _f32, _vp, _u64, _vp]
_lib.backward_workspace_bytes.argtypes = [_i32] * 5
_lib.backward_workspace_bytes.restype = _u64
_lib.swa_prefill_backward.argtypes = [_vp] * 15 + [_i32] * 7 + [_f64, _f32, _vp, _u64, _vp]
_lib.global_prefill_backward.argtypes = [_vp] * 13 + [_i32] * 6 + [_f64, _f32, _vp, _u64, _vp]
_lib.zg_last_error.restype = ctypes.c_char_p
_lib.zg_kernel_timer_enable.argtypes = [_i32]
_lib.zg_kernel_timer_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(_f64), ctypes.POINTER(_i64)]
_lib.zg_kernel_timer_only.argtypes = [ctypes.c_char_p]

EXPORTED = ["kv_cache_alloc", "kv_cache_free", "kv_cache_footprint_bytes", "kv_cache_layer_view", "kv_cache_length",
            "kv_cache_set_length", "prefill_workspace_bytes", "prefill_workspace_bytes_at", "swa_prefill", "global_prefill", "global_prefill_noalloc",
            "global_prefill_noalloc_max_bytes", "hybrid_decode_step",
            "linear_bf16", "layer_workspace_bytes", "gated_swa_layer", "global_layer", "fp8_linear_alloc",
            "fp8_linear_free", "fp8_linear_scales", "fp8_linear_workspace_bytes", "linear_fp8_delayed",
            "fp8_layer_alloc", "fp8_layer_free", "fp8_layer_scales", "fp8_layer_workspace_bytes", "gated_swa_layer_fp8",
            "global_layer_fp8", "swa_prefill_train", "global_prefill_train", "backward_workspace_bytes",
            "swa_prefill_backward", "global_prefill_backward", "zg_last_error", "zg_kernel_timer_enable",
            "zg_kernel_timer_read", "zg_kernel_timer_only"]


class ZgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(rc: int):
    if rc != ZG_OK:
        raise ZgError(rc, _lib.zg_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _bf16(t, name):
    if t is None:
        return None
    if not (t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous bfloat16 CUDA tensor")
    return t


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _shapes(fn, want, device=None):
    """Check every tensor of ``want`` ({name: (tensor or None, expected shape tuple)}) against its expected shape
    and, when ``device`` is given, that it lives on that device, before anything reaches the library (whose kernels
    index raw pointers with the sizes taken from q or the cache).  Raises ValueError naming the first mismatch."""
    for name, (t, shape) in want.items():
        if t is None:
            continue
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if device is not None and t.device != device:
            raise ValueError(f"{fn}: {name} is on {t.device}, expected {device}")


# ------------------------------------------------------------------------------------------- cache
def _desc(n_layers, global_layers, batch, n_kv_heads, head_dim, window, max_tokens):
    gl = (_i32 * max(1, len(global_layers)))(*global_layers)
    d = CacheDesc(n_layers, gl, len(global_layers), batch, n_kv_heads, head_dim, window, max_tokens)
    d._keep = gl
    return d


def footprint_bytes(tokens, *, n_layers=32, global_layers=(6, 12, 18, 24, 30), batch=1, n_kv_heads=8, head_dim=128,
                    window=128) -> int:
    """kv_cache_footprint_bytes: the cache bytes ``tokens`` positions of every sequence take."""
    d = _desc(n_layers, list(global_layers), batch, n_kv_heads, head_dim, window, max(1, tokens))
    return int(_lib.kv_cache_footprint_bytes(ctypes.byref(d), tokens))


class KVCache:
    """Library-owned KV cache (kv_cache_alloc / kv_cache_free)."""

    def __init__(self, *, n_layers=32, global_layers=(6, 12, 18, 24, 30), batch=1, n_kv_heads=8, head_dim=128,
                 window=128, max_tokens):
        self.n_layers, self.global_layers = n_layers, list(global_layers)
        self.batch, self.n_kv_heads, self.head_dim, self.window, self.max_tokens = batch, n_kv_heads, head_dim, window, max_tokens
        self._desc = _desc(n_layers, self.global_layers, batch, n_kv_heads, head_dim, window, max_tokens)
        h = _vp()
        nbytes = _u64()
        _check(_lib.kv_cache_alloc(ctypes.byref(self._desc), ctypes.byref(h), ctypes.byref(nbytes)))
        self.handle = h.value
        self.device_bytes = int(nbytes.value)

    def close(self):
        if getattr(self, "handle", None):
            _check(_lib.kv_cache_free(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def layer_view(self, layer: int):
        """(k device pointer, v device pointer, slots) of a 1-based layer."""
        k, v, s = _vp(), _vp(), _i64()
        _check(_lib.kv_cache_layer_view(self.handle, layer, ctypes.byref(k), ctypes.byref(v), ctypes.byref(s)))
        return k.value, v.value, int(s.value)

    def length(self, layer: int, b: int) -> int:
        n = _i64()
        _check(_lib.kv_cache_length(self.handle, layer, b, ctypes.byref(n)))
        return int(n.value)

    def set_length(self, layer: int, b: int, n: int):
        _check(_lib.kv_cache_set_length(self.handle, layer, b, n))

    def read_layer(self, layer: int):
        """Copy a layer's K and V arrays to the host: two torch uint16-as-int16 CPU tensors
        [B][Hkv][slots][D] (bf16 bits)."""
        k, v, slots = self.layer_view(layer)
        shape = (self.batch, self.n_kv_heads, slots, self.head_dim)
        out = []
        for p in (k, v):
            t = torch.empty(shape, dtype=torch.int16)
            _hip_memcpy_d2h(t.data_ptr(), p, t.numel() * 2)
            out.append(t)
        return out


_hip = None


def _hip_memcpy_d2h(dst, src, n):
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [_vp, _vp, ctypes.c_size_t, ctypes.c_int]
    torch.cuda.synchronize()
    rc = _hip.hipMemcpy(dst, src, n, 2)
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed with {rc}")


# ------------------------------------------------------------------------------------------- prefill
def workspace_bytes(B, S, Hkv, D=128, *, pos0=0, window=0) -> int:
    """prefill_workspace_bytes_at: the workspace a prefill of S tokens at pos0 needs (window 0: a global layer)."""
    return int(_lib.prefill_workspace_bytes_at(B, S, Hkv, D, pos0, window))


def _qkv_shapes(fn, q, k, v, gate, q_norm_w, k_norm_w, out):
    """(B, S, Hq, Hkv, D) from q and k, after checking every tensor of a layer call against them."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError(f"{fn}: q and k must be [B, S, H, D]")
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    _shapes(fn, {"k": (k, (B, S, Hkv, D)), "v": (v, (B, S, Hkv, D)), "gate": (gate, (B, S, Hq, D)),
                 "q_norm_w": (q_norm_w, (D,)), "k_norm_w": (k_norm_w, (D,)), "out": (out, (B, S, Hq, D))}, q.device)
    return B, S, Hq, Hkv, D


def _prefill(gated, q, k, v, gate, q_norm_w, k_norm_w, out, window, rotary_dims, rope_base, eps, pos0, cache, layer,
             workspace):
    fn = "swa_prefill" if gated else "global_prefill"
    if gated and gate is None:
        raise ValueError(f"{fn}: gate is required")
    B, S, Hq, Hkv, D = _qkv_shapes(fn, q, k, v, gate, q_norm_w, k_norm_w, out)
    _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _bf16(gate, "gate"), _bf16(q_norm_w, "q_norm_w"), _bf16(k_norm_w, "k_norm_w")
    if out is None:
        out = torch.empty_like(q)
    _bf16(out, "out")
    if workspace is None:
        need = workspace_bytes(B, S, Hkv, D, pos0=pos0 if cache is not None else 0, window=window if gated else 0)
        workspace = torch.empty(max(16, need), dtype=torch.uint8, device=q.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ch = None if cache is None else cache.handle
    if gated:
        rc = _lib.swa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out),
                              B, S, Hq, Hkv, D, window, rotary_dims, rope_base, eps, pos0, ch, layer, ws_ptr, ws_n,
                              _stream())
    else:
        rc = _lib.global_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out),
                                 B, S, Hq, Hkv, D, rotary_dims, rope_base, eps, pos0, ch, layer, ws_ptr, ws_n,
                                 _stream())
    _check(rc)
    return out


def swa_prefill(q, k, v, gate, q_norm_w, k_norm_w, out=None, *, window=128, rotary_dims=42, rope_base=1e4, eps=1e-6,
                pos0=0, cache: KVCache | None = None, layer=0, workspace=None):
    """Gated sliding-window layer: q/gate [B,S,Hq,D], k/v [B,S,Hkv,D], weights [D] (bf16); returns out."""
    return _prefill(True, q, k, v, gate, q_norm_w, k_norm_w, out, window, rotary_dims, rope_base, eps, pos0, cache,
                    layer, workspace)


def global_prefill(q, k, v, q_norm_w, k_norm_w, out=None, *, rotary_dims=42, rope_base=1e4, eps=1e-6, pos0=0,
                   cache: KVCache | None = None, layer=0, workspace=None):
    """Ungated global causal layer: q [B,S,Hq,D], k/v [B,S,Hkv,D], weights [D] (bf16); returns out."""
    return _prefill(False, q, k, v, None, q_norm_w, k_norm_w, out, 0, rotary_dims, rope_base, eps, pos0, cache,
                    layer, workspace)


def global_prefill_noalloc(q, k, v, q_norm_w, k_norm_w, out, *, rotary_dims=42, rope_base=1e4, eps=1e-6, pos0=0,
                           cache: KVCache | None = None, layer=0):
    """global_prefill staging its keys in the library's per-GPU scratch array (no workspace, no allocation): out must
    be given.  At most global_prefill_noalloc_max_bytes() of staged keys."""
    fn = "global_prefill_noalloc"
    if out is None:
        raise ValueError(f"{fn}: out is required (the call allocates nothing)")
    B, S, Hq, Hkv, D = _qkv_shapes(fn, q, k, v, None, q_norm_w, k_norm_w, out)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w"), (out, "out")):
        _bf16(t, n)
    ch = None if cache is None else cache.handle
    _check(_lib.global_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out), B, S, Hq,
                                       Hkv, D, rotary_dims, rope_base, eps, pos0, ch, layer, _stream()))
    return out


# ------------------------------------------------------------------------------------------- training
def _f32cuda(t, name):
    if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous float32 CUDA tensor")
    return t


def prefill_train(q, k, v, gate, q_norm_w, k_norm_w, *, window=128, rotary_dims=42, rope_base=1e4, eps=1e-6,
                  out=None, lse=None, workspace=None):
    """Training forward (swa_prefill_train, or global_prefill_train when gate is None): returns (out, lse), out
    [B,S,Hq,D] bf16 and lse [B,Hq,S] fp32 (natural log of each softmax denominator)."""
    fn = "swa_prefill_train" if gate is not None else "global_prefill_train"
    B, S, Hq, Hkv, D = _qkv_shapes(fn, q, k, v, gate, q_norm_w, k_norm_w, out)
    _shapes(fn, {"lse": (lse, (B, Hq, S))}, q.device)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        _bf16(t, n)
    out = torch.empty_like(q) if out is None else _bf16(out, "out")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if lse is None else _f32cuda(lse, "lse")
    if workspace is None:
        workspace = torch.empty(max(16, workspace_bytes(B, S, Hkv, D)), dtype=torch.uint8, device=q.device)
    ws_n = workspace.numel() * workspace.element_size()
    if gate is not None:
        rc = _lib.swa_prefill_train(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out),
                                    _ptr(lse), B, S, Hq, Hkv, D, window, rotary_dims, rope_base, eps,
                                    workspace.data_ptr(), ws_n, _stream())
    else:
        rc = _lib.global_prefill_train(_ptr(q), _ptr(k), _ptr(v), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out), _ptr(lse),
                                       B, S, Hq, Hkv, D, rotary_dims, rope_base, eps, workspace.data_ptr(), ws_n,
                                       _stream())
    _check(rc)
    return out, lse


def backward_workspace_bytes(B, S, Hq, Hkv, D=128) -> int:
    return int(_lib.backward_workspace_bytes(B, S, Hq, Hkv, D))


def prefill_backward(q, k, v, gate, q_norm_w, k_norm_w, out, lse, dout, *, window=128, rotary_dims=42, rope_base=1e4,
                     eps=1e-6, grads=None, workspace=None):
    """Backward (swa_prefill_backward, or global_prefill_backward when gate is None): returns a dict with dq, dk,
    dv (bf16, shaped as q/k/v), dgate (bf16, None for a global layer) and dq_norm_w, dk_norm_w ([D] fp32)."""
    fn = "swa_prefill_backward" if gate is not None else "global_prefill_backward"
    B, S, Hq, Hkv, D = _qkv_shapes(fn, q, k, v, gate, q_norm_w, k_norm_w, out)
    g = grads or {}
    _shapes(fn, {"lse": (lse, (B, Hq, S)), "dout": (dout, (B, S, Hq, D)), "dq": (g.get("dq"), (B, S, Hq, D)),
                 "dk": (g.get("dk"), (B, S, Hkv, D)), "dv": (g.get("dv"), (B, S, Hkv, D)),
                 "dgate": (g.get("dgate") if gate is not None else None, (B, S, Hq, D)),
                 "dq_norm_w": (g.get("dq_norm_w"), (D,)), "dk_norm_w": (g.get("dk_norm_w"), (D,))}, q.device)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w"),
                 (out, "out"), (dout, "dout")):
        _bf16(t, n)
    _f32cuda(lse, "lse")
    for n in ("dq", "dk", "dv", "dgate"):
        if g.get(n) is not None:
            _bf16(g[n], n)
    for n in ("dq_norm_w", "dk_norm_w"):
        if g.get(n) is not None:
            _f32cuda(g[n], n)
    dq = g.get("dq", torch.empty_like(q))
    dk = g.get("dk", torch.empty_like(k))
    dv = g.get("dv", torch.empty_like(v))
    dg = None if gate is None else g.get("dgate", torch.empty_like(gate))
    dqw = g.get("dq_norm_w", torch.empty(D, dtype=torch.float32, device=q.device))
    dkw = g.get("dk_norm_w", torch.empty(D, dtype=torch.float32, device=q.device))
    if workspace is None:
        workspace = torch.empty(max(16, backward_workspace_bytes(B, S, Hq, Hkv, D)), dtype=torch.uint8, device=q.device)
    ws_n = workspace.numel() * workspace.element_size()
    if gate is not None:
        rc = _lib.swa_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out),
                                       _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dqw),
                                       _ptr(dkw), B, S, Hq, Hkv, D, window, rotary_dims, rope_base, eps,
                                       workspace.data_ptr(), ws_n, _stream())
    else:
        rc = _lib.global_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out),
                                          _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dqw), _ptr(dkw),
                                          B, S, Hq, Hkv, D, rotary_dims, rope_base, eps, workspace.data_ptr(), ws_n,
                                          _stream())
    _check(rc)
    return {"dq": dq, "dk": dk, "dv": dv, "dgate": dg, "dq_norm_w": dqw, "dk_norm_w": dkw}


# ------------------------------------------------------------------------------------------- projections, layers
def linear_bf16(x, w, y=None):
    """y = x W^T: x [..., K], w [N, K] (bf16); returns y [..., N]."""
    if w.dim() != 2:
        raise ValueError("linear_bf16: w must be [N, K]")
    N, K = w.shape
    if x.dim() < 1 or x.shape[-1] != K:
        raise ValueError(f"linear_bf16: x has {tuple(x.shape)[-1:]} features, w expects {K}")
    _shapes("linear_bf16", {"w": (w, (N, K)), "y": (y, (*x.shape[:-1], N))}, x.device)
    _bf16(x, "x"), _bf16(w, "w")
    T = x.numel() // K
    if y is None:
        y = torch.empty((*x.shape[:-1], N), dtype=torch.bfloat16, device=x.device)
    _bf16(y, "y")
    _check(_lib.linear_bf16(_ptr(x), _ptr(w), _ptr(y), T, K, N, _stream()))
    return y


class Fp8Linear:
    """y = x W^T with E4M3 operands under delayed scaling (fp8_linear_alloc / linear_fp8_delayed): the state holds
    each operand's amax history and current scale.  After a call, ``workspace`` holds the operands' E4M3 codes."""

    def __init__(self, K: int, N: int, history: int = 1024):
        h = _vp()
        _check(_lib.fp8_linear_alloc(K, N, history, ctypes.byref(h)))
        self.handle, self.K, self.N, self.history = h, K, N, history
        self.workspace = None

    def scales(self):
        """(s_x, s_w): the scales the next call will use."""
        out = (_f32 * 2)()
        _check(_lib.fp8_linear_scales(self.handle, out))
        return float(out[0]), float(out[1])

    def __call__(self, x, w, y=None):
        if x.dim() < 1 or x.shape[-1] != self.K:
            raise ValueError(f"linear_fp8_delayed: x has {tuple(x.shape)[-1:]} features, the state expects {self.K}")
        _shapes("linear_fp8_delayed", {"w": (w, (self.N, self.K)), "y": (y, (*x.shape[:-1], self.N))}, x.device)
        _bf16(x, "x"), _bf16(w, "w")
        T = x.numel() // self.K
        if y is None:
            y = torch.empty((*x.shape[:-1], self.N), dtype=torch.bfloat16, device=x.device)
        _bf16(y, "y")
        need = int(_lib.fp8_linear_workspace_bytes(T, self.K, self.N))
        if self.workspace is None or self.workspace.numel() < need:
            self.workspace = torch.empty(max(16, need), dtype=torch.uint8, device=x.device)
        _check(_lib.linear_fp8_delayed(_ptr(x), _ptr(w), _ptr(y), T, self.K, self.N, self.handle,
                                       self.workspace.data_ptr(), self.workspace.numel(), _stream()))
        return y

    def codes(self, T: int):
        """The E4M3 codes of the last call's x [T][K] and W [N][K] (uint8 CPU tensors)."""
        off = (T * self.K + 255) // 256 * 256
        ws = self.workspace.cpu()
        return ws[:T * self.K].reshape(T, self.K), ws[off:off + self.N * self.K].reshape(self.N, self.K)

    def close(self):
        if self.handle:
            _lib.fp8_linear_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def layer_workspace_bytes(B, S, Hq, Hkv, D=128) -> int:
    return int(_lib.layer_workspace_bytes(B, S, Hq, Hkv, D))


class Fp8Layer:
    """Delayed-scaling state of one attention layer with FP8 projections (fp8_layer_alloc): tensors h, W_q, W_k,
    W_v, W_g, o, W_o, each with its own amax history and scale.  Pass it as ``fp8=`` to gated_swa_layer_fp8 /
    global_layer_fp8."""

    TENSORS = ("h", "w_q", "w_k", "w_v", "w_g", "o", "w_o")

    def __init__(self, d_model: int, Hq: int = 32, Hkv: int = 8, D: int = 128, history: int = 1024):
        h = _vp()
        _check(_lib.fp8_layer_alloc(d_model, Hq, Hkv, D, history, ctypes.byref(h)))
        self.handle, self.d_model, self.Hq, self.Hkv, self.D, self.history = h, d_model, Hq, Hkv, D, history

    def scales(self):
        """The seven scales the next call will use, in the order of TENSORS."""
        out = (_f32 * 7)()
        _check(_lib.fp8_layer_scales(self.handle, out))
        return tuple(float(x) for x in out)

    def close(self):
        if self.handle:
            _lib.fp8_layer_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fp8_layer_workspace_bytes(B, S, d_model, Hq, Hkv, D=128) -> int:
    return int(_lib.fp8_layer_workspace_bytes(B, S, d_model, Hq, Hkv, D))


def _layer(gated, h, w_q, w_k, w_v, w_g, w_o, q_norm_w, k_norm_w, y, Hq, Hkv, window, rotary_dims, rope_base, eps,
           pos0, cache, layer, workspace, fp8=None):
    fn = ("gated_swa_layer" if gated else "global_layer") + ("_fp8" if fp8 is not None else "")
    if h.dim() != 3 or q_norm_w.dim() != 1:
        raise ValueError(f"{fn}: h must be [B, S, d_model] and q_norm_w [D]")
    B, S, d_model = h.shape
    D = q_norm_w.shape[0]
    if gated and w_g is None:
        raise ValueError(f"{fn}: w_g is required")
    _shapes(fn, {"w_q": (w_q, (Hq * D, d_model)), "w_k": (w_k, (Hkv * D, d_model)), "w_v": (w_v, (Hkv * D, d_model)),
                 "w_g": (w_g, (Hq * D, d_model)), "w_o": (w_o, (d_model, Hq * D)), "k_norm_w": (k_norm_w, (D,)),
                 "y": (y, (B, S, d_model))}, h.device)
    for t, n in ((h, "h"), (w_q, "w_q"), (w_k, "w_k"), (w_v, "w_v"), (w_g, "w_g"), (w_o, "w_o"), (q_norm_w, "q_norm_w"),
                 (k_norm_w, "k_norm_w")):
        _bf16(t, n)
    if y is None:
        y = torch.empty_like(h)
    _bf16(y, "y")
    if workspace is None:
        need = (layer_workspace_bytes(B, S, Hq, Hkv, D) if fp8 is None
                else fp8_layer_workspace_bytes(B, S, d_model, Hq, Hkv, D))
        if cache is not None:   # the attention's part (the tail) also stages the cached positions
            need += workspace_bytes(B, S, Hkv, D, pos0=pos0, window=window if gated else 0) - workspace_bytes(B, S, Hkv, D)
        workspace = torch.empty(max(16, need), dtype=torch.uint8, device=h.device)
    ws_n = workspace.numel() * workspace.element_size()
    ch = None if cache is None else cache.handle
    common = (B, S, d_model, Hq, Hkv, D)
    if gated:
        args = (_ptr(h), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_g), _ptr(w_o), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(y),
                *common, window, rotary_dims, rope_base, eps, pos0, ch, layer)
    else:
        args = (_ptr(h), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(y),
                *common, rotary_dims, rope_base, eps, pos0, ch, layer)
    tail = (workspace.data_ptr(), ws_n, _stream())
    if fp8 is None:
        rc = (_lib.gated_swa_layer if gated else _lib.global_layer)(*args, *tail)
    else:
        rc = (_lib.gated_swa_layer_fp8 if gated else _lib.global_layer_fp8)(*args, fp8.handle, *tail)
    _check(rc)
    return y


def gated_swa_layer(h, w_q, w_k, w_v, w_g, w_o, q_norm_w, k_norm_w, y=None, *, Hq=32, Hkv=8, window=128, rotary_dims=42,
                    rope_base=1e4, eps=1e-6, pos0=0, cache: KVCache | None = None, layer=0, workspace=None):
    """o_proj(A_SWA(q, k, v) (.) sigmoid(g)) with q/k/v/g = h W^T: h [B,S,d_model], W_q/W_g [Hq*D, d_model],
    W_k/W_v [Hkv*D, d_model], W_o [d_model, Hq*D] (bf16); returns y [B,S,d_model]."""
    return _layer(True, h, w_q, w_k, w_v, w_g, w_o, q_norm_w, k_norm_w, y, Hq, Hkv, window, rotary_dims, rope_base, eps,
                  pos0, cache, layer, workspace)


def global_layer(h, w_q, w_k, w_v, w_o, q_norm_w, k_norm_w, y=None, *, Hq=32, Hkv=8, rotary_dims=42, rope_base=1e4,
                 eps=1e-6, pos0=0, cache: KVCache | None = None, layer=0, workspace=None):
    """o_proj(global causal attention of q, k, v) with q/k/v = h W^T; shapes as gated_swa_layer."""
    return _layer(False, h, w_q, w_k, w_v, None, w_o, q_norm_w, k_norm_w, y, Hq, Hkv, 0, rotary_dims, rope_base, eps,
                  pos0, cache, layer, workspace)


def gated_swa_layer_fp8(h, w_q, w_k, w_v, w_g, w_o, q_norm_w, k_norm_w, y=None, *, fp8: Fp8Layer, Hq=32, Hkv=8,
                        window=128, rotary_dims=42, rope_base=1e4, eps=1e-6, pos0=0, cache: KVCache | None = None,
                        layer=0, workspace=None):
    """gated_swa_layer with every projection on E4M3 operands under the delayed-scaling state ``fp8``."""
    return _layer(True, h, w_q, w_k, w_v, w_g, w_o, q_norm_w, k_norm_w, y, Hq, Hkv, window, rotary_dims, rope_base, eps,
                  pos0, cache, layer, workspace, fp8=fp8)


def global_layer_fp8(h, w_q, w_k, w_v, w_o, q_norm_w, k_norm_w, y=None, *, fp8: Fp8Layer, Hq=32, Hkv=8, rotary_dims=42,
                     rope_base=1e4, eps=1e-6, pos0=0, cache: KVCache | None = None, layer=0, workspace=None):
    """global_layer with every projection on E4M3 operands under the delayed-scaling state ``fp8``."""
    return _layer(False, h, w_q, w_k, w_v, None, w_o, q_norm_w, k_norm_w, y, Hq, Hkv, 0, rotary_dims, rope_base, eps,
                  pos0, cache, layer, workspace, fp8=fp8)


# ------------------------------------------------------------------------------------------- decode
def hybrid_decode_step(q, k, v, gate, q_norm_w, k_norm_w, positions, cache: KVCache, out=None, *, rotary_dims=42,
                       rope_base=1e7, eps=1e-6):
    """q/gate [L,B,Hq,D], k/v [L,B,Hkv,D], weights [L,D] (bf16), positions: B ints; returns out [L,B,Hq,D]."""
    fn = "hybrid_decode_step"
    if q.dim() != 4:
        raise ValueError(f"{fn}: q must be [L, B, Hq, D]")
    L, B, Hq, D = q.shape
    if (L, B, D) != (cache.n_layers, cache.batch, cache.head_dim):
        raise ValueError(f"{fn}: q has shape {tuple(q.shape)}, the cache needs [{cache.n_layers}, {cache.batch}, Hq, "
                         f"{cache.head_dim}]")
    Hkv = cache.n_kv_heads
    _shapes(fn, {"k": (k, (L, B, Hkv, D)), "v": (v, (L, B, Hkv, D)), "gate": (gate, (L, B, Hq, D)),
                 "q_norm_w": (q_norm_w, (L, D)), "k_norm_w": (k_norm_w, (L, D)), "out": (out, (L, B, Hq, D))},
            q.device)
    positions = [int(p) for p in positions]
    if len(positions) != B:
        raise ValueError(f"{fn}: {len(positions)} positions for a batch of {B}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        _bf16(t, n)
    if out is None:
        out = torch.empty_like(q)
    _bf16(out, "out")
    pos = (_i64 * B)(*positions)
    _check(_lib.hybrid_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out),
                                   pos, Hq, rotary_dims, rope_base, eps, cache.handle, _stream()))
    return out


# ------------------------------------------------------------------------------------------- timer
def kernel_timer_enable(on: bool = True, only: str = None):
    """Enable (and reset) or disable the kernel timer; `only` restricts it to one kernel family."""
    _check(_lib.zg_kernel_timer_only((only or "").encode()))
    _check(_lib.zg_kernel_timer_enable(1 if on else 0))


def kernel_timer_read(name: str):
    """(total ms, launches) of a kernel family since the timer was enabled."""
    ms, n = _f64(), _i64()
    _check(_lib.zg_kernel_timer_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)
