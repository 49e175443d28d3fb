"""Plain fp64 CPU oracle of the ZGCM-1 hybrid attention core (gated SWA + global causal).

TEST INFRASTRUCTURE ONLY: only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``global_attention_gated_amd``) and never imports it; the only module both sides use is ``synth``,
the seeded input generator, which holds none of the method's arithmetic.

The arithmetic lives in ``zg_oracle.c`` (plain loops in float64, compiled with gcc); this module
decodes bf16 inputs, orders the steps and keeps the oracle's own KV cache.

Steps and where the pages define them (ZGCM-1 paper summaries on onedev.kr, "How it works", and
jaehun.me, "New Approach" and "How Gated SWA Behaves"):
  1. RMSNorm of each (token, head) row of q and k with a per-layer weight vector     -- QK-norm
  2. partial RoPE on the leading R dims (fraction 0.33 -> R = 42 of 128)               -- Partial RoPE
  3. visible keys: causal; gated-SWA layers also require q_pos - k_pos < W (W = 128)  -- window
  4. softmax(q.k / sqrt(D)) . v                                                        -- A_SWA / global
  5. gated-SWA layers multiply the output element-wise by sigmoid(g)                   -- gate
  6. the KV cache holds the post-norm, post-RoPE key and the raw value, in bf16 (jaehun.me, "Why the KV
     Cache Shrinks by 6.4x": 2 bytes per element since it is bf16); SWA layers keep only the last W
     positions (slot = position mod W), global layers keep every position             -- KV cache
     Keys enter attention in that stored form, k_hat rounded once to bf16 (nearest-even), in prefill as
     in decode; q_hat, the scores, the softmax and the output stay in float64.
Layer schedule: 32 layers, global at 6, 12, 18, 24, 30 (1-indexed), the other 27 gated SWA.

Readings where the pages are silent: softmax scale 1/sqrt(D); one RMSNorm weight vector for q and one for k per
layer, shared by the heads, eps 1e-6; RMSNorm before RoPE; RoFormer's adjacent pairs (2i, 2i+1) rotated by
p * base^(-2i/R); query head h reads KV head h // (Hq / Hkv); the gate is element-wise.  Around the core (the
projections of ``attention_layer``) the layer's tensors are bf16 between operations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zg_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u16p = ctypes.POINTER(ctypes.c_uint16)


def build(force: bool = False) -> str:
    """Compile zg_oracle.c into liboracle.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.zo_rmsnorm.argtypes = [_dp, ctypes.c_int64, ctypes.c_int32, _dp, ctypes.c_double, _dp]
        lib.zo_rope.argtypes = [_dp, ctypes.c_int64, ctypes.c_int32, _i64p, ctypes.c_int32, ctypes.c_double]
        lib.zo_attend.argtypes = [ctypes.c_int64, ctypes.c_int32, _dp, _i64p, ctypes.c_int64, _dp, _dp, _i64p,
                                  ctypes.c_int64, _dp, _dp]
        lib.zo_decode_bf16.argtypes = [_u16p, ctypes.c_int64, _dp]
        lib.zo_round_bf16.argtypes = [_dp, ctypes.c_int64, _u16p]
        lib.zo_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a, t):
    return a.ctypes.data_as(t)


def num_threads() -> int:
    return int(_load().zo_num_threads())


# ---------------------------------------------------------------------------- formats
def bf16_to_f64(bits) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float64."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().zo_decode_bf16(_ptr(b, _u16p), b.size, _ptr(out, _dp))
    return out


def round_bf16(x) -> np.ndarray:
    """Round float64 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    a = _c(x, np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().zo_round_bf16(_ptr(a, _dp), a.size, _ptr(out, _u16p))
    return out


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    return bf16_to_f64(x) if x.dtype == np.uint16 else _c(x, np.float64)


# ---------------------------------------------------------------------------- steps 1-2
def rmsnorm(x, w, eps: float) -> np.ndarray:
    """Step 1: y = x * w / sqrt(mean(x^2) + eps) over the last axis (D)."""
    x = _as_f64(x)
    w = _as_f64(w)
    D = x.shape[-1]
    xf = _c(x.reshape(-1, D), np.float64)
    y = np.empty_like(xf)
    _load().zo_rmsnorm(_ptr(xf, _dp), xf.shape[0], D, _ptr(_c(w, np.float64), _dp), float(eps), _ptr(y, _dp))
    return y.reshape(x.shape)


def rope(x, pos, rotary_dims: int, base: float) -> np.ndarray:
    """Step 2: rotate pairs (2i, 2i+1), 2i+1 < rotary_dims, of each row by pos * base^(-2i/R).

    ``x`` has shape [..., D]; ``pos`` broadcasts against x.shape[:-1].
    """
    x = _as_f64(x)
    D = x.shape[-1]
    p = np.broadcast_to(np.asarray(pos, dtype=np.int64), x.shape[:-1])
    xf = _c(x.reshape(-1, D), np.float64).copy()
    pf = _c(p.reshape(-1), np.int64)
    _load().zo_rope(_ptr(xf, _dp), xf.shape[0], D, _ptr(pf, _i64p), int(rotary_dims), float(base))
    return xf.reshape(x.shape)


def qk_prologue(x, pos, w, eps: float, rotary_dims: int, base: float) -> np.ndarray:
    """Steps 1 then 2 on raw q or k rows (bf16 bits or float); returns float64."""
    return rope(rmsnorm(x, w, eps), pos, rotary_dims, base)


def cache_key(khat) -> np.ndarray:
    """Step 6: the stored (bf16, nearest-even) form of k_hat, as float64: what attention reads."""
    return bf16_to_f64(round_bf16(khat))


# ---------------------------------------------------------------------------- steps 3-5
def attend(qhat, qpos, khat, v, kpos, window: int | None, gate=None) -> np.ndarray:
    """Steps 3-5 for query rows qhat [nq, D] at positions qpos over keys khat/v [nk, D] at kpos.

    window None (or <= 0) = global causal; otherwise the sliding window W.  ``gate`` = logits [nq, D]
    (bf16 bits or float) for gated-SWA layers, None for global layers.
    """
    q = _c(_as_f64(qhat), np.float64)
    k = _c(_as_f64(khat), np.float64)
    vv = _c(_as_f64(v), np.float64)
    nq, D = q.shape
    nk = k.shape[0]
    qp = _c(np.broadcast_to(np.asarray(qpos, dtype=np.int64), (nq,)), np.int64)
    kp = _c(np.broadcast_to(np.asarray(kpos, dtype=np.int64), (nk,)), np.int64)
    g = None if gate is None else _c(_as_f64(gate).reshape(nq, D), np.float64)
    out = np.empty((nq, D), dtype=np.float64)
    _load().zo_attend(nq, D, _ptr(q, _dp), _ptr(qp, _i64p), nk, _ptr(k, _dp), _ptr(vv, _dp), _ptr(kp, _i64p),
                      0 if window is None else int(window), None if g is None else _ptr(g, _dp), _ptr(out, _dp))
    return out


# ---------------------------------------------------------------------------- schedule + footprint
def is_global_layer(layer_1based: int, n_layers: int = 32) -> bool:
    """5:1 hybrid: five blocks of (5 gated-SWA layers + 1 global layer), then 2 gated-SWA layers."""
    if not 1 <= layer_1based <= n_layers:
        raise ValueError("layer out of range")
    return layer_1based % 6 == 0 and layer_1based <= 30


def global_layers(n_layers: int = 32) -> list[int]:
    return [l for l in range(1, n_layers + 1) if is_global_layer(l, n_layers)]


def kv_footprint_bytes(tokens: int, *, n_layers: int = 32, global_layer_ids=None, batch: int = 1,
                       n_kv_heads: int = 8, head_dim: int = 128, window: int = 128, elem_bytes: int = 2) -> int:
    """KV-cache bytes for ``tokens`` positions per sequence: K and V per KV head per layer; global
    layers store every position, SWA layers at most ``window`` positions."""
    g = set(global_layers(n_layers) if global_layer_ids is None else global_layer_ids)
    per_pos = 2 * n_kv_heads * head_dim * elem_bytes
    total = 0
    for l in range(1, n_layers + 1):
        total += per_pos * (tokens if l in g else min(tokens, window))
    return total * batch


# ---------------------------------------------------------------------------- the oracle's KV cache
class OracleCache:
    """The oracle's KV cache: float64 history of (k_hat, v) per layer, sequence and KV head.

    It keeps every position (the visible set is decided by position in ``attend``); ``ring_image`` and
    ``global_image`` give the stored bf16 layout the method defines (SWA: slot = position mod W holding the
    last W positions; global: index = position)."""

    def __init__(self, n_layers: int, global_layer_ids, batch: int, n_kv_heads: int, head_dim: int, window: int):
        self.L, self.B, self.Hkv, self.D, self.W = n_layers, batch, n_kv_heads, head_dim, window
        self.glob = set(global_layer_ids)
        self.k = {l: [[np.zeros((0, head_dim)) for _ in range(n_kv_heads)] for _ in range(batch)]
                  for l in range(1, n_layers + 1)}
        self.v = {l: [[np.zeros((0, head_dim)) for _ in range(n_kv_heads)] for _ in range(batch)]
                  for l in range(1, n_layers + 1)}

    def length(self, layer: int, b: int) -> int:
        return self.k[layer][b][0].shape[0]

    def append(self, layer: int, b: int, khat, v):
        """Append positions length..length+n-1: khat, v of shape [n, Hkv, D]."""
        khat = _as_f64(khat)
        v = _as_f64(v)
        for h in range(self.Hkv):
            self.k[layer][b][h] = np.concatenate([self.k[layer][b][h], khat[:, h, :]], axis=0)
            self.v[layer][b][h] = np.concatenate([self.v[layer][b][h], v[:, h, :]], axis=0)

    def keys(self, layer: int, b: int, h: int):
        n = self.length(layer, b)
        return self.k[layer][b][h], self.v[layer][b][h], np.arange(n, dtype=np.int64)

    def ring_image(self, layer: int):
        """(K bits, V bits, slot positions) of an SWA layer's ring: [B][Hkv][W][D] bf16, [B][W] int64
        (position held by each slot, -1 if none)."""
        K = np.zeros((self.B, self.Hkv, self.W, self.D), dtype=np.uint16)
        V = np.zeros_like(K)
        P = np.full((self.B, self.W), -1, dtype=np.int64)
        for b in range(self.B):
            n = self.length(layer, b)
            for p in range(max(0, n - self.W), n):
                s = p % self.W
                P[b, s] = p
                for h in range(self.Hkv):
                    K[b, h, s] = round_bf16(self.k[layer][b][h][p])
                    V[b, h, s] = round_bf16(self.v[layer][b][h][p])
        return K, V, P

    def global_image(self, layer: int):
        """(K bits, V bits) of a global layer: [B][Hkv][T][D] bf16 with T = the cache length."""
        n = self.length(layer, 0)
        K = np.zeros((self.B, self.Hkv, n, self.D), dtype=np.uint16)
        V = np.zeros_like(K)
        for b in range(self.B):
            for h in range(self.Hkv):
                K[b, h] = round_bf16(self.k[layer][b][h])
                V[b, h] = round_bf16(self.v[layer][b][h])
        return K, V


# ---------------------------------------------------------------------------- whole-layer helpers
def prefill_layer(q, k, v, gate, wq, wk, *, window: int | None, rotary_dims: int, base: float, eps: float,
                  pos0: int = 0, cache: OracleCache | None = None, layer: int | None = None) -> np.ndarray:
    """One attention layer over a chunk of S new tokens at absolute positions pos0..pos0+S-1.

    q [B,S,Hq,D], k/v [B,S,Hkv,D], gate [B,S,Hq,D] (None for a global layer), wq/wk [D].
    Keys are the cache's earlier positions (if a cache is given) followed by the chunk's own keys; the
    chunk's k_hat and v are appended to the cache.  Query head h reads KV head h // (Hq / Hkv).
    Returns float64 [B,S,Hq,D]."""
    q = np.asarray(q)
    B, S, Hq, D = q.shape
    Hkv = np.asarray(k).shape[2]
    G = Hq // Hkv
    if cache is None and pos0 != 0:
        raise ValueError("pos0 > 0 needs a cache holding positions 0..pos0-1")
    pos = pos0 + np.arange(S, dtype=np.int64)
    khat = cache_key(qk_prologue(k, pos[None, :, None], wk, eps, rotary_dims, base))   # [B,S,Hkv,D]
    qhat = qk_prologue(q, pos[None, :, None], wq, eps, rotary_dims, base)      # [B,S,Hq,D]
    vf = _as_f64(v)
    gf = None if gate is None else _as_f64(gate)
    out = np.empty((B, S, Hq, D), dtype=np.float64)
    for b in range(B):
        if cache is not None:
            if cache.length(layer, b) != pos0:
                raise ValueError("cache length differs from pos0")
            cache.append(layer, b, khat[b], vf[b])
        for kh in range(Hkv):
            if cache is not None:
                kk, vv, kp = cache.keys(layer, b, kh)
            else:
                kk, vv, kp = khat[b, :, kh], vf[b, :, kh], pos
            heads = list(range(kh * G, (kh + 1) * G))
            qrows = qhat[b][:, heads, :].transpose(1, 0, 2).reshape(-1, D)       # [G*S, D]
            qp = np.tile(pos, G)
            grows = None if gf is None else gf[b][:, heads, :].transpose(1, 0, 2).reshape(-1, D)
            o = attend(qrows, qp, kk, vv, kp, window, grows)
            out[b][:, heads, :] = o.reshape(G, S, D).transpose(1, 0, 2)
    return out


# ---------------------------------------------------------------------------- backward (training)
def _rope_transpose(dy, pos, rotary_dims: int, base: float) -> np.ndarray:
    """The transpose of step 2 (a rotation per pair, so its inverse): (d0, d1) -> (d0 cos a + d1 sin a,
    -d0 sin a + d1 cos a) with a = pos * base^(-2i/R).  dy [..., D]; pos broadcasts against dy.shape[:-1]."""
    dx = np.array(dy, dtype=np.float64, copy=True)
    p = np.broadcast_to(np.asarray(pos, dtype=np.float64), dx.shape[:-1])
    for i in range(rotary_dims // 2):
        a = p * base ** (-2.0 * i / rotary_dims)
        c, sn = np.cos(a), np.sin(a)
        d0, d1 = dx[..., 2 * i].copy(), dx[..., 2 * i + 1].copy()
        dx[..., 2 * i] = d0 * c + d1 * sn
        dx[..., 2 * i + 1] = -d0 * sn + d1 * c
    return dx


def _rmsnorm_backward(x, w, dy, eps: float):
    """Derivatives of step 1, y = x w / r with r = sqrt(mean(x^2) + eps), over the last axis:
    dx = (w dy) / r - x (sum_d w_d dy_d x_d) / (D r^3);  dw = sum over the rows of dy x / r."""
    x = _as_f64(x)
    w = _as_f64(w)
    D = x.shape[-1]
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    wdy = w * dy
    dx = wdy / r - x * np.sum(wdy * x, axis=-1, keepdims=True) / (D * r ** 3)
    dw = np.sum((dy * x / r).reshape(-1, D), axis=0)
    return dx, dw


def prefill_layer_backward(q, k, v, gate, wq, wk, dout, *, window: int | None, rotary_dims: int, base: float,
                           eps: float, delta_from_bf16_out: bool = False, dA_bf16: bool = False) -> dict:
    """Gradients of one attention layer's output (prefill_layer without a cache, positions 0..S-1) with respect
    to its inputs, given dout = dL/d(out) [B,S,Hq,D].  Returns float64 arrays: dq [B,S,Hq,D], dk, dv [B,S,Hkv,D],
    dgate [B,S,Hq,D] (None for a global layer), dwq, dwk [D]; and the forward's out and lse [B,S,Hq] (natural log
    of the softmax denominator: p_ij = exp(s_ij - lse_i)).

    Chain rule through steps 5 to 1, per (sequence, query head) with dense masked score matrices:
      A = p v, out = A (.) sigmoid(g):   dA = dout (.) sigmoid(g),  dg = dout (.) A (.) sigmoid(g) (1 - sigmoid(g))
      p = softmax(s):                    dp = dA v^T,  ds = p (.) (dp - rowsum(p (.) dp))
      s = q_hat k_hat^T / sqrt(D):       dq_hat = ds k_hat / sqrt(D),  dk_hat = ds^T q_hat / sqrt(D)
      A = p v:                           dv = p^T dA
    summed over the query heads that share a KV head; then through RoPE (its transpose) and RMSNorm.  The bf16
    rounding of k_hat (the cache form keys are read in) passes its gradient through unchanged.

    rowsum(p (.) dp) equals dout . out; delta_from_bf16_out=True forms it from the layer's bf16 output instead, as
    a backward that is handed the bf16 output must (the exact result is the default; the variant measures what
    that rounding alone costs).  dA_bf16=True rounds dA to bf16 before it enters dp and dv, as a backward whose
    gradient products take bf16 operands does (at a query that sees one key, p = 1 and the exact ds is zero; with
    the rounded dA and the bf16 output's Delta it is not)."""
    q = np.asarray(q)
    B, S, Hq, D = q.shape
    Hkv = np.asarray(k).shape[2]
    G = Hq // Hkv
    pos = np.arange(S, dtype=np.int64)
    qhat = qk_prologue(q, pos[None, :, None], wq, eps, rotary_dims, base)
    khat = cache_key(qk_prologue(k, pos[None, :, None], wk, eps, rotary_dims, base))
    vf = _as_f64(v)
    gf = None if gate is None else _as_f64(gate)
    do = _as_f64(dout)
    i, j = np.meshgrid(pos, pos, indexing="ij")
    vis = j <= i
    if window is not None and window > 0:
        vis &= (i - j) < window
    scale = 1.0 / np.sqrt(D)
    dqhat = np.zeros((B, S, Hq, D))
    dkhat = np.zeros((B, S, Hkv, D))
    dv = np.zeros((B, S, Hkv, D))
    dg = None if gf is None else np.zeros((B, S, Hq, D))
    out = np.zeros((B, S, Hq, D))
    lse = np.zeros((B, S, Hq))
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            sc = np.where(vis, (qhat[b, :, h] @ khat[b, :, kh].T) * scale, -np.inf)
            m = sc.max(axis=1, keepdims=True)
            e = np.exp(sc - m)
            l = e.sum(axis=1, keepdims=True)
            p = e / l
            lse[b, :, h] = (m + np.log(l))[:, 0]
            A = p @ vf[b, :, kh]
            if gf is None:
                out[b, :, h] = A
                dA = do[b, :, h]
            else:
                sg = 1.0 / (1.0 + np.exp(-gf[b, :, h]))
                out[b, :, h] = A * sg
                dA = do[b, :, h] * sg
                dg[b, :, h] = do[b, :, h] * A * sg * (1.0 - sg)
            if dA_bf16:
                dA = bf16_to_f64(round_bf16(dA))
            dp = dA @ vf[b, :, kh].T
            if delta_from_bf16_out:
                delta = np.sum(do[b, :, h] * bf16_to_f64(round_bf16(out[b, :, h])), axis=1, keepdims=True)
            else:
                delta = np.sum(p * dp, axis=1, keepdims=True)
            ds = p * (dp - delta)
            dqhat[b, :, h] = ds @ khat[b, :, kh] * scale
            dkhat[b, :, kh] += ds.T @ qhat[b, :, h] * scale
            dv[b, :, kh] += p.T @ dA
    dqn = _rope_transpose(dqhat, pos[None, :, None], rotary_dims, base)
    dkn = _rope_transpose(dkhat, pos[None, :, None], rotary_dims, base)
    dq, dwq = _rmsnorm_backward(q, wq, dqn, eps)
    dk, dwk = _rmsnorm_backward(k, wk, dkn, eps)
    return {"dq": dq, "dk": dk, "dv": dv, "dgate": dg, "dwq": dwq, "dwk": dwk, "out": out, "lse": lse}


def prefill_layer_backward_rows(q, k, v, gate, wq, wk, dout, *, window: int | None, rotary_dims: int, base: float,
                                eps: float, b: int, kv_head: int, query_rows, key_rows, block: int = 512) -> dict:
    """prefill_layer_backward at full size, for one (sequence b, KV head) on sampled rows: the gradients of the
    group's query heads at query_rows (dq, dgate [n_q, G, D]) and of the KV head at key_rows (dk, dv [n_k, D]).
    Each query row's scores, softmax, output and Delta are formed whole, exactly as in prefill_layer_backward; rows
    are taken `block` at a time only to bound memory, and the key-side sums add every row block's terms.  Each
    result comes twice: exact, and with Delta from the bf16 output ("*_d16")."""
    q = np.asarray(q)
    B, S, Hq, D = q.shape
    Hkv = np.asarray(k).shape[2]
    G = Hq // Hkv
    heads = list(range(kv_head * G, (kv_head + 1) * G))
    pos = np.arange(S, dtype=np.int64)
    qhat = qk_prologue(q[b][:, heads], pos[:, None], wq, eps, rotary_dims, base)             # [S, G, D]
    khat = cache_key(qk_prologue(np.asarray(k)[b][:, kv_head], pos, wk, eps, rotary_dims, base))   # [S, D]
    vf = _as_f64(np.asarray(v)[b][:, kv_head])
    gf = None if gate is None else _as_f64(np.asarray(gate)[b][:, heads])
    do = _as_f64(np.asarray(dout)[b][:, heads])
    qr = np.asarray(query_rows, dtype=np.int64)
    kr = np.asarray(key_rows, dtype=np.int64)
    scale = 1.0 / np.sqrt(D)
    res = {n: np.zeros((len(qr), G, D)) for n in ("dqhat", "dqhat_d16", "dgate")}
    for n in ("dkhat", "dkhat_d16", "dv"):
        res[n] = np.zeros((len(kr), D))
    for r0 in range(0, S, block):
        r1 = min(S, r0 + block)
        c0 = 0 if window is None or window <= 0 else max(0, r0 - window + 1)
        i = pos[r0:r1, None]
        j = pos[None, c0:r1]
        vis = j <= i
        if window is not None and window > 0:
            vis &= (i - j) < window
        kin = (kr >= c0) & (kr < r1)
        qin = (qr >= r0) & (qr < r1)
        for g in range(G):
            sc = np.where(vis, (qhat[r0:r1, g] @ khat[c0:r1].T) * scale, -np.inf)
            m = sc.max(axis=1, keepdims=True)
            e = np.exp(sc - m)
            p = e / e.sum(axis=1, keepdims=True)
            A = p @ vf[c0:r1]
            if gf is None:
                out, dA = A, do[r0:r1, g]
            else:
                sg = 1.0 / (1.0 + np.exp(-gf[r0:r1, g]))
                out, dA = A * sg, do[r0:r1, g] * sg
                res["dgate"][qin, g] = (do[r0:r1, g] * A * sg * (1.0 - sg))[qr[qin] - r0]
            delta = {"": np.sum(p * (dA @ vf[c0:r1].T), axis=1, keepdims=True),
                     "_d16": np.sum(do[r0:r1, g] * bf16_to_f64(round_bf16(out)), axis=1, keepdims=True)}
            if kin.any():
                jj = kr[kin] - c0
                dpJ = dA @ vf[kr[kin]].T                       # [rows, nJ]
                res["dv"][kin] += p[:, jj].T @ dA
                for sfx, dl in delta.items():
                    res["dkhat" + sfx][kin] += (p[:, jj] * (dpJ - dl)).T @ qhat[r0:r1, g] * scale
            if qin.any():
                ii = qr[qin] - r0
                dpI = dA[ii] @ vf[c0:r1].T
                for sfx, dl in delta.items():
                    res["dqhat" + sfx][qin, g] = (p[ii] * (dpI - dl[ii])) @ khat[c0:r1] * scale
    out = {"dv": res["dv"], "dgate": None if gf is None else res["dgate"]}
    for sfx in ("", "_d16"):
        dqn = _rope_transpose(res["dqhat" + sfx], qr[:, None], rotary_dims, base)
        out["dq" + sfx], _ = _rmsnorm_backward(q[b][qr][:, heads], wq, dqn, eps)
        dkn = _rope_transpose(res["dkhat" + sfx], kr, rotary_dims, base)
        out["dk" + sfx], _ = _rmsnorm_backward(np.asarray(k)[b][kr, kv_head], wk, dkn, eps)
    return out


# ---------------------------------------------------------------------------- projections around the core
def linear(x, w) -> np.ndarray:
    """A linear layer's forward y = x W^T in float64: x [..., K], w [N, K] (W stored out x in)."""
    return _as_f64(x) @ _as_f64(w).T


# FP8 E4M3 (OCP) from its definition: sign, 4 exponent bits (bias 7), 3 mantissa bits; normals
# 2^(e-7) (1 + m/8) for e = 1..15 except e = 15, m = 7 (NaN), largest finite 448; subnormals m 2^-9.
E4M3_MAX = 448.0


def e4m3_encode(v) -> np.ndarray:
    """Codes (uint8) of float32 values, nearest-even, saturating at +-448 (finite inputs).  The decision is
    taken on the float32 value itself (what the quantised product is before encoding)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    code = np.zeros(a.shape, dtype=np.int64)
    sat = a >= E4M3_MAX
    sub = a < 2.0 ** -6
    nrm = ~sat & ~sub
    code[sat] = 0x7E
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)              # 0..8 (8 = the smallest normal)
    f, p = np.frexp(a[nrm])                                            # a = f 2^p, f in [0.5, 1)
    e = p - 1
    q = np.rint((a[nrm] / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)   # 0..8, nearest-even
    code[nrm] = np.minimum((e + 7) * 8 + q, 0x7E)                    # q = 8 carries into the exponent
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (the NaN code is not produced by e4m3_encode)."""
    c = np.asarray(codes, dtype=np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where(c & 0x80, -mag, mag)


class Fp8DelayedScaling:
    """Delayed scaling of n FP8 tensors (onedev.kr "What differs": FP8 matmuls with delayed scaling over a
    1,024-step amax history).  Per tensor t: the scale in use s_t (float32, 1 at first); encode(t, v) gives the codes
    E4M3(v * s_t) of the float32 products and notes this call's max |v|; commit() ends a call: every tensor encoded
    in it gets its max |v| in history slot idx and its next scale 448 / max(history) in float32 (1 if the history
    is zero), then idx advances.  Tensors not encoded in a call keep their state."""

    def __init__(self, n: int, history: int = 1024):
        self.n, self.H = n, history
        self.hist = np.zeros((n, history), dtype=np.float32)
        self.idx = 0
        self.scale = np.ones(n, dtype=np.float32)
        self._amax = {}

    def encode(self, t: int, v) -> np.ndarray:
        vf = _as_f64(v).astype(np.float32)          # bf16 values are exact in float32
        self._amax[t] = max(self._amax.get(t, np.float32(0)), np.float32(np.max(np.abs(vf))) if vf.size else np.float32(0))
        return e4m3_encode(vf * self.scale[t])      # float32 products, as the kernels form them

    def inv(self, t: int) -> np.float64:
        """The dequantisation factor 1/s_t, formed in float32."""
        return np.float64(np.float32(1.0) / self.scale[t])

    def commit(self):
        for t, a in self._amax.items():
            self.hist[t, self.idx] = a
            m = self.hist[t].max()
            self.scale[t] = np.float32(E4M3_MAX) / m if m > 0 else np.float32(1.0)
        self._amax = {}
        self.idx = (self.idx + 1) % self.H


def fp8_matmul(cx, cw, inv_x, inv_w) -> np.ndarray:
    """x W^T from E4M3 codes: (decode(cx) . decode(cw)^T) * (1/s_x) * (1/s_w), float64."""
    return (e4m3_decode(cx) @ e4m3_decode(cw).T) * inv_x * inv_w


class Fp8DelayedLinear:
    """y = x W^T with both operands in E4M3 under delayed scaling: tensors 0 = x, 1 = W of a
    Fp8DelayedScaling state; one call encodes both with the current scales, multiplies and commits."""

    def __init__(self, K: int, N: int, history: int = 1024):
        self.K, self.N, self.H = K, N, history
        self.state = Fp8DelayedScaling(2, history)

    @property
    def scale(self):
        return self.state.scale

    def __call__(self, x, w):
        st = self.state
        cx, cw = st.encode(0, x), st.encode(1, w)
        y = fp8_matmul(cx, cw, st.inv(0), st.inv(1))
        st.commit()
        return y, cx, cw


def attention_layer(h, w_q, w_k, w_v, w_g, w_o, q_norm_w, k_norm_w, *, Hq: int, Hkv: int, window: int | None,
                    rotary_dims: int, base: float, eps: float) -> np.ndarray:
    """The layer around the core (onedev.kr "How it works": o_proj(A_SWA(q, k, v) (.) sigmoid(g_proj(h))); the
    global layer without the gate): q, k, v, g = h W^T, the attention of prefill_layer, y = o W_o^T.

    The layer's tensors are bf16 between its operations (bf16 I/O, fp32 or better accumulation), so q, k, v, g
    and the attention output o are rounded once to bf16 (nearest-even) before the next operation reads them;
    everything else is float64.  h [B,S,d_model]; returns y float64 [B,S,d_model]."""
    B, S, dm = np.asarray(h).shape
    D = np.asarray(q_norm_w).shape[-1]
    def proj(w, H):
        return round_bf16(linear(h, w)).reshape(B, S, H, D)
    q, k, v = proj(w_q, Hq), proj(w_k, Hkv), proj(w_v, Hkv)
    g = None if w_g is None else proj(w_g, Hq)
    o = prefill_layer(q, k, v, g, q_norm_w, k_norm_w, window=window, rotary_dims=rotary_dims, base=base, eps=eps)
    return linear(round_bf16(o).reshape(B, S, Hq * D), w_o)


FP8_LAYER_TENSORS = ("h", "w_q", "w_k", "w_v", "w_g", "o", "w_o")


def attention_layer_fp8(h, w_q, w_k, w_v, w_g, w_o, q_norm_w, k_norm_w, state: Fp8DelayedScaling, *, Hq: int, Hkv: int,
                        window: int | None, rotary_dims: int, base: float, eps: float,
                        codes: dict | None = None) -> np.ndarray:
    """attention_layer with every projection on E4M3 operands (onedev.kr "What differs": FP8 matmuls, E4M3 in the
    forward pass, delayed scaling).  state holds seven tensors in the order of FP8_LAYER_TENSORS; h is encoded once
    for the four input projections and the bf16 attention output o once for o_proj, each weight once, all with the
    scales in use before the call; the call ends with state.commit().  q, k, v, g and o are bf16 between the
    operations as in attention_layer.  Returns y float64 [B,S,d_model]; a dict passed as codes receives every
    tensor's E4M3 codes by name."""
    B, S, dm = np.asarray(h).shape
    D = np.asarray(q_norm_w).shape[-1]
    t = {name: i for i, name in enumerate(FP8_LAYER_TENSORS)}
    ch = state.encode(t["h"], np.asarray(h).reshape(B * S, dm))

    got = {"h": ch}

    def proj(name, w, H):
        cw = got[name] = state.encode(t[name], w)
        return round_bf16(fp8_matmul(ch, cw, state.inv(t["h"]), state.inv(t[name]))).reshape(B, S, H, D)

    q, k, v = proj("w_q", w_q, Hq), proj("w_k", w_k, Hkv), proj("w_v", w_v, Hkv)
    g = None if w_g is None else proj("w_g", w_g, Hq)
    o = round_bf16(prefill_layer(q, k, v, g, q_norm_w, k_norm_w, window=window, rotary_dims=rotary_dims, base=base,
                                 eps=eps)).reshape(B * S, Hq * D)
    co, cwo = got["o"], got["w_o"] = state.encode(t["o"], o), state.encode(t["w_o"], w_o)
    y = fp8_matmul(co, cwo, state.inv(t["o"]), state.inv(t["w_o"]))
    state.commit()
    if codes is not None:
        codes.update(got)
    return y.reshape(B, S, dm)


def decode_step(q, k, v, gate, wq, wk, positions, cache: OracleCache, *, rotary_dims: int, base: float,
                eps: float) -> np.ndarray:
    """One new token per sequence in every layer: q/gate [L,B,Hq,D], k/v [L,B,Hkv,D], wq/wk [L,D],
    positions [B] (absolute position of the new token; the cache must hold positions 0..p-1).
    The new key and value are appended first, then the token attends over the cache (itself included).
    Layer l (1-indexed) is global iff it is in the cache's global set; others use the window and gate.
    Returns float64 [L,B,Hq,D]."""
    q = np.asarray(q)
    L, B, Hq, D = q.shape
    Hkv = np.asarray(k).shape[2]
    G = Hq // Hkv
    positions = np.asarray(positions, dtype=np.int64)
    out = np.empty((L, B, Hq, D), dtype=np.float64)
    for li in range(L):
        layer = li + 1
        glob = layer in cache.glob
        for b in range(B):
            p = int(positions[b])
            if cache.length(layer, b) != p:
                raise ValueError("cache length differs from the new token's position")
            khat = cache_key(qk_prologue(np.asarray(k)[li, b][None], p, wk[li], eps, rotary_dims, base))
            cache.append(layer, b, khat, _as_f64(np.asarray(v)[li, b])[None])
            qhat = qk_prologue(np.asarray(q)[li, b], p, wq[li], eps, rotary_dims, base)   # [Hq, D]
            for kh in range(Hkv):
                kk, vv, kp = cache.keys(layer, b, kh)
                heads = slice(kh * G, (kh + 1) * G)
                g = None if glob else np.asarray(gate)[li, b, heads]
                out[li, b, heads] = attend(qhat[heads], p, kk, vv, kp, None if glob else cache.W, g)
    return out
