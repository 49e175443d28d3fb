"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no arithmetic of the attention method.  It only makes
numbers: every element is

    TABLE[ splitmix64_output(stream_key(seed, layer, tensor), index) >> 48 ]

where ``splitmix64_output(k, n)`` is the n-th output (0-based) of a SplitMix64
generator seeded with ``k`` (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014: state += 0x9E3779B97F4A7C15,
then the 30/27/31 xor-shift-multiply finaliser), and TABLE is the 65,536-entry
bf16 quantile table of the standard normal distribution,
``TABLE[u] = bf16_rne(Phi^-1((u + 0.5) / 65536))``.

The same bits come out on the CPU (numpy, here) and on the GPU
(``synth/synth_fill.hip``), so either side can regenerate any slice of a
tensor from its logical flat index without moving the tensor.

Tensor ids: q=0, k=1, v=2, gate=3, q-norm weight=4, k-norm weight=5,
cached K=6, cached V=7.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_GATE = 0, 1, 2, 3
TENSOR_WQ, TENSOR_WK, TENSOR_CACHE_K, TENSOR_CACHE_V = 4, 5, 6, 7
# the hidden state and the projection weights around the core (q, k, v, g, o)
TENSOR_H, TENSOR_PQ, TENSOR_PK, TENSOR_PV, TENSOR_PG, TENSOR_PO = 8, 9, 10, 11, 12, 13
# the output gradient of the backward
TENSOR_DOUT = 14


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on uint64 arrays (wrapping arithmetic)."""
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _mix_scalar(x: int) -> int:
    m = (1 << 64) - 1
    z = x & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def stream_key(seed: int, layer: int, tensor: int) -> int:
    """64-bit key of the stream for (seed, layer, tensor).

    It is the first SplitMix64 output of a generator seeded with
    ``seed ^ (layer << 16 | tensor) * 0x9E3779B97F4A7C15`` (mod 2^64), so
    distinct (layer, tensor) pairs start far apart.
    """
    m = (1 << 64) - 1
    tag = ((layer & 0xFFFFFFFF) << 16) | (tensor & 0xFFFF)
    s = (seed ^ ((tag * 0x9E3779B97F4A7C15) & m)) & m
    return _mix_scalar((s + 0x9E3779B97F4A7C15) & m)


def _bf16_bits_rne_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); return the bits.

    Exact single rounding: the significand is scaled to 8 bits and rounded
    with numpy's half-to-even ``rint``; the result is representable in bf16,
    hence exactly in float32, whose top 16 bits are the bf16 encoding.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Hand-made inputs: bf16 bits (nearest-even) of float values."""
    return _bf16_bits_rne_from_f64(np.asarray(x, dtype=np.float64))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _make_table() -> np.ndarray:
    from scipy.special import ndtri
    u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return _bf16_bits_rne_from_f64(ndtri(u))


TABLE = _make_table()            # uint16[65536], bf16 bits of N(0,1) quantiles


def normal_bf16_at(seed: int, layer: int, tensor: int, index) -> np.ndarray:
    """bf16 bits of the stream's elements at the given flat indices."""
    idx = np.asarray(index, dtype=np.int64).astype(np.uint64)
    k = np.uint64(stream_key(seed, layer, tensor))
    with np.errstate(over="ignore"):
        z = k + (idx + np.uint64(1)) * GOLDEN
    return TABLE[(_mix(z) >> np.uint64(48)).astype(np.int64)]


def normal_bf16(seed: int, layer: int, tensor: int, shape, index_offset: int = 0) -> np.ndarray:
    """bf16 bits, in C order of ``shape``, of flat indices offset .. offset+n-1."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, n, step):
        e = min(n, s + step)
        out[s:e] = normal_bf16_at(seed, layer, tensor,
                                  np.arange(index_offset + s, index_offset + e, dtype=np.int64))
    return out.reshape(shape)


def norm_weight_bf16(seed: int, layer: int, tensor: int, D: int, spread: float = 0.1) -> np.ndarray:
    """RMSNorm weight vector bf16(1 + spread * z), z from the stream; spread 0 gives ones."""
    z = bf16_bits_to_f64(normal_bf16(seed, layer, tensor, (D,)))
    return _bf16_bits_rne_from_f64(1.0 + spread * z)


def table_device(device):
    """The quantile table as a device tensor (int16 view of the bf16 bits)."""
    import torch
    return torch.from_numpy(TABLE.view(np.int16).copy()).to(device)


# ---------------------------------------------------------------------------
# GPU fill (synth/libsynth.so, built from synth/synth_fill.hip)
# ---------------------------------------------------------------------------
_lib = None
_tables = {}


def _load_gpu_lib():
    global _lib
    if _lib is None:
        import ctypes
        import os
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(path)
        lib.synth_fill_bf16.restype = ctypes.c_int
        lib.synth_fill_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_void_p]
        _lib = lib
    return _lib


def fill_device(dst_ptr: int, seed: int, layer: int, tensor: int, n_outer: int, n_inner: int,
                dst_outer_stride: int, idx_start: int, idx_outer_stride: int, device=None, stream=None):
    """Fill device memory (bf16 elements at ``dst_ptr``) with the stream's values.

    dst[o*dst_outer_stride + i] = value(idx_start + o*idx_outer_stride + i), o < n_outer, i < n_inner.
    """
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if dev not in _tables:
        _tables[dev] = table_device(dev)
    lib = _load_gpu_lib()
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    rc = lib.synth_fill_bf16(dst_ptr, n_outer, n_inner, dst_outer_stride, stream_key(seed, layer, tensor),
                             idx_start, idx_outer_stride, _tables[dev].data_ptr(), s)
    if rc != 0:
        raise RuntimeError(f"synth_fill_bf16 failed with status {rc}")


def normal_bf16_device(seed: int, layer: int, tensor: int, shape, index_offset: int = 0, device="cuda"):
    """A new contiguous device tensor (torch.bfloat16) holding the stream's values in C order."""
    import torch
    n = 1
    for s in shape:
        n *= int(s)
    t = torch.empty(tuple(shape), dtype=torch.bfloat16, device=device)
    if n:
        fill_device(t.data_ptr(), seed, layer, tensor, 1, n, n, index_offset, n, device=t.device)
    return t


def fill_kv_cache_layer(k_ptr: int, v_ptr: int, slots: int, *, seed: int, layer: int, batch: int, n_kv_heads: int,
                        head_dim: int, n_positions: int, is_global: bool, window: int, device=None):
    """Fill one layer of a KV cache in device memory as if positions 0..P-1 (P = n_positions) had been
    stored: K/V arrays [batch][n_kv_heads][slots][head_dim] (bf16); a global layer holds position p in
    row p, an SWA ring holds positions max(0, P-W)..P-1 in slot p mod W.  The value of (b, h, p, d) is
    stream (seed, layer, cached K = 6 / cached V = 7) at flat index ((b*n_kv_heads + h)*P + p)*head_dim + d.
    """
    P, D, W = n_positions, head_dim, window
    rows = batch * n_kv_heads
    for ptr, tid in ((k_ptr, TENSOR_CACHE_K), (v_ptr, TENSOR_CACHE_V)):
        if is_global:
            fill_device(ptr, seed, layer, tid, rows, P * D, slots * D, 0, P * D, device=device)
        else:
            p = max(0, P - W)
            while p < P:                      # contiguous runs of positions land in contiguous slots
                s = p % W
                run = min(P - p, W - s)
                fill_device(ptr + s * D * 2, seed, layer, tid, rows, run * D, slots * D, p * D, P * D, device=device)
                p += run


def kv_cache_values(seed: int, layer: int, tensor: int, b: int, h: int, positions, *, n_kv_heads: int,
                    head_dim: int, n_positions: int) -> np.ndarray:
    """Host bits [len(positions), head_dim] of the values fill_kv_cache_layer stores for (b, h)."""
    pos = np.asarray(positions, dtype=np.int64)
    idx = ((b * n_kv_heads + h) * n_positions + pos)[:, None] * head_dim + np.arange(head_dim)[None, :]
    return normal_bf16_at(seed, layer, tensor, idx)
