"""Seeded inputs for the parity tests (host bits for the oracle, device tensors for the HIP path)."""
from __future__ import annotations

import numpy as np

import synth

TOL_MAX_ABS = 1e-2    # per element, |gpu_bf16 - oracle_fp64|
TOL_MEAN_ABS = 1e-3   # mean over the compared elements


def to_dev(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def to_host_f64(t):
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


def to_host_bits(t):
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


class Layer:
    """Inputs of one prefill layer: bits (numpy uint16) and device tensors."""

    def __init__(self, seed, layer, B, S, Hq, Hkv, D=128, gated=True, w_spread=0.1, device="cuda", pos0=0,
                 S_total=None):
        # inputs of a chunk at rows pos0..pos0+S-1 of a sequence of S_total rows: flat indices follow
        # the full [B, S_total, H, D] layout so chunks of one sequence are slices of the same stream
        S_total = S if S_total is None else S_total
        self.seed, self.layer, self.B, self.S, self.Hq, self.Hkv, self.D = seed, layer, B, S, Hq, Hkv, D

        def gen(tensor, H):
            out = np.empty((B, S, H, D), dtype=np.uint16)
            for b in range(B):
                off = ((b * S_total) + pos0) * H * D
                out[b] = synth.normal_bf16(seed, layer, tensor, (S, H, D), index_offset=off)
            return out

        self.q = gen(synth.TENSOR_Q, Hq)
        self.k = gen(synth.TENSOR_K, Hkv)
        self.v = gen(synth.TENSOR_V, Hkv)
        self.gate = gen(synth.TENSOR_GATE, Hq) if gated else None
        self.wq = synth.norm_weight_bf16(seed, layer, synth.TENSOR_WQ, D, spread=w_spread)
        self.wk = synth.norm_weight_bf16(seed, layer, synth.TENSOR_WK, D, spread=w_spread)
        if device is not None:
            self.dq, self.dk, self.dv = to_dev(self.q, device), to_dev(self.k, device), to_dev(self.v, device)
            self.dgate = None if self.gate is None else to_dev(self.gate, device)
            self.dwq, self.dwk = to_dev(self.wq, device), to_dev(self.wk, device)


def compare(got_f64, ref_f64, what=""):
    err = np.abs(np.asarray(got_f64) - np.asarray(ref_f64))
    assert np.all(np.isfinite(got_f64)), f"{what}: non-finite GPU output"
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= TOL_MAX_ABS and mean <= TOL_MEAN_ABS, f"{what}: max_abs {mx:.3e} mean_abs {mean:.3e}"
    return mx, mean
