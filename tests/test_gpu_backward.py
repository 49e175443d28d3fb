"""GPU parity of the training path: the forward's log-sum-exp and the backward of a gated-SWA or global layer
(dq, dk, dv, dgate and the two norm-weight gradients), against the fp64 oracle's exact gradients on the same seeded
inputs.

Bar of the backward, per gradient X against the exact X_ref (elementwise, then the mean):
    |err| <= 2 |D_X| + 2^-7 |X_ref| + R_X / 16,        mean |err| <= 2 mean |D_X| + 0.005 R_X
with R_X = rms(X_ref) (dv's rms where X_ref is identically zero: one visible key), and D_X the change in the
exact gradient when Delta_i = dout_i . out_i is formed from the bf16 output, as this backward (the standard
flash-attention form) must: out is handed over in bf16, 2^-9 relative per element; and when dA = dout (.)
sigmoid(g) enters dp and dv as the bf16 operand the gradient products take.  At the first positions of a sequence,
where a query sees one to three keys (p near 1), ds = p (dp - Delta) is the difference of two values of size
|dA| |v| whose exact difference is zero or small, and these two roundings are most of the error there; R_X, the
rms over the whole gradient, shrinks as windows widen and sequences grow, so the R_X / 16 term alone does not cover
them (a seeded random case with 32 query heads, W 200-300, S 1045: 1.04 x that bound at positions 0-2 only).  The other terms: the bf16
rounding of every result (2^-9 |X|, 2^-7 leaves margin), and the bf16 operands of the gradient products (dA, P,
dS, q_hat: 2^-9 each, fp32 accumulation), whose errors scale with the summed terms rather than with the result:
ds_ij = p_ij (dp_ij - Delta_i) subtracts two values of size ~sqrt(D) |dout| |v| to get a much smaller one.
Measured (small cases and 1 x 16384): the largest element error is 0.055 R_X (a 16K gated layer's dq), 0.78 of this
bound; at 0.03 R_X it would be 1.46.  These errors come from the bf16 gradient products (dA = dout sigmoid(g) in
bf16 enters dp, whose difference with Delta is small), not from a missed term: a missed tile, wrong mask, head or
scale errs by ~R_X on whole rows.  Mean 0.1-0.3% of R_X.
"""
import numpy as np
import pytest

import oracle
import synth
from _inputs import Layer, compare, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zg():
    import torch
    assert torch.cuda.is_available()
    import global_attention_gated_amd as m
    return m


def _problem(seed, gated, B, S, Hq, Hkv, W):
    L = Layer(seed, 1, B, S, Hq, Hkv, gated=gated)
    dout = synth.normal_bf16(seed, 1, synth.TENSOR_DOUT, (B, S, Hq, 128))
    kw = dict(window=W if gated else None, rotary_dims=42, base=1e4, eps=1e-6)
    ref = oracle.prefill_layer_backward(L.q, L.k, L.v, L.gate, L.wq, L.wk, dout, **kw)
    ref16 = oracle.prefill_layer_backward(L.q, L.k, L.v, L.gate, L.wq, L.wk, dout, delta_from_bf16_out=True,
                                          dA_bf16=True, **kw)
    return L, dout, ref, ref16


def _check(g, ref, ref16, gated, tag):
    names = [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dq_norm_w", "dwq"), ("dk_norm_w", "dwk")]
    if gated:
        names.append(("dgate", "dgate"))
    rms_dv = float(np.sqrt(np.mean(ref["dv"] ** 2)))
    for gn, rn in names:
        got = to_host_f64(g[gn])
        r, r16 = ref[rn], ref16[rn]
        assert np.all(np.isfinite(got)), f"{tag} {gn}: non-finite"
        err = np.abs(got - r)
        dlt = np.abs(r16 - r)
        rms = float(np.sqrt(np.mean(r ** 2)))
        R = rms if rms > 0.01 * rms_dv else rms_dv
        bound = 2 * dlt + 2.0 ** -7 * np.abs(r) + R / 16
        print(f"{tag} {gn}: max_abs {err.max():.3e} mean_abs {err.mean():.3e} R {R:.3e} "
              f"max err/bound {np.max(err / bound):.3f} mean/R {err.mean() / R:.2e}")
        assert np.all(err <= bound), f"{tag} {gn}: max err/bound {np.max(err / bound):.3f}"
        mean_bound = 2 * float(np.mean(dlt)) + 0.005 * R
        assert err.mean() <= mean_bound, f"{tag} {gn}: mean_abs {err.mean():.3e} > {mean_bound:.3e}"


CASES = [(True, 1, 300, 8, 2, 128), (False, 1, 257, 8, 2, 0), (True, 2, 129, 4, 1, 16), (True, 1, 33, 4, 1, 128),
         (False, 1, 1, 4, 1, 0), (True, 1, 1, 4, 1, 128),
         # window 1 (no score gradient), a window wider than the tile ring, 3 sequences x 4 KV heads, ragged ends
         (True, 1, 97, 4, 1, 1), (True, 1, 400, 4, 1, 256), (True, 3, 70, 16, 4, 32), (False, 3, 161, 16, 4, 0),
         # causal: three 256-key blocks (a pair and the middle one alone), the last one past the sequence's end
         (False, 2, 600, 8, 2, 0)]


@pytest.mark.parametrize("gated,B,S,Hq,Hkv,W", CASES)
def test_backward_alone_matches_oracle(zg, gated, B, S, Hq, Hkv, W):
    """The backward fed the oracle's own out (rounded to bf16) and lse (float32)."""
    import torch
    L, dout, ref, ref16 = _problem(61, gated, B, S, Hq, Hkv, W)
    out = to_dev(oracle.round_bf16(ref["out"]))
    lse = torch.from_numpy(np.ascontiguousarray(ref["lse"].transpose(0, 2, 1)).astype(np.float32)).cuda()
    g = zg.prefill_backward(L.dq, L.dk, L.dv, L.dgate, L.dwq, L.dwk, out, lse, to_dev(dout), window=W,
                            rotary_dims=42, rope_base=1e4, eps=1e-6)
    _check(g, ref, ref16, gated, f"alone {'swa' if gated else 'global'} B{B} S{S}")


@pytest.mark.parametrize("gated,B,S,Hq,Hkv,W", CASES)
def test_training_forward_backward_matches_oracle(zg, gated, B, S, Hq, Hkv, W):
    """The training pipeline: the GPU forward's out and lse feed the GPU backward."""
    L, dout, ref, ref16 = _problem(61, gated, B, S, Hq, Hkv, W)
    out, lse = zg.prefill_train(L.dq, L.dk, L.dv, L.dgate, L.dwq, L.dwk, window=W, rotary_dims=42, rope_base=1e4,
                                eps=1e-6)
    compare(to_host_f64(out), ref["out"], "training forward out")
    compare(lse.detach().cpu().numpy().transpose(0, 2, 1).astype(np.float64), ref["lse"], "training forward lse")
    g = zg.prefill_backward(L.dq, L.dk, L.dv, L.dgate, L.dwq, L.dwk, out, lse, to_dev(dout), window=W,
                            rotary_dims=42, rope_base=1e4, eps=1e-6)
    _check(g, ref, ref16, gated, f"train {'swa' if gated else 'global'} B{B} S{S}")
