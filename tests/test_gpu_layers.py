"""GPU parity of the projections around the core (hipBLASLt bf16 GEMMs) and of whole attention layers from the
hidden state, against the fp64 oracle on the same seeded inputs.

Bars: a projection alone is within its own rounding: |y - y_64| <= 2^-8 |y_64| (the bf16 rounding of the
result) + 1e-3 rms(y_64) (fp32 accumulation over K = 4096 products); a whole layer is held to the attention
core's bar (max-abs 1e-2, mean-abs 1e-3), its output being o W_o^T of an attention output within that bar.
"""
import numpy as np
import pytest

import oracle
import synth
from _inputs import TOL_MAX_ABS, TOL_MEAN_ABS, compare, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

D_MODEL, HQ, HKV, D = 4096, 32, 8, 128


@pytest.fixture(scope="module")
def zg():
    import torch
    assert torch.cuda.is_available()
    import global_attention_gated_amd as m
    return m


def weight_bits(seed, tensor, n_out, n_in):
    """N(0,1) / sqrt(n_in) in bf16 (n_in a power of 4, so the scale is an exact power of two)."""
    w = synth.bf16_bits_to_f64(synth.normal_bf16(seed, 0, tensor, (n_out, n_in)))
    return synth.f64_to_bf16_bits(w / np.sqrt(n_in))


@pytest.mark.parametrize("T,K,N", [(300, 4096, 1024), (513, 4096, 4096), (1, 4096, 4096), (64, 256, 96)])
def test_linear_bf16_matches_oracle(zg, T, K, N):
    x = synth.normal_bf16(11, 0, synth.TENSOR_H, (T, K))
    w = weight_bits(11, synth.TENSOR_PQ, N, K)
    y = to_host_f64(zg.linear_bf16(to_dev(x), to_dev(w)))
    ref = oracle.linear(x, w)
    err = np.abs(y - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
    assert np.all(err <= bound), f"max excess {float((err - bound).max()):.3e}"


def _layer_inputs(seed, B, S, gated):
    h = synth.normal_bf16(seed, 0, synth.TENSOR_H, (B, S, D_MODEL))
    w = {"q": weight_bits(seed, synth.TENSOR_PQ, HQ * D, D_MODEL), "k": weight_bits(seed, synth.TENSOR_PK, HKV * D, D_MODEL),
         "v": weight_bits(seed, synth.TENSOR_PV, HKV * D, D_MODEL),
         "g": weight_bits(seed, synth.TENSOR_PG, HQ * D, D_MODEL) if gated else None,
         "o": weight_bits(seed, synth.TENSOR_PO, D_MODEL, HQ * D)}
    qn = synth.norm_weight_bf16(seed, 1, synth.TENSOR_WQ, D)
    kn = synth.norm_weight_bf16(seed, 1, synth.TENSOR_WK, D)
    return h, w, qn, kn


@pytest.mark.parametrize("gated,B,S", [(True, 1, 400), (False, 1, 300), (True, 2, 129)])
def test_attention_layer_from_hidden_state_matches_oracle(zg, gated, B, S):
    h, w, qn, kn = _layer_inputs(21 + S, B, S, gated)
    dv = {k: (None if v is None else to_dev(v)) for k, v in w.items()}
    if gated:
        y = zg.gated_swa_layer(to_dev(h), dv["q"], dv["k"], dv["v"], dv["g"], dv["o"], to_dev(qn), to_dev(kn), Hq=HQ,
                               Hkv=HKV, window=128, rotary_dims=42, rope_base=1e4, eps=1e-6)
    else:
        y = zg.global_layer(to_dev(h), dv["q"], dv["k"], dv["v"], dv["o"], to_dev(qn), to_dev(kn), Hq=HQ, Hkv=HKV,
                            rotary_dims=42, rope_base=1e4, eps=1e-6)
    ref = oracle.attention_layer(h, w["q"], w["k"], w["v"], w["g"], w["o"], qn, kn, Hq=HQ, Hkv=HKV,
                                 window=128 if gated else None, rotary_dims=42, base=1e4, eps=1e-6)
    got = to_host_f64(y)
    print(f"layer {'swa' if gated else 'global'} B{B} S{S}: max_abs {np.abs(got - ref).max():.3e} "
          f"mean_abs {np.abs(got - ref).mean():.3e} rms(y) {np.sqrt(np.mean(ref ** 2)):.3f}")
    compare(got, ref, f"{'gated SWA' if gated else 'global'} layer B{B} S{S}")


def test_fp8_delayed_scaling_matches_oracle_over_calls(zg):
    """Five FP8 projections through one state whose input magnitude changes by powers of two: the E4M3 codes of
    x and W equal the oracle's byte for byte, the scales in use equal its float32 scales, and y is within its
    rounding bound (the codes' products are exact; fp32 accumulation; bf16 result)."""
    T, K, N = 300, 4096, 1024
    f = zg.Fp8Linear(K, N, history=1024)
    ref = oracle.Fp8DelayedLinear(K, N, history=1024)
    w = weight_bits(31, synth.TENSOR_PK, N, K)
    x0 = synth.bf16_bits_to_f64(synth.normal_bf16(31, 0, synth.TENSOR_H, (T, K)))
    for call, mag in enumerate((1.0, 4.0, 0.25, 16.0, 1.0)):
        x = synth.f64_to_bf16_bits(x0 * mag)                     # exact: power-of-two factors
        sx, sw = f.scales()
        assert (np.float32(sx), np.float32(sw)) == (ref.scale[0], ref.scale[1]), f"call {call}"
        y = to_host_f64(f(to_dev(x), to_dev(w)))
        yr, cx, cw = ref(x, w)
        gx, gw = f.codes(T)
        np.testing.assert_array_equal(gx.numpy(), cx, err_msg=f"x codes, call {call}")
        np.testing.assert_array_equal(gw.numpy(), cw, err_msg=f"W codes, call {call}")
        err = np.abs(y - yr)
        bound = 2.0 ** -8 * np.abs(yr) + 1e-3 * np.sqrt(np.mean(yr ** 2))
        assert np.all(err <= bound), f"call {call}: max excess {float((err - bound).max()):.3e}"
    f.close()


def _e4m3_step(a):
    """Spacing of E4M3 values at magnitude a (normals: 2^(e-3) in [2^e, 2^(e+1)); subnormals 2^-9)."""
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.exp2(e - 3)


def _fp8_layer_codes(ws, B, S, gated):
    """The E4M3 codes the layer leaves in its workspace (after the activations; the attention's part is last)."""
    import global_attention_gated_amd as zgm
    a = lambda n: (n + 255) // 256 * 256
    T, qd, kd = B * S, HQ * D, HKV * D
    off = zgm.layer_workspace_bytes(B, S, HQ, HKV, D) - zgm.workspace_bytes(B, S, HKV, D)   # right after the activations
    mem = ws.cpu().numpy()
    out = {}
    for name, n, shape in (("h", T * D_MODEL, (T, D_MODEL)), ("o", T * qd, (T, qd)), ("w_q", qd * D_MODEL, (qd, D_MODEL)),
                           ("w_k", kd * D_MODEL, (kd, D_MODEL)), ("w_v", kd * D_MODEL, (kd, D_MODEL)),
                           ("w_g", qd * D_MODEL, (qd, D_MODEL)), ("w_o", D_MODEL * qd, (D_MODEL, qd))):
        out[name] = mem[off:off + n].reshape(shape)
        off += a(n)
    if not gated:
        del out["w_g"]
    return out


@pytest.mark.parametrize("gated,B,S", [(True, 1, 400), (False, 1, 300)])
def test_fp8_layer_matches_oracle_over_calls(zg, gated, B, S):
    """Three calls of a layer with FP8 projections through one delayed-scaling state, h scaled by 1, 1/2, 1 (exact
    power-of-two factors).  Per call:
    - the scales in use equal the oracle's float32 scales (h and the weights exactly; o, whose max |o| comes from
      the attention output, within one bf16 step of the maximum, 2^-7 relative);
    - the E4M3 codes of h and of every weight equal the oracle's byte for byte (same inputs, same float32 decision);
    - the codes of the attention output o: the GPU's o is within the core's bar of the oracle's (and its scale
      within 2^-7), so a code's value may differ from the oracle's by that bar plus one E4M3 step at its magnitude
      (o s on a rounding boundary), and no more; such differences stay rare (<= 5% of the elements);
    - y: mean-abs within the core's bar (1e-3); max-abs within the core's 1e-2 plus two such steps at the largest
      |o| times the largest |W_o| entry (one flipped code moves y_j by its step times w_jk)."""
    h, w, qn, kn = _layer_inputs(41 + S, B, S, gated)
    h0 = synth.bf16_bits_to_f64(h)
    dv = {k: (None if v is None else to_dev(v)) for k, v in w.items()}
    st = zg.Fp8Layer(D_MODEL, HQ, HKV, D, history=1024)
    ref = oracle.Fp8DelayedScaling(7, history=1024)
    o_t = oracle.FP8_LAYER_TENSORS.index("o")
    import torch
    ws = torch.empty(zg.fp8_layer_workspace_bytes(B, S, D_MODEL, HQ, HKV, D), dtype=torch.uint8, device="cuda")
    wo_max = float(np.abs(synth.bf16_bits_to_f64(w["o"])).max())
    for call, mag in enumerate((1.0, 0.5, 1.0)):
        hb = synth.f64_to_bf16_bits(h0 * mag)
        got_s = np.asarray(st.scales(), dtype=np.float32)
        for t, name in enumerate(oracle.FP8_LAYER_TENSORS):
            if t == o_t:
                assert abs(got_s[t] / ref.scale[t] - 1) <= 2.0 ** -7, f"call {call}: scale of o"
            else:
                assert got_s[t] == ref.scale[t], f"call {call}: scale of {name}"
        s_o = float(ref.scale[o_t])
        if gated:
            y = zg.gated_swa_layer_fp8(to_dev(hb), dv["q"], dv["k"], dv["v"], dv["g"], dv["o"], to_dev(qn), to_dev(kn),
                                       fp8=st, Hq=HQ, Hkv=HKV, window=128, rotary_dims=42, rope_base=1e4, eps=1e-6,
                                       workspace=ws)
        else:
            y = zg.global_layer_fp8(to_dev(hb), dv["q"], dv["k"], dv["v"], dv["o"], to_dev(qn), to_dev(kn), fp8=st,
                                    Hq=HQ, Hkv=HKV, rotary_dims=42, rope_base=1e4, eps=1e-6, workspace=ws)
        rc = {}
        yr = oracle.attention_layer_fp8(hb, w["q"], w["k"], w["v"], w["g"], w["o"], qn, kn, ref, Hq=HQ, Hkv=HKV,
                                        window=128 if gated else None, rotary_dims=42, base=1e4, eps=1e-6, codes=rc)
        gc = _fp8_layer_codes(ws, B, S, gated)
        for name in gc:
            if name != "o":
                np.testing.assert_array_equal(gc[name], rc[name], err_msg=f"call {call}: codes of {name}")
        diff = gc["o"] != rc["o"]
        vg = oracle.e4m3_decode(gc["o"]) / float(got_s[o_t])
        vr = oracle.e4m3_decode(rc["o"]) / s_o
        lim = TOL_MAX_ABS + _e4m3_step(np.maximum(np.abs(vg), np.abs(vr)) * s_o) / s_o
        assert np.all(np.abs(vg - vr) <= lim), f"call {call}: o codes beyond one step of the oracle's"
        assert diff.mean() <= 0.05, f"call {call}: {diff.mean():.4f} of the o codes differ"
        got = to_host_f64(y)
        err = np.abs(got - yr)
        o_max = float(np.abs(oracle.e4m3_decode(rc["o"])).max()) / s_o
        allow = 2 * float(_e4m3_step(o_max * s_o)) / s_o * wo_max
        print(f"fp8 layer {'swa' if gated else 'global'} call {call}: max_abs {err.max():.3e} mean_abs {err.mean():.3e} "
              f"rms(y) {np.sqrt(np.mean(yr ** 2)):.3f}; o codes differing {diff.mean():.2e}; flip allowance {allow:.3e}; "
              f"s_o {float(got_s[o_t]):.6g} vs {s_o:.6g}")
        assert err.mean() <= TOL_MEAN_ABS, f"call {call}: mean_abs {err.mean():.3e}"
        assert err.max() <= TOL_MAX_ABS + allow, f"call {call}: max_abs {err.max():.3e} > {TOL_MAX_ABS + allow:.3e}"
    st.close()
