"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix (CPU only).

Each test ties one step of the oracle to something other than the oracle itself: a library routine
(torch's rms_norm and scaled_dot_product_attention in float64), the textbook complex form of RoPE, a
closed form, a special case, an invariant, or a value the pages print (tests/golden/*.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

RNG = np.random.default_rng(12345)


def _sdpa(q, k, v, mask):
    """torch's softmax attention in float64 on the CPU: q [H,Sq,D], k/v [H,Sk,D], mask [Sq,Sk] bool."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(mask)[None, None]).numpy()[0]


# ----------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_matches_torch_rms_norm():
    x = RNG.standard_normal((37, 128)) * 3.0
    w = 1.0 + 0.1 * RNG.standard_normal(128)
    for eps in (1e-6, 0.5):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps).numpy()
        np.testing.assert_allclose(oracle.rmsnorm(x, w, eps), ref, rtol=1e-13, atol=1e-13)


def test_rmsnorm_constant_vector_closed_form():
    c, eps = -2.5, 1e-6
    w = 1.0 + 0.1 * RNG.standard_normal(128)
    y = oracle.rmsnorm(np.full((1, 128), c), w, eps)[0]
    np.testing.assert_allclose(y, w * c / math.sqrt(c * c + eps), rtol=1e-14)


def test_rmsnorm_scale_invariant_without_eps():
    x = RNG.standard_normal((5, 64))
    w = RNG.standard_normal(64)
    np.testing.assert_allclose(oracle.rmsnorm(7.0 * x, w, 0.0), oracle.rmsnorm(x, w, 0.0), rtol=1e-13)


# ----------------------------------------------------------------------------- partial RoPE
def _rope_complex(x, pos, R, base):
    """RoFormer's rotary embedding in complex form: pair (x_2i, x_2i+1) as x_2i + i x_2i+1, multiplied by
    exp(i * pos * theta_i), theta_i = base^(-2i/R), for the leading R dims."""
    y = x.copy()
    i = np.arange(R // 2)
    theta = base ** (-2.0 * i / R)
    z = x[..., 0:R:2] + 1j * x[..., 1:R:2]
    z = z * np.exp(1j * np.asarray(pos)[..., None] * theta)
    y[..., 0:R:2] = z.real
    y[..., 1:R:2] = z.imag
    return y


@pytest.mark.parametrize("R,base", [(42, 1e4), (42, 1e7), (128, 1e4), (6, 10.0)])
def test_rope_matches_complex_form(R, base):
    x = RNG.standard_normal((9, 128))
    pos = np.array([0, 1, 2, 127, 128, 4095, 16383, 262143, 262144])
    np.testing.assert_allclose(oracle.rope(x, pos, R, base), _rope_complex(x, pos, R, base), rtol=0, atol=1e-9)


def test_rope_leaves_trailing_dims_and_position_zero_alone():
    x = RNG.standard_normal((3, 128))
    y = oracle.rope(x, np.array([5, 77, 262144]), 42, 1e4)
    np.testing.assert_array_equal(y[:, 42:], x[:, 42:])
    np.testing.assert_array_equal(oracle.rope(x, 0, 42, 1e4), x)


def test_rope_preserves_norm_and_is_relative():
    q = RNG.standard_normal(128)
    k = RNG.standard_normal(128)
    for R in (42, 128):
        a = oracle.rope(q[None], 1000, R, 1e4)[0]
        assert abs(np.linalg.norm(a) - np.linalg.norm(q)) < 1e-12
        d1 = oracle.rope(q[None], 1000, R, 1e4)[0] @ oracle.rope(k[None], 990, R, 1e4)[0]
        d2 = oracle.rope(q[None], 5010, R, 1e4)[0] @ oracle.rope(k[None], 5000, R, 1e4)[0]
        assert abs(d1 - d2) < 1e-9


def test_rope_rotation_direction_at_position_one():
    # e_0 rotated by +theta_0 = +1 rad lands at (cos 1, sin 1) in dims (0, 1): counter-clockwise.
    e0 = np.zeros((1, 128))
    e0[0, 0] = 1.0
    y = oracle.rope(e0, 1, 42, 1e4)[0]
    assert abs(y[0] - math.cos(1.0)) < 1e-15 and abs(y[1] - math.sin(1.0)) < 1e-15


# ----------------------------------------------------------------------------- attention
def _band(Sq, Sk, qpos, kpos, window):
    m = (kpos[None, :] <= qpos[:, None]) & (kpos[None, :] >= 0)
    if window:
        m &= (qpos[:, None] - kpos[None, :]) < window
    return m


@pytest.mark.parametrize("window", [None, 1, 4, 128])
def test_attend_matches_torch_sdpa(window):
    S, D = 300, 128
    q = RNG.standard_normal((S, D))
    k = RNG.standard_normal((S, D))
    v = RNG.standard_normal((S, D))
    pos = np.arange(S)
    out = oracle.attend(q, pos, k, v, pos, window)
    ref = _sdpa(q[None], k[None], v[None], _band(S, S, pos, pos, window))[0]
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_attend_gqa_matches_sdpa_with_repeated_kv():
    B, S, Hq, Hkv, D = 1, 200, 8, 2, 32
    G = Hq // Hkv
    q = RNG.standard_normal((B, S, Hq, D))
    k = RNG.standard_normal((B, S, Hkv, D))
    v = RNG.standard_normal((B, S, Hkv, D))
    w = np.ones(D)
    o = oracle.prefill_layer(q, k, v, None, w, w, window=None, rotary_dims=0, base=1e4, eps=0.0)
    qh = oracle.rmsnorm(q, w, 0.0)[0].transpose(1, 0, 2)
    # keys enter attention in the bf16 cache format
    kb = oracle.bf16_to_f64(oracle.round_bf16(oracle.rmsnorm(k, w, 0.0)))
    kh = np.repeat(kb[0].transpose(1, 0, 2), G, axis=0)
    vh = np.repeat(v[0].transpose(1, 0, 2), G, axis=0)
    pos = np.arange(S)
    ref = _sdpa(qh, kh, vh, _band(S, S, pos, pos, None)).transpose(1, 0, 2)
    np.testing.assert_allclose(o[0], ref, rtol=1e-11, atol=1e-12)


def test_zero_query_gives_mean_of_visible_values_page_window_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "window_example.json")))
    W, S, D = ex["window"], 7, 16
    v = RNG.standard_normal((S, D))
    k = RNG.standard_normal((S, D))
    pos = np.arange(S)
    out = oracle.attend(np.zeros((S, D)), pos, k, v, pos, W)
    i = ex["query_index"]
    np.testing.assert_allclose(out[i], v[ex["visible_key_indices"]].mean(axis=0), rtol=1e-14)
    for i in range(S):
        lo = max(0, i - W + 1)
        np.testing.assert_allclose(out[i], v[lo:i + 1].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_identical_keys_give_uniform_weights():
    S, D = 50, 32
    k = np.tile(RNG.standard_normal(D), (S, 1))
    v = RNG.standard_normal((S, D))
    q = RNG.standard_normal((S, D))
    pos = np.arange(S)
    out = oracle.attend(q, pos, k, v, pos, None)
    for i in range(S):
        np.testing.assert_allclose(out[i], v[:i + 1].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_window_one_is_gated_value():
    S, D = 20, 16
    q, k, v, g = (RNG.standard_normal((S, D)) for _ in range(4))
    pos = np.arange(S)
    out = oracle.attend(q, pos, k, v, pos, 1, g)
    np.testing.assert_allclose(out, v / (1.0 + np.exp(-g)), rtol=1e-14)


def test_window_at_least_sequence_equals_global():
    S, D = 64, 32
    q, k, v = (RNG.standard_normal((S, D)) for _ in range(3))
    pos = np.arange(S)
    np.testing.assert_array_equal(oracle.attend(q, pos, k, v, pos, S), oracle.attend(q, pos, k, v, pos, None))
    np.testing.assert_array_equal(oracle.attend(q, pos, k, v, pos, 10 * S), oracle.attend(q, pos, k, v, pos, None))


def test_gate_plus_infinity_is_ungated_minus_infinity_is_zero():
    S, D = 40, 16
    q, k, v = (RNG.standard_normal((S, D)) for _ in range(3))
    pos = np.arange(S)
    un = oracle.attend(q, pos, k, v, pos, 8)
    np.testing.assert_array_equal(oracle.attend(q, pos, k, v, pos, 8, np.full((S, D), np.inf)), un)
    assert np.all(oracle.attend(q, pos, k, v, pos, 8, np.full((S, D), -np.inf)) == 0.0)


def test_gate_matches_page_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "gate_example.json")))
    a = np.array(ex["attention_output"])
    s = np.array(ex["sigmoid_of_gate"])
    g = np.log(s / (1.0 - s))                       # logits whose sigmoid is the page's gate
    # window 1: the output is the query's own value, gated -- so v = the page's attention output
    out = oracle.attend(np.zeros((1, 3)), [0], np.zeros((1, 3)), a[None], [0], 1, g[None])[0]
    np.testing.assert_allclose(out, ex["gated_output"], rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------- cache, decode, chunks
def _small_problem(seed, L, B, S, Hq, Hkv, D):
    r = np.random.default_rng(seed)
    return (r.standard_normal((L, B, S, Hq, D)), r.standard_normal((L, B, S, Hkv, D)),
            r.standard_normal((L, B, S, Hkv, D)), r.standard_normal((L, B, S, Hq, D)),
            1 + 0.1 * r.standard_normal((L, D)), 1 + 0.1 * r.standard_normal((L, D)))


def test_decode_equals_prefill_at_every_position():
    L, B, S, Hq, Hkv, D, W, R = 3, 2, 140, 4, 2, 16, 8, 6
    glob = [2]
    q, k, v, g, wq, wk = _small_problem(7, L, B, S, Hq, Hkv, D)
    kw = dict(rotary_dims=R, base=1e4, eps=1e-6)
    ref = [oracle.prefill_layer(q[l], k[l], v[l], None if (l + 1) in glob else g[l], wq[l], wk[l],
                                window=None if (l + 1) in glob else W, **kw) for l in range(L)]
    cache = oracle.OracleCache(L, glob, B, Hkv, D, W)
    for t in range(S):
        o = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], wq, wk, [t] * B, cache, **kw)
        for l in range(L):
            np.testing.assert_allclose(o[l], ref[l][:, t], rtol=0, atol=1e-12)


def test_chunked_prefill_equals_one_shot():
    L, B, S, Hq, Hkv, D, W, R = 2, 1, 300, 4, 1, 16, 32, 6
    glob = [2]
    q, k, v, g, wq, wk = _small_problem(9, L, B, S, Hq, Hkv, D)
    kw = dict(rotary_dims=R, base=1e7, eps=1e-6)
    cache = oracle.OracleCache(L, glob, B, Hkv, D, W)
    for l in range(L):
        gl = (l + 1) in glob
        one = oracle.prefill_layer(q[l], k[l], v[l], None if gl else g[l], wq[l], wk[l], window=None if gl else W, **kw)
        parts = []
        for c0, c1 in ((0, 100), (100, 131), (131, 300)):
            parts.append(oracle.prefill_layer(q[l][:, c0:c1], k[l][:, c0:c1], v[l][:, c0:c1],
                                              None if gl else g[l][:, c0:c1], wq[l], wk[l], window=None if gl else W,
                                              pos0=c0, cache=cache, layer=l + 1, **kw))
        np.testing.assert_allclose(np.concatenate(parts, axis=1), one, rtol=0, atol=1e-12)


def test_prefill_keys_are_read_in_bf16_cache_form():
    """Attention over keys reads k_hat as stored in the bf16 cache: rounding k_hat first changes nothing,
    perturbing it by less than half a bf16 ulp changes nothing either."""
    B, S, Hq, Hkv, D = 1, 50, 2, 1, 16
    r = np.random.default_rng(5)
    q, k, v = r.standard_normal((B, S, Hq, D)), r.standard_normal((B, S, Hkv, D)), r.standard_normal((B, S, Hkv, D))
    w = np.ones(D)
    kw = dict(window=None, rotary_dims=4, base=1e4, eps=1e-6)
    o = oracle.prefill_layer(q, k, v, None, w, w, **kw)
    pos = np.arange(S)
    qh = oracle.qk_prologue(q, pos[None, :, None], w, 1e-6, 4, 1e4)[0]
    kh = oracle.qk_prologue(k, pos[None, :, None], w, 1e-6, 4, 1e4)[0, :, 0]
    kb = oracle.bf16_to_f64(oracle.round_bf16(kh))
    for h in range(Hq):
        np.testing.assert_allclose(o[0, :, h], oracle.attend(qh[:, h], pos, kb, v[0, :, 0], pos, None), rtol=1e-12, atol=1e-13)


def _bf16_exact(a):
    """Round float64 data to bf16 values (torch's conversion) and return them as float64 (exact inputs)."""
    return torch.from_numpy(np.asarray(a, dtype=np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def _torch_bits(x):
    """bf16 bit patterns of float64 data through torch's own conversion (not the oracle's rounding)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _khat_independent(k, w, eps, R, base):
    """k_hat of raw rows k [B,S,H,D] at positions 0..S-1 without the oracle: torch's rms_norm in float64, then
    RoFormer's complex form of the rotation."""
    B, S, H, D = k.shape
    y = torch.nn.functional.rms_norm(torch.from_numpy(k), (D,), torch.from_numpy(np.asarray(w, dtype=np.float64)),
                                     eps).numpy()
    return _rope_complex(y, np.arange(S)[None, :, None], R, base)


def _image_problem(seed, B, S, Hq, Hkv, D):
    r = np.random.default_rng(seed)
    q = _bf16_exact(r.standard_normal((B, S, Hq, D)))
    k = _bf16_exact(r.standard_normal((B, S, Hkv, D)))
    v = _bf16_exact(r.standard_normal((B, S, Hkv, D)))
    g = _bf16_exact(r.standard_normal((B, S, Hq, D)))
    w = _bf16_exact(1 + 0.1 * r.standard_normal(D))
    return q, k, v, g, w


def test_ring_image_holds_last_window_positions_by_slot():
    """The SWA ring (jaehun.me, "Why the KV Cache Shrinks by 6.4x": only the last W keys are kept): slot s of
    sequence b, KV head h holds position p = the one of the last W with p mod W = s, its k_hat rounded to bf16 and
    its v bits unchanged; k_hat comes from torch's rms_norm and the complex form of RoPE, not from the oracle.
    Two sequences and two KV heads with different data catch a swapped (b, h); prefill in chunks catches an
    off-by-one slot."""
    B, S, Hq, Hkv, D, W, R, eps, base = 2, 300, 4, 2, 16, 128, 6, 1e-6, 1e4
    q, k, v, g, w = _image_problem(3, B, S, Hq, Hkv, D)
    cache = oracle.OracleCache(1, [], B, Hkv, D, W)
    for c0, c1 in ((0, 90), (90, 91), (91, 300)):
        oracle.prefill_layer(q[:, c0:c1], k[:, c0:c1], v[:, c0:c1], g[:, c0:c1], w, w, window=W, rotary_dims=R,
                             base=base, eps=eps, pos0=c0, cache=cache, layer=1)
    K, V, P = cache.ring_image(1)
    kref = _torch_bits(_khat_independent(k, w, eps, R, base))
    vbits = _torch_bits(v)
    for b in range(B):
        assert sorted(P[b]) == list(range(S - W, S))
        for s in range(W):
            p = P[b, s]
            assert p % W == s
            for h in range(Hkv):
                np.testing.assert_array_equal(V[b, h, s], vbits[b, p, h])
                np.testing.assert_array_equal(K[b, h, s], kref[b, p, h])
    # fewer positions than slots: the others stay empty (position -1, zero bits)
    short = oracle.OracleCache(1, [], B, Hkv, D, W)
    oracle.prefill_layer(q[:, :5], k[:, :5], v[:, :5], g[:, :5], w, w, window=W, rotary_dims=R, base=base, eps=eps,
                         cache=short, layer=1)
    K, V, P = short.ring_image(1)
    assert np.all(P[:, :5] == np.arange(5)) and np.all(P[:, 5:] == -1)
    assert not K[:, :, 5:].any() and not V[:, :, 5:].any()
    np.testing.assert_array_equal(K[:, :, :5], kref[:, :5].transpose(0, 2, 1, 3))


def test_global_image_holds_every_position_by_row():
    """A global layer's cache keeps every position: row p of sequence b, KV head h holds k_hat at position p
    (rounded to bf16) and v unchanged, whether the rows were written by one prefill or by chunks (jaehun.me, "Why
    the KV Cache Shrinks by 6.4x": K and V of every earlier token, 2 bytes per element).  k_hat comes from torch's
    rms_norm and the complex form of RoPE, not from the oracle."""
    B, S, Hq, Hkv, D, R, eps, base = 2, 70, 4, 2, 16, 6, 1e-6, 1e7
    q, k, v, _, w = _image_problem(4, B, S, Hq, Hkv, D)
    kref = _torch_bits(_khat_independent(k, w, eps, R, base)).transpose(0, 2, 1, 3)   # [B][Hkv][S][D]
    vref = _torch_bits(v).transpose(0, 2, 1, 3)
    for chunks in (((0, S),), ((0, 1), (1, 33), (33, 70))):
        cache = oracle.OracleCache(2, [2], B, Hkv, D, 16)
        for c0, c1 in chunks:
            oracle.prefill_layer(q[:, c0:c1], k[:, c0:c1], v[:, c0:c1], None, w, w, window=None, rotary_dims=R,
                                 base=base, eps=eps, pos0=c0, cache=cache, layer=2)
        K, V = cache.global_image(2)
        assert K.shape == (B, Hkv, S, D)
        np.testing.assert_array_equal(K, kref)
        np.testing.assert_array_equal(V, vref)


# ----------------------------------------------------------------------------- pages' closed forms
def test_kv_footprint_matches_page(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "kv_footprint.json")))
    L = ex["n_layers"]
    kw = dict(n_layers=L, n_kv_heads=ex["n_kv_heads"], head_dim=ex["head_dim"], window=ex["window"],
              elem_bytes=ex["bytes_per_elem"])
    all_global = list(range(1, L + 1))
    T = ex["tokens_256k"]
    full = oracle.kv_footprint_bytes(T, global_layer_ids=all_global, **kw)
    hyb = oracle.kv_footprint_bytes(T, **kw)
    assert full // T == ex["full_attention_bytes_per_token"]
    # per-token growth once every SWA ring is full
    assert oracle.kv_footprint_bytes(T + 1, **kw) - hyb == ex["hybrid_bytes_per_token"]
    assert round(full / 2**30, 1) == ex["full_attention_gib_256k"]
    assert round(hyb / 2**30, 1) == ex["hybrid_gib_256k"]
    assert round(round(full / 2**30, 1) / round(hyb / 2**30, 1), 1) == ex["reduction"]


def test_layer_schedule_matches_page(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "layer_schedule.json")))
    assert oracle.global_layers(ex["n_layers"]) == ex["global_layers_1based"]
    n_glob = sum(oracle.is_global_layer(l) for l in range(1, ex["n_layers"] + 1))
    assert (ex["n_layers"] - n_glob, n_glob) == (ex["n_swa"], ex["n_global"])


def test_bf16_rounding_ties_to_even_and_matches_torch():
    cases = {1.0: 0x3F80, 1.0 + 2**-8: 0x3F80, 1.0 + 3 * 2**-8: 0x3F82, -2.0: 0xC000, 0.0: 0, 3.0 + 2**-7: 0x4040}
    for x, bits in cases.items():
        assert int(oracle.round_bf16(np.array([x]))[0]) == bits, x
    x = RNG.standard_normal(10000).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.round_bf16(x), ref)
    np.testing.assert_array_equal(oracle.bf16_to_f64(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


# ------------------------------------------------------------------------------------------ projections
def test_linear_is_x_times_w_transposed_brute_force():
    """y = x W^T with W stored out x in: against explicit fsum loops, the identity and one-hot rows."""
    x = RNG.standard_normal((3, 5))
    w = RNG.standard_normal((4, 5))
    y = oracle.linear(x, w)
    for t in range(3):
        for n in range(4):
            assert y[t, n] == pytest.approx(math.fsum(x[t, k] * w[n, k] for k in range(5)), rel=1e-14, abs=1e-14)
    np.testing.assert_array_equal(oracle.linear(x, np.eye(5)), x)
    onehot = np.zeros((1, 5)); onehot[0, 2] = 1.0
    np.testing.assert_array_equal(oracle.linear(onehot, w)[0], w[:, 2])


@pytest.mark.parametrize("gated", [True, False])
def test_attention_layer_with_identity_projections_is_the_core(gated):
    """With every projection the identity (d_model = Hq*D, one query head per KV head), the layer is the
    attention of prefill_layer on h itself, its output rounded to bf16 (the bf16 hand-off between ops)."""
    import synth
    B, S, H, D = 1, 40, 2, 128
    h = synth.normal_bf16(7, 1, synth.TENSOR_H, (B, S, H * D))
    eye = synth.f64_to_bf16_bits(np.eye(H * D))
    wn = synth.norm_weight_bf16(7, 1, synth.TENSOR_WQ, D)
    y = oracle.attention_layer(h, eye, eye, eye, eye if gated else None, eye, wn, wn, Hq=H, Hkv=H,
                               window=16 if gated else None, rotary_dims=42, base=1e4, eps=1e-6)
    hq = h.reshape(B, S, H, D)
    o = oracle.prefill_layer(hq, hq, hq, hq if gated else None, wn, wn, window=16 if gated else None, rotary_dims=42,
                             base=1e4, eps=1e-6)
    np.testing.assert_array_equal(y, oracle.bf16_to_f64(oracle.round_bf16(o)).reshape(B, S, H * D))


# ------------------------------------------------------------------------------------------ FP8 E4M3
def test_e4m3_codes_of_defining_values():
    """OCP E4M3: bias 7, 3 mantissa bits, largest finite 448 (0x7E), smallest subnormal 2^-9 (0x01)."""
    cases = {0.0: 0x00, 1.0: 0x38, -1.0: 0xB8, 448.0: 0x7E, -448.0: 0xFE, 2.0 ** -9: 0x01, 2.0 ** -6: 0x08,
             1.75: 0x3E, 240.0: 0x77, 0.5: 0x30,
             1.0 + 1 / 16: 0x38,          # tie -> even mantissa (0)
             1.0 + 3 / 16: 0x3A,          # tie -> even mantissa (2)
             3 * 2.0 ** -10: 0x02,        # subnormal tie 1.5 -> 2
             2.0 ** -10: 0x00,            # half the smallest subnormal: tie -> 0
             1000.0: 0x7E, -1e6: 0xFE,    # saturation
             15.5: 0x58,                  # 15.5 = 2^3 * 1.9375: mantissa tie 7.5 -> 8, carries into 16 = 2^4
             56.0: 0x66}                  # 56 = 2^5 * 1.75
    for v, code in cases.items():
        assert int(oracle.e4m3_encode(np.array([v]))[0]) == code, v
    for code in range(256):
        if code & 0x7F == 0x7F:
            continue                       # NaN codes
        val = oracle.e4m3_decode(np.array([code]))[0]
        back = int(oracle.e4m3_encode(np.array([val]))[0])
        assert back == code or (val == 0.0 and back & 0x7F == 0), code


def test_e4m3_matches_torch_float8_in_range():
    """Against torch's float8_e4m3fn cast (nearest-even) for finite values inside +-448."""
    v = np.concatenate([RNG.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)]).astype(np.float32)
    v = v[np.abs(v) < 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(v), ref)


def test_fp8_delayed_scaling_lags_by_one_call():
    """Scales start at 1, then follow 448 / max(amax history) of the calls before (history of 2 here)."""
    f = oracle.Fp8DelayedLinear(K=8, N=2, history=2)
    w = np.full((2, 8), 0.5)
    for amax_x, expect_scale_x in ((2.0, 1.0), (8.0, 448.0 / 2.0), (1.0, 448.0 / 8.0), (1.0, 448.0 / 8.0)):
        x = np.zeros((1, 8)); x[0, 3] = amax_x
        assert float(f.scale[0]) == np.float32(expect_scale_x)
        y, cx, cw = f(x, w)
        assert float(f.scale[1]) == np.float32(448.0 / 0.5)
    # after the fourth call the history holds {1, 1}: the next scale is 448
    assert float(f.scale[0]) == 448.0
    # with the scale 448/8 = 56 in use, x = 1 is coded as 56 -> E4M3(56) = 0x66 and dequantised exactly
    f2 = oracle.Fp8DelayedLinear(K=8, N=1, history=4)
    f2(np.full((1, 8), 8.0), np.full((1, 8), 1.0))
    y, cx, cw = f2(np.full((1, 8), 1.0), np.full((1, 8), 1.0))
    assert int(cx[0, 0]) == 0x66 and y[0, 0] == pytest.approx(8.0)


def _e4m3_grid(rng, shape, e_lo, e_hi, signed=True):
    """Random values (1 + m/8) 2^e, e in [e_lo, e_hi]: normal E4M3 values, exact in bf16 too."""
    m = rng.integers(0, 8, size=shape)
    e = rng.integers(e_lo, e_hi + 1, size=shape)
    v = (1.0 + m / 8.0) * np.exp2(e)
    if signed:
        v = v * rng.choice([-1.0, 1.0], size=shape)
    return synth.f64_to_bf16_bits(v)


@pytest.mark.parametrize("gated", [True, False])
def test_fp8_layer_equals_bf16_layer_when_operands_are_e4m3_exact(gated):
    """First call (all scales 1) with every quantised operand exactly representable in E4M3: h and the q/k/w_o
    weights on the E4M3 grid, W_v picking columns of h that are constant over the tokens (so v, the attention
    average and o are that constant, whatever the weights), W_g = 64 x picking positive columns (sigmoid(g) rounds
    to 1).  Then quantisation changes nothing and the FP8 layer equals the bf16 layer exactly; afterwards each
    quantised tensor's scale is 448 / its max |v|, and a global layer leaves W_g's state alone."""
    rng = np.random.default_rng(11)
    B, S, Hq, Hkv, D, dm = 1, 24, 2, 1, 128, 256
    hv = oracle.bf16_to_f64(_e4m3_grid(rng, (B, S, dm), -1, 1, signed=False))
    cols = rng.choice(dm, size=Hkv * D, replace=False)
    hv[:, :, cols] = hv[:, :1, cols]                        # constant over the tokens
    h = synth.f64_to_bf16_bits(hv)
    onehot = np.zeros((Hkv * D, dm))
    onehot[np.arange(Hkv * D), cols] = 1.0
    w_q = _e4m3_grid(rng, (Hq * D, dm), -6, -3)
    w_k = _e4m3_grid(rng, (Hkv * D, dm), -6, -3)
    w_v = synth.f64_to_bf16_bits(onehot)
    w_g = synth.f64_to_bf16_bits(64.0 * np.eye(Hq * D, dm)) if gated else None
    w_o = _e4m3_grid(rng, (dm, Hq * D), -6, -3)
    wn = synth.norm_weight_bf16(7, 1, synth.TENSOR_WQ, D)
    kw = dict(Hq=Hq, Hkv=Hkv, window=4 if gated else None, rotary_dims=42, base=1e4, eps=1e-6)
    st = oracle.Fp8DelayedScaling(7, history=16)
    y8 = oracle.attention_layer_fp8(h, w_q, w_k, w_v, w_g, w_o, wn, wn, st, **kw)
    y = oracle.attention_layer(h, w_q, w_k, w_v, w_g, w_o, wn, wn, **kw)
    np.testing.assert_array_equal(y8, y)
    o_max = np.max(np.abs(hv[0, 0, cols]))                 # o = v = the constant columns (each head repeats them)
    for name, v in (("h", hv), ("w_q", w_q), ("w_k", w_k), ("w_v", onehot), ("w_g", w_g), ("o", o_max), ("w_o", w_o)):
        t = oracle.FP8_LAYER_TENSORS.index(name)
        if v is None:
            assert st.scale[t] == 1.0 and not st.hist[t].any()
            continue
        m = np.float32(np.max(np.abs(oracle.bf16_to_f64(v) if np.asarray(v).dtype == np.uint16 else v)))
        assert st.scale[t] == np.float32(448.0) / m, name


@pytest.mark.parametrize("gated", [True, False])
def test_fp8_layer_tracks_bf16_layer_within_e4m3_precision(gated):
    """Random operands over three calls: E4M3 keeps 3 mantissa bits, so each quantised operand is off by at most
    2^-4 relative (normals) and the layer output by a few percent rms, at every call (scales 1, then fitted).
    A dropped or misapplied dequantisation factor is off by the scale itself (factors of 10-10^4 here)."""
    B, S, Hq, Hkv, D, dm = 1, 48, 2, 1, 128, 256
    h = synth.normal_bf16(5, 1, synth.TENSOR_H, (B, S, dm))
    def wt(t, n, k):
        return synth.f64_to_bf16_bits(oracle.bf16_to_f64(synth.normal_bf16(5, 1, t, (n, k))) / np.sqrt(k))
    w_q, w_k, w_v = wt(synth.TENSOR_PQ, Hq * D, dm), wt(synth.TENSOR_PK, Hkv * D, dm), wt(synth.TENSOR_PV, Hkv * D, dm)
    w_g = wt(synth.TENSOR_PG, Hq * D, dm) if gated else None
    w_o = wt(synth.TENSOR_PO, dm, Hq * D)
    wn = synth.norm_weight_bf16(5, 1, synth.TENSOR_WQ, D)
    kw = dict(Hq=Hq, Hkv=Hkv, window=16 if gated else None, rotary_dims=42, base=1e4, eps=1e-6)
    y = oracle.attention_layer(h, w_q, w_k, w_v, w_g, w_o, wn, wn, **kw)
    st = oracle.Fp8DelayedScaling(7, history=16)
    for call in range(3):
        y8 = oracle.attention_layer_fp8(h, w_q, w_k, w_v, w_g, w_o, wn, wn, st, **kw)
        rel = np.sqrt(np.mean((y8 - y) ** 2) / np.mean(y ** 2))
        assert 1e-4 < rel < 0.15, (call, rel)


# ------------------------------------------------------------------------------------------ backward
def _bwd_problem(seed, B, S, Hq, Hkv, D=128, gated=True):
    q = synth.normal_bf16(seed, 1, synth.TENSOR_Q, (B, S, Hq, D))
    k = synth.normal_bf16(seed, 1, synth.TENSOR_K, (B, S, Hkv, D))
    v = synth.normal_bf16(seed, 1, synth.TENSOR_V, (B, S, Hkv, D))
    g = synth.normal_bf16(seed, 1, synth.TENSOR_GATE, (B, S, Hq, D)) if gated else None
    wq = synth.norm_weight_bf16(seed, 1, synth.TENSOR_WQ, D)
    wk = synth.norm_weight_bf16(seed, 1, synth.TENSOR_WK, D)
    do = np.random.default_rng(seed).standard_normal((B, S, Hq, D))
    return q, k, v, g, wq, wk, do


def _torch_layer(q, k, v, g, wq, wk, *, window, R, base, eps):
    """The forward from library routines: torch's rms_norm, RoPE as a complex product (RoFormer), masked
    scaled_dot_product_attention, sigmoid gate; k_hat rounded to bf16 with its gradient passed straight through."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    pos = torch.arange(S, dtype=torch.float64)
    inv = base ** (-torch.arange(0, R, 2, dtype=torch.float64) / R)
    rot = torch.polar(torch.ones(S, R // 2, dtype=torch.float64), pos[:, None] * inv[None, :])   # [S, R/2]

    def rope(x):
        xr = torch.view_as_complex(x[..., :R].reshape(*x.shape[:-1], R // 2, 2).contiguous())
        xr = torch.view_as_real(xr * rot[None, :, None, :]).reshape(*x.shape[:-1], R)
        return torch.cat([xr, x[..., R:]], dim=-1)

    qh = rope(torch.nn.functional.rms_norm(q, (D,), wq, eps))
    kh = rope(torch.nn.functional.rms_norm(k, (D,), wk, eps))
    kh = kh + (kh.to(torch.bfloat16).to(torch.float64) - kh).detach()
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    vis = j <= i
    if window:
        vis = vis & (i - j < window)
    G = Hq // Hkv
    kr = kh.repeat_interleave(G, dim=2)
    vr = v.repeat_interleave(G, dim=2)
    a = torch.nn.functional.scaled_dot_product_attention(qh.transpose(1, 2), kr.transpose(1, 2), vr.transpose(1, 2),
                                                         attn_mask=vis)
    a = a.transpose(1, 2)
    return a * torch.sigmoid(g) if g is not None else a


@pytest.mark.parametrize("gated,window,B,S,Hq,Hkv", [(True, 8, 1, 24, 4, 1), (False, None, 2, 17, 4, 2),
                                                     (True, 5, 1, 19, 2, 2)])
def test_backward_matches_torch_autograd(gated, window, B, S, Hq, Hkv):
    """The oracle's hand-derived gradients against torch autograd (float64) through the forward built from
    library routines: every input, and the norm weights."""
    q, k, v, g, wq, wk, do = _bwd_problem(3, B, S, Hq, Hkv, gated=gated)
    ref = oracle.prefill_layer_backward(q, k, v, g, wq, wk, do, window=window, rotary_dims=42, base=1e4, eps=1e-6)
    t = {n: torch.tensor(oracle.bf16_to_f64(x), requires_grad=True)
         for n, x in (("q", q), ("k", k), ("v", v), ("wq", wq), ("wk", wk)) + ((("g", g),) if gated else ())}
    out = _torch_layer(t["q"], t["k"], t["v"], t.get("g"), t["wq"], t["wk"], window=window, R=42, base=1e4, eps=1e-6)
    np.testing.assert_allclose(out.detach().numpy(), ref["out"], rtol=0, atol=1e-12)
    (out * torch.tensor(do)).sum().backward()
    for n, r in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("wq", "dwq"), ("wk", "dwk")) + ((("g", "dgate"),) if gated else ()):
        np.testing.assert_allclose(t[n].grad.numpy(), ref[r], rtol=1e-9, atol=1e-11, err_msg=n)


def test_backward_matches_finite_differences():
    """Central differences of the oracle's own forward (prefill_layer) on sampled elements of q, v, g and w_q (k
    and w_k feed the bf16-rounded k_hat, whose true derivative is a step function: autograd pins those)."""
    B, S, Hq, Hkv, D = 1, 10, 2, 1, 128
    q, k, v, g, wq, wk, do = _bwd_problem(4, B, S, Hq, Hkv)
    kw = dict(window=4, rotary_dims=42, base=1e4, eps=1e-6)
    ref = oracle.prefill_layer_backward(q, k, v, g, wq, wk, do, **kw)
    f = {n: oracle.bf16_to_f64(x) for n, x in (("q", q), ("k", k), ("v", v), ("g", g), ("wq", wq), ("wk", wk))}
    rng = np.random.default_rng(9)

    def loss(**over):
        a = {**f, **over}
        return float(np.sum(oracle.prefill_layer(a["q"], a["k"], a["v"], a["g"], a["wq"], a["wk"], **kw) * do))

    h = 1e-5
    for n, r in (("q", "dq"), ("v", "dv"), ("g", "dgate"), ("wq", "dwq")):
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in f[n].shape)
            xp, xm = f[n].copy(), f[n].copy()
            xp[idx] += h
            xm[idx] -= h
            fd = (loss(**{n: xp}) - loss(**{n: xm})) / (2 * h)
            assert abs(fd - ref[r][idx]) <= 1e-6 * max(1.0, abs(fd)), (n, idx, fd, ref[r][idx])


def test_backward_window_one_and_closed_gate():
    """W = 1: each query sees only itself, p = 1, so the scores carry no gradient (dq = dk = dw = 0) and
    dv = sum over the group's heads of dout (.) sigmoid(g), dg = dout (.) v (.) sigmoid'(g).
    g = -inf: the output is identically zero, so every gradient is zero."""
    B, S, Hq, Hkv, D = 1, 9, 2, 1, 128
    q, k, v, g, wq, wk, do = _bwd_problem(5, B, S, Hq, Hkv)
    r = oracle.prefill_layer_backward(q, k, v, g, wq, wk, do, window=1, rotary_dims=42, base=1e4, eps=1e-6)
    for n in ("dq", "dk", "dwq", "dwk"):
        assert np.abs(r[n]).max() < 1e-13, n
    sg = 1.0 / (1.0 + np.exp(-oracle.bf16_to_f64(g)))
    vf = oracle.bf16_to_f64(v)
    np.testing.assert_allclose(r["dv"][:, :, 0], (do * sg).sum(axis=2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["dgate"], do * vf[:, :, [0, 0]] * sg * (1 - sg), rtol=1e-12, atol=1e-13)
    gneg = synth.f64_to_bf16_bits(np.full(oracle.bf16_to_f64(g).shape, -np.inf))
    z = oracle.prefill_layer_backward(q, k, v, gneg, wq, wk, do, window=4, rotary_dims=42, base=1e4, eps=1e-6)
    for n in ("dq", "dk", "dv", "dgate", "dwq", "dwk"):
        assert not np.any(z[n]), n


def test_backward_bf16_dA_variant():
    """dA_bf16 rounds dA = dout (.) sigmoid(g) to bf16 before dp and dv.  W = 1 (p = 1): dv is then exactly the sum
    over the group's heads of the rounded dA; with the exact Delta (the row sum of p dp, same dp) ds is still zero,
    so dq = dk = 0; the gate's gradient does not go through dA and is unchanged."""
    B, S, Hq, Hkv = 1, 9, 2, 1
    q, k, v, g, wq, wk, do = _bwd_problem(5, B, S, Hq, Hkv)
    kw = dict(window=1, rotary_dims=42, base=1e4, eps=1e-6)
    r = oracle.prefill_layer_backward(q, k, v, g, wq, wk, do, dA_bf16=True, **kw)
    exact = oracle.prefill_layer_backward(q, k, v, g, wq, wk, do, **kw)
    sg = 1.0 / (1.0 + np.exp(-oracle.bf16_to_f64(g)))
    dA16 = oracle.bf16_to_f64(oracle.round_bf16(do * sg))
    np.testing.assert_allclose(r["dv"][:, :, 0], dA16.sum(axis=2), rtol=1e-12, atol=1e-13)
    assert np.abs(r["dv"] - exact["dv"]).max() > 0          # the rounding is applied
    for n in ("dq", "dk", "dwq", "dwk"):
        assert np.abs(r[n]).max() < 1e-13, n
    np.testing.assert_array_equal(r["dgate"], exact["dgate"])


@pytest.mark.parametrize("window", [7, None])
def test_backward_rows_equals_full_backward(window):
    """The row-sampled backward (row blocks, one KV head) against the whole-layer backward at a small size, for
    sampled query and key rows spanning several blocks, both with the exact Delta and with Delta from the bf16
    output."""
    B, S, Hq, Hkv = 2, 45, 4, 2
    q, k, v, g, wq, wk, do = _bwd_problem(6, B, S, Hq, Hkv, gated=window is not None)
    kw = dict(window=window, rotary_dims=42, base=1e4, eps=1e-6)
    full = oracle.prefill_layer_backward(q, k, v, g, wq, wk, do, **kw)
    full16 = oracle.prefill_layer_backward(q, k, v, g, wq, wk, do, delta_from_bf16_out=True, **kw)
    qr, kr = np.array([0, 3, 16, 31, 44]), np.array([0, 5, 15, 16, 40, 44])
    r = oracle.prefill_layer_backward_rows(q, k, v, g, wq, wk, do, b=1, kv_head=1, query_rows=qr, key_rows=kr,
                                           block=16, **kw)
    np.testing.assert_allclose(r["dq"], full["dq"][1][qr][:, 2:4], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dq_d16"], full16["dq"][1][qr][:, 2:4], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dk"], full["dk"][1][kr][:, 1], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dk_d16"], full16["dk"][1][kr][:, 1], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dv"], full["dv"][1][kr][:, 1], rtol=1e-10, atol=1e-12)
    if window is not None:
        np.testing.assert_allclose(r["dgate"], full["dgate"][1][qr][:, 2:4], rtol=1e-10, atol=1e-12)
