"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the same seeded inputs.

Bar: |gpu_bf16 - oracle_fp64| <= 1e-2 per element and <= 1e-3 on average; KV-cache layout and indexing
bit-exact (V bytes equal; K within one bf16 ulp of the oracle's rounding of k_hat, or 4e-6 absolute where the
rotation cancels to a value near zero).
"""
import numpy as np
import pytest

import oracle
import synth
from _inputs import Layer, compare, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zg():
    import torch
    assert torch.cuda.is_available()
    import global_attention_gated_amd as m
    return m


def gpu_prefill(zg, L, gated, window, R, base, eps, **kw):
    if gated:
        return zg.swa_prefill(L.dq, L.dk, L.dv, L.dgate, L.dwq, L.dwk, window=window, rotary_dims=R, rope_base=base,
                              eps=eps, **kw)
    return zg.global_prefill(L.dq, L.dk, L.dv, L.dwq, L.dwk, rotary_dims=R, rope_base=base, eps=eps, **kw)


def oracle_prefill(L, gated, window, R, base, eps, **kw):
    return oracle.prefill_layer(L.q, L.k, L.v, L.gate if gated else None, L.wq, L.wk,
                                window=window if gated else None, rotary_dims=R, base=base, eps=eps, **kw)


# ------------------------------------------------------------------------------------------ generator
def test_gpu_generator_is_bit_equal_to_cpu(zg):
    import torch
    for shape, off in (((1000,), 0), ((3, 77), 5), ((2, 4096, 8, 128), 123456789)):
        d = synth.normal_bf16_device(1004, 7, synth.TENSOR_CACHE_K, shape, index_offset=off)
        np.testing.assert_array_equal(to_host_bits(d), synth.normal_bf16(1004, 7, synth.TENSOR_CACHE_K, shape, off))
    # strided fill: 5 rows of 40 elements into a buffer of row stride 64, indices 1000 + 100*o + i
    buf = torch.zeros(5 * 64, dtype=torch.bfloat16, device="cuda")
    synth.fill_device(buf.data_ptr(), 1, 2, 3, 5, 40, 64, 1000, 100)
    got = to_host_bits(buf).reshape(5, 64)
    for o in range(5):
        np.testing.assert_array_equal(got[o, :40], synth.normal_bf16_at(1, 2, 3, 1000 + 100 * o + np.arange(40)))
        assert np.all(got[o, 40:] == 0)


# ------------------------------------------------------------------------------------------ prefill
def test_single_gated_swa_layer_1x512_4q1kv(zg):
    """One gated-SWA layer: batch 1, seq 512, 4 query / 1 KV head, window 128, weights 1, eps 1e-6, RoPE on
    42 dims with base 10,000, seed 1001 -- compared in full."""
    L = Layer(1001, 0, 1, 512, 4, 1, w_spread=0.0)
    got = to_host_f64(gpu_prefill(zg, L, True, 128, 42, 1e4, 1e-6))
    mx, mean = compare(got, oracle_prefill(L, True, 128, 42, 1e4, 1e-6), "swa 1x512")
    print(f"swa 1x512 4q/1kv: max_abs {mx:.3e} mean_abs {mean:.3e}")


SHAPES = [
    # gated, B, S, Hq, Hkv, window, rotary dims
    (True, 2, 300, 8, 2, 128, 42),
    (True, 1, 200, 4, 4, 16, 42),
    (True, 1, 257, 16, 2, 128, 42),
    (True, 1, 130, 2, 1, 1, 42),
    (True, 1, 100, 4, 1, 4, 128),
    (True, 1, 97, 4, 1, 1000, 0),
    (True, 3, 33, 32, 8, 128, 42),
    # streaming SWA kernel (GQA group 4, window <= 128): multi-step runs, several units, window edges
    (True, 1, 9000, 4, 1, 128, 42),
    (True, 2, 3000, 8, 2, 100, 42),
    (True, 1, 1500, 4, 1, 1, 42),
    (True, 1, 1537, 4, 1, 16, 42),
    (True, 1, 1029, 4, 1, 33, 42),
    (True, 1, 700, 4, 1, 64, 128),
    (True, 1, 65, 4, 1, 127, 42),
    (True, 1, 31, 4, 1, 128, 42),
    (True, 1, 600, 4, 1, 128, 64),   # the most rotary dims the streaming kernel carries (32 pairs)
    (True, 1, 300, 4, 1, 128, 66),   # one pair more: the tile kernel
    (False, 2, 300, 8, 2, None, 42),
    (False, 1, 700, 4, 1, None, 42),
    (False, 1, 257, 16, 2, None, 42),
    (False, 1, 1, 4, 1, None, 42),
    (False, 1, 65, 4, 4, None, 42),
    (False, 1, 129, 32, 8, None, 128),
]


@pytest.mark.parametrize("gated,B,S,Hq,Hkv,W,R", SHAPES)
def test_prefill_shapes(zg, gated, B, S, Hq, Hkv, W, R):
    L = Layer(2000 + S, 3, B, S, Hq, Hkv, gated=gated)
    got = to_host_f64(gpu_prefill(zg, L, gated, W, R, 1e4, 1e-6))
    compare(got, oracle_prefill(L, gated, W, R, 1e4, 1e-6), f"{'swa' if gated else 'global'} B{B} S{S} {Hq}/{Hkv} W{W} R{R}")


@pytest.mark.parametrize("gated", [False, True])
def test_prefill_running_max_jumps(zg, gated):
    """Scores that jump late in the sequence: every query is one vector u (zero on the rotary dims, so
    RoPE leaves it alone) and the keys at a few positions are blends of u and noise, up to u itself. A
    query that reaches such a key sees its score max rise by more than 8 in log2 units over the keys
    before it, several times along the sequence, which drives the online softmax's rescaling paths."""
    B, S, Hq, Hkv, W, R = 1, 2500, 4, 1, 128, 42
    L = Layer(4242, 2, B, S, Hq, Hkv, gated=gated, w_spread=0.0)
    rng = np.random.default_rng(7)
    u = rng.standard_normal(128)
    u[:R] = 0.0
    q = np.broadcast_to(u, (B, S, Hq, 128))
    k = synth.bf16_bits_to_f64(L.k).copy()
    for pos, a in ((90, 0.45), (700, 0.7), (1500, 0.9), (2300, 1.0), (2310, 0.5)):
        k[:, pos, :, :] = a * u + (1.0 - a) * k[:, pos, :, :]
    L.q = synth.f64_to_bf16_bits(q)
    L.k = synth.f64_to_bf16_bits(k)
    L.wq = synth.f64_to_bf16_bits(np.full(128, 2.0))   # doubles every score: the max jumps by 13.6, then 10.5
    L.dq, L.dk, L.dwq = to_dev(L.q), to_dev(L.k), to_dev(L.wq)
    got = to_host_f64(gpu_prefill(zg, L, gated, W, R, 1e4, 1e-6))
    compare(got, oracle_prefill(L, gated, W, R, 1e4, 1e-6), f"{'swa' if gated else 'global'} max jumps")


def test_gate_infinities(zg):
    """sigma(+inf) = 1 exactly: a gated layer whose window covers the whole context is the global layer, bit for bit
    (both run on the tile kernel: same staging, same tiles, same masks; the gated epilogue multiplies by exactly 1);
    sigma(-inf) = 0 exactly (jaehun.me, "How Gated SWA Behaves": global layers skip the gate)."""
    import torch
    L = Layer(77, 1, 1, 300, 8, 2)
    plus = torch.full_like(L.dgate, float("inf"))
    minus = torch.full_like(L.dgate, float("-inf"))
    o_plus = zg.swa_prefill(L.dq, L.dk, L.dv, plus, L.dwq, L.dwk, window=1 << 20, rotary_dims=42, rope_base=1e4, eps=1e-6)
    o_glob = zg.global_prefill(L.dq, L.dk, L.dv, L.dwq, L.dwk, rotary_dims=42, rope_base=1e4, eps=1e-6)
    o_minus = zg.swa_prefill(L.dq, L.dk, L.dv, minus, L.dwq, L.dwk, window=128, rotary_dims=42, rope_base=1e4, eps=1e-6)
    ref = oracle_prefill(L, False, None, 42, 1e4, 1e-6)
    compare(to_host_f64(o_glob), ref, "global")
    np.testing.assert_array_equal(to_host_bits(o_plus), to_host_bits(o_glob))
    assert np.all(to_host_f64(o_minus) == 0.0)


def test_gate_plus_infinity_with_a_cache_is_the_global_layer_bit_for_bit(zg):
    """The same invariant on chunks against a KV cache: a 2-layer cache (layer 1 gated with a window longer than the
    sequence, layer 2 global), chunks of 70, 1 and 129 positions; with gate = +inf every chunk's output of layer 1
    equals layer 2's bit for bit, and both match the oracle's global layer."""
    import torch
    B, Hq, Hkv, R, base, eps, S_total = 2, 8, 2, 42, 1e7, 1e-6, 200
    W = 4096
    cache = zg.KVCache(n_layers=2, global_layers=[2], batch=B, n_kv_heads=Hkv, window=W, max_tokens=256)
    pos0 = 0
    for S in (70, 1, 129):
        L = Layer(41, 0, B, S, Hq, Hkv, gated=True, pos0=pos0, S_total=S_total)
        full = Layer(41, 0, B, pos0 + S, Hq, Hkv, gated=False, S_total=S_total, device=None)
        plus = torch.full_like(L.dgate, float("inf"))
        o_g = zg.swa_prefill(L.dq, L.dk, L.dv, plus, L.dwq, L.dwk, window=W, rotary_dims=R, rope_base=base, eps=eps,
                             pos0=pos0, cache=cache, layer=1)
        o_c = zg.global_prefill(L.dq, L.dk, L.dv, L.dwq, L.dwk, rotary_dims=R, rope_base=base, eps=eps, pos0=pos0,
                                cache=cache, layer=2)
        np.testing.assert_array_equal(to_host_bits(o_g), to_host_bits(o_c))
        ref = oracle_prefill(full, False, None, R, base, eps)[:, pos0:]
        compare(to_host_f64(o_c), ref, f"global chunk at {pos0}")
        pos0 += S
    cache.close()


@pytest.mark.parametrize("W", [200, 128])
def test_cached_first_chunk_is_the_cacheless_layer_bit_for_bit(zg, W):
    """A chunk at position 0 against an empty cache runs the same kernels as a call without a cache, so the outputs
    agree bit for bit: the global layer, and the gated layer on the tile kernel (window 200) or on the streaming
    kernel (window 128, GQA group 4, whose ring prefix is then empty)."""
    B, Hq, Hkv, S, R = 1, 16, 2, 333, 42
    if W <= 128:
        Hq = 4 * Hkv
    cache = zg.KVCache(n_layers=2, global_layers=[2], batch=B, n_kv_heads=Hkv, window=W, max_tokens=512)
    for layer, gated in ((1, True), (2, False)):
        L = Layer(12, layer, B, S, Hq, Hkv, gated=gated)
        a = gpu_prefill(zg, L, gated, W, R, 1e4, 1e-6)
        c = gpu_prefill(zg, L, gated, W, R, 1e4, 1e-6, pos0=0, cache=cache, layer=layer)
        np.testing.assert_array_equal(to_host_bits(a), to_host_bits(c))
    cache.close()


@pytest.mark.parametrize("W", [128, 33])
def test_chunked_swa_stream_small_chunks_match_oracle(zg, W):
    """Gated chunks on the streaming kernel against a cache ring (GQA group 4, W <= 128): chunks of 1, 33, 1, 97
    and 160 positions, so the ring prefix is partly empty (pos0 < W), a chunk is shorter than a 32-position step or
    than the window, and chunk starts fall off the 32-key tile grid; every chunk against the oracle, then the ring."""
    B, Hq, Hkv, R, base, eps = 2, 8, 2, 42, 1e7, 1e-6
    S_total = 292
    cache = zg.KVCache(n_layers=2, global_layers=[2], batch=B, n_kv_heads=Hkv, window=W, max_tokens=512)
    ocache = oracle.OracleCache(2, [2], B, Hkv, 128, W)
    pos0 = 0
    for S in (1, 33, 1, 97, 160):
        L = Layer(57, 1, B, S, Hq, Hkv, gated=True, pos0=pos0, S_total=S_total)
        got = to_host_f64(gpu_prefill(zg, L, True, W, R, base, eps, pos0=pos0, cache=cache, layer=1))
        ref = oracle_prefill(L, True, W, R, base, eps, pos0=pos0, cache=ocache, layer=1)
        compare(got, ref, f"W {W} chunk of {S} at {pos0}")
        pos0 += S
    assert cache.length(1, 0) == S_total
    assert _cache_check(zg, cache, ocache, 1, False) < 0.01
    cache.close()


def test_empty_inputs_are_noops(zg):
    import torch
    L = Layer(5, 0, 1, 8, 4, 1)
    e = torch.empty((1, 0, 4, 128), dtype=torch.bfloat16, device="cuda")
    ek = torch.empty((1, 0, 1, 128), dtype=torch.bfloat16, device="cuda")
    out = zg.swa_prefill(e, ek, ek, e, L.dwq, L.dwk, window=128)
    assert out.numel() == 0
    out = zg.global_prefill(e, ek, ek, L.dwq, L.dwk)
    assert out.numel() == 0


# ------------------------------------------------------------------------------------------ cache
def _cache_check(zg, cache, ocache, layer, glob):
    K, V = cache.read_layer(layer)
    K = K.numpy().view(np.uint16)
    V = V.numpy().view(np.uint16)
    if glob:
        OK, OV = ocache.global_image(layer)
        n = OK.shape[2]
        K, V = K[:, :, :n], V[:, :, :n]
    else:
        OK, OV, P = ocache.ring_image(layer)
        valid = P >= 0
        K = np.where(valid[:, None, :, None], K, 0)
        V = np.where(valid[:, None, :, None], V, 0)
    np.testing.assert_array_equal(V, OV)
    kd = np.abs(K.astype(np.int32) - OK.astype(np.int32))     # same sign: bit distance = ulp distance
    # k_hat is computed in fp32 (the rotary angle reduced to one revolution in fp64, then rounded to 24 bits for the
    # hardware sine and cosine: ~1e-6 absolute on the O(1) terms of x cos - y sin).  Rounded to bf16 that is one ulp
    # at most, except where the rotation cancels to a value near zero: there the same absolute error spans a few
    # ulps (or a sign), so elements beyond one ulp are held to it in absolute terms.
    far = kd > 1
    if far.any():
        ad = np.abs(synth.bf16_bits_to_f64(K[far]) - synth.bf16_bits_to_f64(OK[far]))
        assert ad.max() <= 4e-6, f"layer {layer}: k_hat differs by {kd[far].max()} ulp, {ad.max():.2e} absolute"
    return float(np.mean(kd != 0))


@pytest.mark.parametrize("W", [128, 16, 200])
def test_chunked_prefill_with_cache_matches_oracle(zg, W):
    """A 2-layer cache (layer 1 gated SWA with window W, layer 2 global), 2 sequences of 400 tokens in chunks of
    150, 40 and 210 (a chunk shorter than the window, chunk starts off the 32- and 64-key tile grid): every chunk's
    output against the oracle, then the cache images."""
    B, Hq, Hkv, R, base, eps = 2, 8, 2, 42, 1e7, 1e-6
    cache = zg.KVCache(n_layers=2, global_layers=[2], batch=B, n_kv_heads=Hkv, window=W, max_tokens=512)
    ocache = oracle.OracleCache(2, [2], B, Hkv, 128, W)
    S_total = 400
    mism = []
    for layer, gated in ((1, True), (2, False)):
        pos0 = 0
        for S in (150, 40, 210):
            L = Layer(31, layer, B, S, Hq, Hkv, gated=gated, pos0=pos0, S_total=S_total)
            got = to_host_f64(gpu_prefill(zg, L, gated, W, R, base, eps, pos0=pos0, cache=cache, layer=layer))
            ref = oracle_prefill(L, gated, W, R, base, eps, pos0=pos0, cache=ocache, layer=layer)
            compare(got, ref, f"layer {layer} chunk at {pos0}")
            pos0 += S
        assert cache.length(layer, 0) == S_total and cache.length(layer, 1) == S_total
        mism.append(_cache_check(zg, cache, ocache, layer, not gated))
    assert max(mism) < 0.01
    cache.close()


# ------------------------------------------------------------------------------------------ decode
def _decode_inputs(seed, L, B, Hq, Hkv, step):
    def gen(tensor, H, layer_base=0):
        return synth.normal_bf16(seed, 1000 + step, tensor, (L, B, H, 128))
    q, k, v, g = gen(synth.TENSOR_Q, Hq), gen(synth.TENSOR_K, Hkv), gen(synth.TENSOR_V, Hkv), gen(synth.TENSOR_GATE, Hq)
    return q, k, v, g


def test_decode_after_prefill_matches_oracle(zg):
    """3 layers (global = layer 2), window 16, 3 sequences: prefill 37 tokens into the cache, then 24
    decode steps (ring wrap-around included); every step against the oracle's decode."""
    Lh, B, Hq, Hkv, W, R, base, eps = 3, 3, 8, 2, 16, 42, 1e7, 1e-6
    glob = [2]
    cache = zg.KVCache(n_layers=Lh, global_layers=glob, batch=B, n_kv_heads=Hkv, window=W, max_tokens=100)
    ocache = oracle.OracleCache(Lh, glob, B, Hkv, 128, W)
    wq = np.stack([synth.norm_weight_bf16(9, l, synth.TENSOR_WQ, 128) for l in range(Lh)])
    wk = np.stack([synth.norm_weight_bf16(9, l, synth.TENSOR_WK, 128) for l in range(Lh)])
    S0 = 37
    for li in range(Lh):
        gated = (li + 1) not in glob
        L = Layer(9, li, B, S0, Hq, Hkv, gated=gated)
        L.wq, L.wk, L.dwq, L.dwk = wq[li], wk[li], to_dev(wq[li]), to_dev(wk[li])
        gpu_prefill(zg, L, gated, W, R, base, eps, cache=cache, layer=li + 1)
        oracle_prefill(L, gated, W, R, base, eps, cache=ocache, layer=li + 1)
    dwq, dwk = to_dev(wq), to_dev(wk)
    for step in range(24):
        p = S0 + step
        q, k, v, g = _decode_inputs(9, Lh, B, Hq, Hkv, step)
        got = to_host_f64(zg.hybrid_decode_step(to_dev(q), to_dev(k), to_dev(v), to_dev(g), dwq, dwk, [p] * B, cache,
                                                rotary_dims=R, rope_base=base, eps=eps))
        ref = oracle.decode_step(q, k, v, g, wq, wk, [p] * B, ocache, rotary_dims=R, base=base, eps=eps)
        compare(got, ref, f"decode step at {p}")
    for li in range(Lh):
        _cache_check(zg, cache, ocache, li + 1, (li + 1) in glob)
    cache.close()


def test_decode_from_empty_cache_equals_prefill(zg):
    """Token-by-token decode from position 0 reproduces the oracle's prefill of the same inputs."""
    Lh, B, Hq, Hkv, W, R, base, eps, S = 2, 2, 4, 1, 8, 42, 1e4, 1e-6, 40
    glob = [2]
    cache = zg.KVCache(n_layers=Lh, global_layers=glob, batch=B, n_kv_heads=Hkv, window=W, max_tokens=64)
    layers = [Layer(11, li, B, S, Hq, Hkv, gated=(li + 1) not in glob, device=None) for li in range(Lh)]
    wq = np.stack([l.wq for l in layers])
    wk = np.stack([l.wk for l in layers])
    refs = [oracle_prefill(l, (li + 1) not in glob, W, R, base, eps) for li, l in enumerate(layers)]
    dwq, dwk = to_dev(wq), to_dev(wk)
    for t in range(S):
        q = np.stack([l.q[:, t] for l in layers])
        k = np.stack([l.k[:, t] for l in layers])
        v = np.stack([l.v[:, t] for l in layers])
        g = np.stack([l.gate[:, t] if l.gate is not None else np.zeros_like(l.q[:, t]) for l in layers])
        got = to_host_f64(zg.hybrid_decode_step(to_dev(q), to_dev(k), to_dev(v), to_dev(g), dwq, dwk, [t] * B, cache,
                                                rotary_dims=R, rope_base=base, eps=eps))
        for li in range(Lh):
            compare(got[li], refs[li][:, t], f"decode t={t} layer {li + 1}")
    cache.close()


# ------------------------------------------------------------------------------------------ value range
@pytest.mark.parametrize("gated", [True, False])
def test_values_beyond_fp16_range_stay_finite_and_causal(zg, gated):
    """k_hat and v enter the prefill MFMAs as fp16 (include/zgattn.h, "Value range"): a value beyond +-65504
    saturates.  One key at position j carries |v| = 1e5 (and -2e5): the queries before j (which must not see it,
    also those sharing its 32- and 64-key tiles) match the oracle exactly as without it, and the queries that see it
    match the oracle with that value clamped to +-65504.  Streaming kernel (gated) and tile kernel (global)."""
    B, S, Hq, Hkv, W = 1, 700, 4, 1, 128
    L = Layer(808, 4, B, S, Hq, Hkv, gated=gated)
    j = 333                                   # inside a 64-key tile and a 32-key ring tile, not at their start
    v = synth.bf16_bits_to_f64(L.v).copy()
    v[0, j, 0, :64] = 1.0e5
    v[0, j, 0, 64:] = -2.0e5
    L.v = synth.f64_to_bf16_bits(v)
    L.dv = to_dev(L.v)
    got = to_host_f64(gpu_prefill(zg, L, gated, W, 42, 1e4, 1e-6))
    assert np.all(np.isfinite(got))
    clamped = Layer(808, 4, B, S, Hq, Hkv, gated=gated, device=None)
    clamped.v = synth.f64_to_bf16_bits(np.clip(v, -65504.0, 65504.0))
    ref = oracle_prefill(clamped, gated, W, 42, 1e4, 1e-6)
    compare(got[:, :j], ref[:, :j], "queries before the out-of-range key")
    see = slice(j, min(S, j + W)) if gated else slice(j, S)
    # the clamped value is exact in bf16 and fp16; errors scale with |v| ~ 6.5e4 where the output is dominated by it
    err = np.abs(got[:, see] - ref[:, see]) / np.maximum(1.0, np.abs(ref[:, see]))
    assert err.max() < 1e-2, err.max()
    if gated:
        compare(got[:, j + W:], ref[:, j + W:], "queries past the window of the out-of-range key")


# ------------------------------------------------------------------------------------------ error paths
def test_cache_beyond_device_memory_is_enomem(zg):
    """kv_cache_alloc of more than the GPU holds: ENOMEM, nothing allocated, and the device stays usable."""
    import torch
    with pytest.raises(zg.ZgError) as e:
        zg.KVCache(n_layers=32, global_layers=[6, 12, 18, 24, 30], batch=64, n_kv_heads=8, max_tokens=1 << 22)
    assert e.value.status == zg.ZG_ENOMEM
    x = torch.ones(4, device="cuda")
    assert float(x.sum()) == 4.0


def test_decode_positions_out_of_range_are_erange(zg):
    """hybrid_decode_step refuses a position that differs from the cache length, or that reaches the capacity, with
    ERANGE before anything is enqueued (the cache lengths stay as they were)."""
    L, B, Hq, Hkv = 2, 2, 8, 2
    cache = zg.KVCache(n_layers=L, global_layers=[2], batch=B, n_kv_heads=Hkv, window=16, max_tokens=8)
    q, k, v, g = _decode_inputs(3, L, B, Hq, Hkv, 0)
    w = np.stack([synth.norm_weight_bf16(3, l, synth.TENSOR_WQ, 128) for l in range(L)])
    args = (to_dev(q), to_dev(k), to_dev(v), to_dev(g), to_dev(w), to_dev(w))
    for positions in ([1, 0], [0, 5], [-1, 0]):           # the caches hold 0 positions
        with pytest.raises(zg.ZgError) as e:
            zg.hybrid_decode_step(*args, positions, cache)
        assert e.value.status == zg.ZG_ERANGE
    for l in (1, 2):
        for b in range(B):
            cache.set_length(l, b, 8)
    with pytest.raises(zg.ZgError) as e:                  # position 8 = max_tokens: no row left in the global cache
        zg.hybrid_decode_step(*args, [8, 8], cache)
    assert e.value.status == zg.ZG_ERANGE and b"capacity" in zg._lib.zg_last_error()
    assert all(cache.length(l, b) == 8 for l in (1, 2) for b in range(B))
    cache.close()


def test_prefill_workspace_too_small_for_the_cached_context_is_erange(zg):
    """A global chunk at pos0 stages every earlier key: a workspace sized for the chunk alone is refused."""
    import torch
    B, Hq, Hkv, S = 1, 4, 1, 64
    cache = zg.KVCache(n_layers=1, global_layers=[1], batch=B, n_kv_heads=Hkv, max_tokens=256)
    L0 = Layer(5, 0, B, S, Hq, Hkv, gated=False)
    gpu_prefill(zg, L0, False, None, 42, 1e4, 1e-6, cache=cache, layer=1)
    small = torch.empty(zg.workspace_bytes(B, S, Hkv), dtype=torch.uint8, device="cuda")
    with pytest.raises(zg.ZgError) as e:
        gpu_prefill(zg, L0, False, None, 42, 1e4, 1e-6, pos0=S, cache=cache, layer=1, workspace=small)
    assert e.value.status == zg.ZG_ERANGE
    assert cache.length(1, 0) == S
    cache.close()
