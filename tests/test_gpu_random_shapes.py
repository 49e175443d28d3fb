"""GPU parity over seeded random shapes: one-shot prefill of a gated SWA or a global layer, through the C ABI,
against the fp64 CPU oracle (same bar as the fixed shapes: |gpu - oracle| <= 1e-2 per element, <= 1e-3 on average).

Each case draws batch, length, heads, GQA group, window, rotary dims, RoPE base and eps from its own seed; half of
the gated cases fall in the streaming kernel's case (group 4, window <= 128, rotary dims <= 64) and half anywhere,
so both SWA kernels and the global kernel see lengths that end mid-tile and mid-step.
"""
import numpy as np
import pytest

from _inputs import Layer, compare, to_dev, to_host_f64
from test_gpu_parity import gpu_prefill, oracle_prefill, zg  # noqa: F401  (zg is a fixture)

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw_case(idx):
    rng = np.random.default_rng(7100 + idx)
    gated = idx % 4 != 3                       # three gated cases in four
    stream = gated and idx % 2 == 0            # half of the gated cases in the streaming kernel's case
    B = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = 4 if stream else int(rng.choice([1, 2, 4, 8]))
    while Hkv * G > 32:
        Hkv //= 2
    if stream:
        W = int(rng.integers(1, 129))
        R = 2 * int(rng.integers(0, 33))
    else:
        W = int(rng.integers(1, 400)) if gated else None
        R = 2 * int(rng.integers(0, 65))
    max_tokens = 6000 if gated else 2500     # per sequence; the oracle finishes each case in about a second
    S = int(rng.integers(1, max_tokens // B + 1))
    base = float(rng.choice([1e4, 5e5, 1e7]))
    eps = float(rng.choice([1e-6, 1e-5]))
    return gated, B, S, G * Hkv, Hkv, W, R, base, eps


CASES = [draw_case(i) for i in range(N_CASES)]


def _id(c):
    gated, B, S, Hq, Hkv, W, R, base, eps = c
    return f"{'swa' if gated else 'global'}-B{B}-S{S}-{Hq}q{Hkv}kv-W{W}-R{R}-base{base:g}-eps{eps:g}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_prefill_random_shape(zg, case):
    gated, B, S, Hq, Hkv, W, R, base, eps = case
    L = Layer(5000 + S, 4, B, S, Hq, Hkv, gated=gated)
    got = to_host_f64(gpu_prefill(zg, L, gated, W, R, base, eps))
    compare(got, oracle_prefill(L, gated, W, R, base, eps), _id(case))


# ------------------------------------------------------------------------------------------ chunks against a cache
N_CHUNK_CASES = 8


def draw_chunk_case(idx):
    rng = np.random.default_rng(7300 + idx)
    stream = idx % 2 == 0                       # the gated layer on the streaming kernel in half of the cases
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2, 4]))
    G = 4 if stream else int(rng.choice([1, 2, 8]))
    W = int(rng.integers(1, 129)) if stream else int(rng.integers(1, 300))
    R = 2 * int(rng.integers(0, 33 if stream else 65))
    chunks = [int(x) for x in rng.integers(1, 400, size=int(rng.integers(2, 5)))]
    return B, G * Hkv, Hkv, W, R, chunks


CHUNK_CASES = [draw_chunk_case(i) for i in range(N_CHUNK_CASES)]


def _chunk_id(c):
    B, Hq, Hkv, W, R, chunks = c
    return f"B{B}-{Hq}q{Hkv}kv-W{W}-R{R}-chunks{'+'.join(map(str, chunks))}"


@pytest.mark.parametrize("case", CHUNK_CASES, ids=[_chunk_id(c) for c in CHUNK_CASES])
def test_chunked_prefill_random_splits(zg, case):
    """A 2-layer cache (layer 1 gated SWA, layer 2 global) filled chunk by chunk: every chunk's output against the
    oracle with its own cache, then both layers' cache images (V bytes equal, k_hat as in the fixed-shape cache tests)."""
    import oracle
    from test_gpu_parity import _cache_check
    B, Hq, Hkv, W, R, chunks = case
    base, eps = 1e7, 1e-6
    S_total = sum(chunks)
    cache = zg.KVCache(n_layers=2, global_layers=[2], batch=B, n_kv_heads=Hkv, window=W, max_tokens=S_total + 64)
    ocache = oracle.OracleCache(2, [2], B, Hkv, 128, W)
    try:
        mism = []
        for layer, gated in ((1, True), (2, False)):
            pos0 = 0
            for S in chunks:
                L = Layer(91 + S_total, layer, B, S, Hq, Hkv, gated=gated, pos0=pos0, S_total=S_total)
                got = to_host_f64(gpu_prefill(zg, L, gated, W, R, base, eps, pos0=pos0, cache=cache, layer=layer))
                ref = oracle_prefill(L, gated, W, R, base, eps, pos0=pos0, cache=ocache, layer=layer)
                compare(got, ref, f"{_chunk_id(case)} layer {layer} chunk of {S} at {pos0}")
                pos0 += S
            assert all(cache.length(layer, b) == S_total for b in range(B))
            mism.append(_cache_check(zg, cache, ocache, layer, not gated))
        assert max(mism) < 0.01
    finally:
        cache.close()


# ------------------------------------------------------------------------------------------ decode
N_DECODE_CASES = 6


def draw_decode_case(idx):
    rng = np.random.default_rng(7500 + idx)
    Lh = int(rng.integers(2, 5))
    glob = sorted(int(x) + 1 for x in rng.choice(Lh, size=int(rng.integers(1, Lh)), replace=False))
    B = int(rng.integers(1, 5))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    W = int(rng.integers(1, 65))
    R = 2 * int(rng.integers(0, 65))
    S0 = int(rng.integers(1, 600))
    base = float(rng.choice([1e4, 1e7]))
    return Lh, glob, B, G * Hkv, Hkv, W, R, S0, base


DECODE_CASES = [draw_decode_case(i) for i in range(N_DECODE_CASES)]


def _decode_id(c):
    Lh, glob, B, Hq, Hkv, W, R, S0, base = c
    return f"L{Lh}-global{'_'.join(map(str, glob))}-B{B}-{Hq}q{Hkv}kv-W{W}-R{R}-S0_{S0}-base{base:g}"


@pytest.mark.parametrize("case", DECODE_CASES, ids=[_decode_id(c) for c in DECODE_CASES])
def test_decode_random_shape(zg, case):
    """Prefill S0 tokens into a cache of Lh layers (the drawn ones global), then decode until every ring has wrapped
    (at least 6 steps); each step against the oracle's decode, then every layer's cache image."""
    import oracle
    import synth
    from test_gpu_parity import _cache_check, _decode_inputs
    Lh, glob, B, Hq, Hkv, W, R, S0, base = case
    eps = 1e-6
    steps = 6 if S0 >= W else W - S0 + 6     # past the ring's first wrap in every case
    cache = zg.KVCache(n_layers=Lh, global_layers=glob, batch=B, n_kv_heads=Hkv, window=W, max_tokens=S0 + steps + 8)
    ocache = oracle.OracleCache(Lh, glob, B, Hkv, 128, W)
    try:
        wq = np.stack([synth.norm_weight_bf16(13, li, synth.TENSOR_WQ, 128) for li in range(Lh)])
        wk = np.stack([synth.norm_weight_bf16(13, li, synth.TENSOR_WK, 128) for li in range(Lh)])
        for li in range(Lh):
            gated = (li + 1) not in glob
            L = Layer(13 + S0, li, B, S0, Hq, Hkv, gated=gated)
            L.wq, L.wk, L.dwq, L.dwk = wq[li], wk[li], to_dev(wq[li]), to_dev(wk[li])
            gpu_prefill(zg, L, gated, W, R, base, eps, cache=cache, layer=li + 1)
            oracle_prefill(L, gated, W, R, base, eps, cache=ocache, layer=li + 1)
        dwq, dwk = to_dev(wq), to_dev(wk)
        for step in range(steps):
            p = S0 + step
            q, k, v, g = _decode_inputs(13 + S0, Lh, B, Hq, Hkv, step)
            got = to_host_f64(zg.hybrid_decode_step(to_dev(q), to_dev(k), to_dev(v), to_dev(g), dwq, dwk, [p] * B,
                                                    cache, rotary_dims=R, rope_base=base, eps=eps))
            ref = oracle.decode_step(q, k, v, g, wq, wk, [p] * B, ocache, rotary_dims=R, base=base, eps=eps)
            compare(got, ref, f"{_decode_id(case)} step at {p}")
        for li in range(Lh):
            _cache_check(zg, cache, ocache, li + 1, (li + 1) in glob)
    finally:
        cache.close()


# ------------------------------------------------------------------------------------------ backward
N_BACKWARD_CASES = 6


def draw_backward_case(idx):
    rng = np.random.default_rng(7700 + idx)
    gated = idx % 3 != 2
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = 4                                       # the backward's one GQA group (others are EUNSUPPORTED)
    W = int(rng.integers(1, 300)) if gated else 0
    R = 2 * int(rng.integers(0, 65))
    S = int(rng.integers(1, (1500 if gated else 1000) // B + 1))
    base = float(rng.choice([1e4, 1e7]))
    eps = float(rng.choice([1e-6, 1e-5]))
    return gated, B, S, G * Hkv, Hkv, W, R, base, eps


BACKWARD_CASES = [draw_backward_case(i) for i in range(N_BACKWARD_CASES)]


def _backward_id(c):
    gated, B, S, Hq, Hkv, W, R, base, eps = c
    return f"{'swa' if gated else 'global'}-B{B}-S{S}-{Hq}q{Hkv}kv-W{W}-R{R}-base{base:g}-eps{eps:g}"


@pytest.mark.parametrize("case", BACKWARD_CASES, ids=[_backward_id(c) for c in BACKWARD_CASES])
def test_training_backward_random_shape(zg, case):
    """The training forward's out and lse feed the backward; forward against the oracle at the forward bar, every
    gradient against the oracle's exact gradients at the backward bar of the fixed-shape backward tests."""
    import oracle
    import synth
    from test_gpu_backward import _check
    gated, B, S, Hq, Hkv, W, R, base, eps = case
    L = Layer(8100 + S, 1, B, S, Hq, Hkv, gated=gated)
    dout = synth.normal_bf16(8100 + S, 1, synth.TENSOR_DOUT, (B, S, Hq, 128))
    kw = dict(window=W if gated else None, rotary_dims=R, base=base, eps=eps)
    ref = oracle.prefill_layer_backward(L.q, L.k, L.v, L.gate, L.wq, L.wk, dout, **kw)
    ref16 = oracle.prefill_layer_backward(L.q, L.k, L.v, L.gate, L.wq, L.wk, dout, delta_from_bf16_out=True,
                                          dA_bf16=True, **kw)
    out, lse = zg.prefill_train(L.dq, L.dk, L.dv, L.dgate, L.dwq, L.dwk, window=W, rotary_dims=R, rope_base=base,
                                eps=eps)
    compare(to_host_f64(out), ref["out"], f"{_backward_id(case)} training forward out")
    compare(lse.detach().cpu().numpy().transpose(0, 2, 1).astype(np.float64), ref["lse"],
            f"{_backward_id(case)} training forward lse")
    g = zg.prefill_backward(L.dq, L.dk, L.dv, L.dgate, L.dwq, L.dwk, out, lse, to_dev(dout), window=W,
                            rotary_dims=R, rope_base=base, eps=eps)
    _check(g, ref, ref16, gated, _backward_id(case))
