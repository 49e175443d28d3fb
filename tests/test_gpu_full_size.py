"""GPU parity at the full workload sizes, on sampled outputs the oracle computes row by row.

  two layers at 4 x 4096, 32 query / 8 KV heads: the gated-SWA layer in full, the global layer sampled
  the 32-layer schedule at 1 x 16384 (the benchmark's launch configuration): sampled rows of 4 layers
  the hybrid decode step, 32 sequences at position 262144: sampled (layer, sequence, KV head) units
  chunked prefill of 262144 tokens in 16384-token chunks: chunk boundaries and random rows of 3 layers

Inputs come from the seeded generator: the GPU fills its tensors on the device, the oracle regenerates
exactly the slices it needs on the host (the two generators are bit-equal, see test_gpu_parity).
"""
import numpy as np
import pytest

import oracle
import synth
from _inputs import compare, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

D, W = 128, 128
GLOBAL_LAYERS = (6, 12, 18, 24, 30)


@pytest.fixture(scope="module")
def zg():
    import torch
    assert torch.cuda.is_available()
    import global_attention_gated_amd as m
    return m


def dev_layer(seed, layer, B, S, Hq, Hkv, gated, w_spread=0.1, index_offset_tokens=0, S_total=None):
    """Device tensors of a layer (or of a chunk of S rows at token offset index_offset_tokens of a sequence of
    S_total tokens; B must be 1 for a chunk)."""
    import torch
    S_total = S if S_total is None else S_total
    out = {}
    for name, tid, H in (("q", synth.TENSOR_Q, Hq), ("k", synth.TENSOR_K, Hkv), ("v", synth.TENSOR_V, Hkv)) + \
            ((("gate", synth.TENSOR_GATE, Hq),) if gated else ()):
        t = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
        # rows of sequence b start at flat index (b*S_total + offset)*H*D
        synth.fill_device(t.data_ptr(), seed, layer, tid, B, S * H * D, S * H * D, index_offset_tokens * H * D,
                          S_total * H * D)
        out[name] = t
    out["wq_bits"] = synth.norm_weight_bf16(seed, layer, synth.TENSOR_WQ, D, spread=w_spread)
    out["wk_bits"] = synth.norm_weight_bf16(seed, layer, synth.TENSOR_WK, D, spread=w_spread)
    out["wq"], out["wk"] = to_dev(out["wq_bits"]), to_dev(out["wk_bits"])
    return out


def oracle_rows(seed, layer, b, kvh, positions, *, S_total, Hq, Hkv, gated, R, base, eps=1e-6, w_spread=0.1):
    """Oracle outputs [len(positions), G, D] of query heads kvh*G.. for sampled positions of sequence b."""
    G = Hq // Hkv
    pos = np.asarray(sorted(positions), dtype=np.int64)
    if gated:   # the union of the sampled rows' windows
        kpos = np.unique(np.concatenate([np.arange(max(0, p - W + 1), p + 1) for p in pos])).astype(np.int64)
    else:
        kpos = np.arange(0, int(pos.max()) + 1, dtype=np.int64)
    kidx = (((b * S_total + kpos) * Hkv + kvh)[:, None]) * D + np.arange(D)[None, :]
    k = synth.normal_bf16_at(seed, layer, synth.TENSOR_K, kidx)
    v = synth.normal_bf16_at(seed, layer, synth.TENSOR_V, kidx)
    heads = np.arange(kvh * G, (kvh + 1) * G)
    qidx = (((b * S_total + pos)[:, None] * Hq + heads[None, :])[:, :, None]) * D + np.arange(D)[None, None, :]
    q = synth.normal_bf16_at(seed, layer, synth.TENSOR_Q, qidx)                       # [n, G, D]
    g = synth.normal_bf16_at(seed, layer, synth.TENSOR_GATE, qidx) if gated else None
    wq = synth.norm_weight_bf16(seed, layer, synth.TENSOR_WQ, D, spread=w_spread)
    wk = synth.norm_weight_bf16(seed, layer, synth.TENSOR_WK, D, spread=w_spread)
    khat = oracle.cache_key(oracle.qk_prologue(k, kpos, wk, eps, R, base))
    qhat = oracle.qk_prologue(q, pos[:, None], wq, eps, R, base)
    out = np.empty((len(pos), G, D))
    for j in range(G):
        out[:, j] = oracle.attend(qhat[:, j], pos, khat, v, kpos, W if gated else None, None if g is None else g[:, j])
    return pos, out


def sample_positions(S, rng, n_random, extra=()):
    s = {0, 1, 2, 3, 125, 126, 127, 128, 129, 130, S - 1} | set(int(x) for x in extra)
    s |= set(int(x) for x in rng.choice(S, size=min(n_random, S), replace=False))
    return sorted(p for p in s if 0 <= p < S)


# ------------------------------------------------------------------------------------------ 4 x 4096
def test_two_layers_4x4096_32q8kv(zg):
    B, S, Hq, Hkv, R, base, seed = 4, 4096, 32, 8, 42, 1e4, 1002
    rng = np.random.default_rng(2)
    for layer, gated in ((1, True), (2, False)):
        t = dev_layer(seed, layer, B, S, Hq, Hkv, gated)
        if gated:
            out = zg.swa_prefill(t["q"], t["k"], t["v"], t["gate"], t["wq"], t["wk"], window=W, rotary_dims=R,
                                 rope_base=base, eps=1e-6)
            got = to_host_f64(out)
            bits = {n: synth.normal_bf16(seed, layer, tid, (B, S, H, D)) for n, tid, H in
                    (("q", 0, Hq), ("k", 1, Hkv), ("v", 2, Hkv), ("g", 3, Hq))}
            ref = oracle.prefill_layer(bits["q"], bits["k"], bits["v"], bits["g"], t["wq_bits"], t["wk_bits"],
                                       window=W, rotary_dims=R, base=base, eps=1e-6)
            compare(got, ref, "4x4096 gated SWA layer, every output")
        else:
            out = zg.global_prefill(t["q"], t["k"], t["v"], t["wq"], t["wk"], rotary_dims=R, rope_base=base, eps=1e-6)
            got = to_host_f64(out)
            pos = sample_positions(S, rng, 40)
            G = Hq // Hkv
            for b in range(B):
                for kvh in range(Hkv):
                    p, ref = oracle_rows(seed, layer, b, kvh, pos, S_total=S, Hq=Hq, Hkv=Hkv, gated=False, R=R, base=base)
                    compare(got[b, p][:, kvh * G:(kvh + 1) * G], ref, f"4x4096 global layer b={b} kvh={kvh}")


# ------------------------------------------------------------------------------------------ 1 x 16384 x 32 layers
def test_schedule_1x16384_sampled_layers(zg):
    """The benchmark's workload: all 32 layers run on the GPU exactly as bench.py launches them; four layers
    (two gated SWA, two global) are checked on sampled rows."""
    import torch
    B, S, Hq, Hkv, R, base, seed = 1, 16384, 32, 8, 42, 1e4, 1003
    checked = {1: None, 6: None, 17: None, 30: None}
    ws = torch.empty(zg.workspace_bytes(B, S, Hkv, D), dtype=torch.uint8, device="cuda")
    for layer in range(1, 33):
        gated = layer not in GLOBAL_LAYERS
        t = dev_layer(seed, layer, B, S, Hq, Hkv, gated)
        if gated:
            out = zg.swa_prefill(t["q"], t["k"], t["v"], t["gate"], t["wq"], t["wk"], window=W, rotary_dims=R,
                                 rope_base=base, eps=1e-6, workspace=ws)
        else:
            out = zg.global_prefill(t["q"], t["k"], t["v"], t["wq"], t["wk"], rotary_dims=R, rope_base=base, eps=1e-6,
                                    workspace=ws)
        if layer in checked:
            checked[layer] = to_host_f64(out)
        del t, out
    rng = np.random.default_rng(3)
    G = Hq // Hkv
    for layer, got in checked.items():
        gated = layer not in GLOBAL_LAYERS
        pos = sample_positions(S, rng, 24)
        for kvh in range(Hkv):
            p, ref = oracle_rows(seed, layer, 0, kvh, pos, S_total=S, Hq=Hq, Hkv=Hkv, gated=gated, R=R, base=base)
            compare(got[0, p][:, kvh * G:(kvh + 1) * G], ref, f"16K layer {layer} kvh={kvh}")


# ------------------------------------------------------------------------------------------ one shot at 256K
def test_one_shot_prefill_1x262144_sampled(zg):
    """The schedule sweep's longest point: one gated-SWA and one global layer prefilled in one call over
    262,144 tokens (RoPE base 1e7), checked on sampled rows (the global layer on two KV heads)."""
    import torch
    B, S, Hq, Hkv, R, base, seed = 1, 262144, 32, 8, 42, 1e7, 1006
    G = Hq // Hkv
    rng = np.random.default_rng(5)
    ws = torch.empty(zg.workspace_bytes(B, S, Hkv, D), dtype=torch.uint8, device="cuda")
    for layer, gated, heads in ((1, True, range(Hkv)), (6, False, (0, Hkv - 1))):
        t = dev_layer(seed, layer, B, S, Hq, Hkv, gated)
        if gated:
            out = zg.swa_prefill(t["q"], t["k"], t["v"], t["gate"], t["wq"], t["wk"], window=W, rotary_dims=R,
                                 rope_base=base, eps=1e-6, workspace=ws)
        else:
            out = zg.global_prefill(t["q"], t["k"], t["v"], t["wq"], t["wk"], rotary_dims=R, rope_base=base, eps=1e-6,
                                    workspace=ws)
        pos = sample_positions(S, rng, 12 if gated else 6, extra=(65535, 65536, 131071, 200000))
        got = to_host_f64(out[0, torch.tensor(pos, device="cuda")])
        del t, out
        torch.cuda.empty_cache()
        for kvh in heads:
            p, ref = oracle_rows(seed, layer, 0, kvh, pos, S_total=S, Hq=Hq, Hkv=Hkv, gated=gated, R=R, base=base)
            compare(got[:, kvh * G:(kvh + 1) * G], ref, f"262144 one-shot layer {layer} kvh={kvh}")


# ------------------------------------------------------------------------------------------ decode at 256K
def test_hybrid_decode_32x262144_sampled(zg):
    import torch
    B, P, Hq, Hkv, R, base, seed, L = 32, 262144, 32, 8, 42, 1e7, 1004, 32
    G = Hq // Hkv
    torch.cuda.empty_cache()
    cache = zg.KVCache(n_layers=L, global_layers=GLOBAL_LAYERS, batch=B, n_kv_heads=Hkv, head_dim=D, window=W,
                       max_tokens=P + 1)
    for l in range(1, L + 1):
        kp, vp, slots = cache.layer_view(l)
        synth.fill_kv_cache_layer(kp, vp, slots, seed=seed, layer=l, batch=B, n_kv_heads=Hkv, head_dim=D, n_positions=P,
                                  is_global=l in GLOBAL_LAYERS, window=W)
        for b in range(B):
            cache.set_length(l, b, P)
    shapes = {"q": (L, B, Hq, D), "k": (L, B, Hkv, D), "v": (L, B, Hkv, D), "g": (L, B, Hq, D)}
    tids = {"q": synth.TENSOR_Q, "k": synth.TENSOR_K, "v": synth.TENSOR_V, "g": synth.TENSOR_GATE}
    bits = {n: synth.normal_bf16(seed, 1000, tids[n], shapes[n]) for n in shapes}
    wq = np.stack([synth.norm_weight_bf16(seed, l, synth.TENSOR_WQ, D) for l in range(1, L + 1)])
    wk = np.stack([synth.norm_weight_bf16(seed, l, synth.TENSOR_WK, D) for l in range(1, L + 1)])
    got = to_host_f64(zg.hybrid_decode_step(to_dev(bits["q"]), to_dev(bits["k"]), to_dev(bits["v"]), to_dev(bits["g"]),
                                            to_dev(wq), to_dev(wk), [P] * B, cache, rotary_dims=R, rope_base=base,
                                            eps=1e-6))
    assert all(cache.length(l, b) == P + 1 for l in (1, 6, 32) for b in (0, 31))

    def oracle_unit(l, b, kvh):
        glob = l in GLOBAL_LAYERS
        kpos = np.arange(0 if glob else P - W + 1, P, dtype=np.int64)
        kc = oracle.bf16_to_f64(synth.kv_cache_values(seed, l, synth.TENSOR_CACHE_K, b, kvh, kpos, n_kv_heads=Hkv,
                                                      head_dim=D, n_positions=P))
        vc = oracle.bf16_to_f64(synth.kv_cache_values(seed, l, synth.TENSOR_CACHE_V, b, kvh, kpos, n_kv_heads=Hkv,
                                                      head_dim=D, n_positions=P))
        knew = oracle.cache_key(oracle.qk_prologue(bits["k"][l - 1, b, kvh][None], P, wk[l - 1], 1e-6, R, base))
        keys = np.concatenate([kc, knew])
        vals = np.concatenate([vc, oracle.bf16_to_f64(bits["v"][l - 1, b, kvh][None])])
        kp = np.concatenate([kpos, [P]])
        heads = slice(kvh * G, (kvh + 1) * G)
        qhat = oracle.qk_prologue(bits["q"][l - 1, b, heads], P, wq[l - 1], 1e-6, R, base)
        return oracle.attend(qhat, P, keys, vals, kp, None if glob else W, None if glob else bits["g"][l - 1, b, heads])

    rng = np.random.default_rng(4)
    units = [(6, 0, 0), (18, 17, 5), (30, 31, 7)]                                     # global layers
    units += [(int(l), int(rng.integers(B)), int(rng.integers(Hkv)))                   # gated-SWA layers
              for l in rng.choice([l for l in range(1, L + 1) if l not in GLOBAL_LAYERS], size=24, replace=False)]
    units += [(1, 0, 0), (32, 31, 7)]
    for l, b, kvh in units:
        compare(got[l - 1, b, kvh * G:(kvh + 1) * G], oracle_unit(l, b, kvh), f"decode layer {l} b={b} kvh={kvh}")
    cache.close()
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------------------------ chunked 256K prefill
def test_chunked_prefill_262144_in_16384_chunks(zg):
    import torch
    S_total, C, Hq, Hkv, R, base, seed, L = 262144, 16384, 32, 8, 42, 1e7, 1005, 32
    G = Hq // Hkv
    torch.cuda.empty_cache()
    cache = zg.KVCache(n_layers=L, global_layers=GLOBAL_LAYERS, batch=1, n_kv_heads=Hkv, head_dim=D, window=W,
                       max_tokens=S_total)
    # KV footprint of this cache as the pages count it: 5.0 GiB hybrid vs 32.0 GiB if every layer were global
    hybrid = zg.footprint_bytes(S_total)
    assert round(hybrid / 2**30, 1) == 5.0
    assert zg.footprint_bytes(S_total, global_layers=range(1, 33)) == 32 * 2**30
    assert hybrid <= cache.device_bytes < hybrid + 512 * 2**20          # + rings' padding and decode partials
    rng = np.random.default_rng(5)
    bounds = [c * C + d for c in range(1, S_total // C) for d in (-128, -127, -1, 0, 1, 127)]
    pos = sample_positions(S_total, rng, 16, extra=bounds)
    checked = {1: {}, 6: {}, 32: {}}
    # the largest workspaces a chunk needs: a gated chunk stages W-1 earlier keys, the last global chunk every key
    ws = torch.empty(zg.workspace_bytes(1, C, Hkv, D, pos0=C, window=W), dtype=torch.uint8, device="cuda")
    gws = torch.empty(zg.workspace_bytes(1, C, Hkv, D, pos0=S_total - C), dtype=torch.uint8, device="cuda")
    for layer in range(1, L + 1):
        gated = layer not in GLOBAL_LAYERS
        for c in range(S_total // C):
            t = dev_layer(seed, layer, 1, C, Hq, Hkv, gated, index_offset_tokens=c * C, S_total=S_total)
            if gated:
                out = zg.swa_prefill(t["q"], t["k"], t["v"], t["gate"], t["wq"], t["wk"], window=W, rotary_dims=R,
                                     rope_base=base, eps=1e-6, pos0=c * C, cache=cache, layer=layer, workspace=ws)
            else:
                out = zg.global_prefill(t["q"], t["k"], t["v"], t["wq"], t["wk"], rotary_dims=R, rope_base=base,
                                        eps=1e-6, pos0=c * C, cache=cache, layer=layer, workspace=gws)
            if layer in checked:
                rows = [p - c * C for p in pos if c * C <= p < (c + 1) * C]
                if rows:
                    got = to_host_f64(out[0, rows])
                    for r, p in zip(rows, got):
                        checked[layer][r + c * C] = p
            del t, out
        assert cache.length(layer, 0) == S_total
    for layer, rows in checked.items():
        gated = layer not in GLOBAL_LAYERS
        p_sorted = sorted(rows)
        got = np.stack([rows[p] for p in p_sorted])                                     # [n, Hq, D]
        for kvh in ((0, 7) if not gated else range(Hkv)):
            p, ref = oracle_rows(seed, layer, 0, kvh, p_sorted, S_total=S_total, Hq=Hq, Hkv=Hkv, gated=gated, R=R,
                                 base=base)
            compare(got[:, kvh * G:(kvh + 1) * G], ref, f"262144-token chunked prefill layer {layer} kvh={kvh}")
    cache.close()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("gated", [True, False])
def test_backward_1x16384_sampled(zg, gated):
    """Training forward and backward at 1 x 16384, 32 query / 8 KV heads (the backward benchmark's launch
    configuration): sampled query rows (dq, dgate) and key rows (dk, dv) of one KV head's group against the
    row-sampled oracle, to the bar of test_gpu_backward (2 |D_X| + 2^-7 |X_ref| + R_X / 16; mean 2 mean|D_X| + 0.005 R_X)."""
    import torch
    seed, layer, S, Hq, Hkv, kvh = 1009, 2 if gated else 6, 16384, 32, 8, 5
    G = Hq // Hkv
    L = dev_layer(seed, layer, 1, S, Hq, Hkv, gated)
    dout = torch.empty((1, S, Hq, D), dtype=torch.bfloat16, device="cuda")
    synth.fill_device(dout.data_ptr(), seed, layer, synth.TENSOR_DOUT, 1, S * Hq * D, S * Hq * D, 0, S * Hq * D)
    out, lse = zg.prefill_train(L["q"], L["k"], L["v"], L.get("gate"), L["wq"], L["wk"], window=W, rotary_dims=42,
                                rope_base=1e4, eps=1e-6)
    g = zg.prefill_backward(L["q"], L["k"], L["v"], L.get("gate"), L["wq"], L["wk"], out, lse, dout, window=W,
                            rotary_dims=42, rope_base=1e4, eps=1e-6)
    rng = np.random.default_rng(3)
    qr = np.unique(np.concatenate([[0, 1, 31, 127, 128, 4095, 8191, S - 1], rng.integers(0, S, 24)]))
    kr = np.unique(np.concatenate([[0, 1, 32, 127, 128, 8192, S - 2, S - 1], rng.integers(0, S, 24)]))
    heads = np.arange(kvh * G, (kvh + 1) * G)
    tok = np.arange(S)

    def host(tid, H, hs):
        idx = ((tok[:, None, None] * H + hs[None, :, None]) * D + np.arange(D)[None, None, :])
        return synth.normal_bf16_at(seed, layer, tid, idx)[None]              # [1, S, len(hs), D]

    q, gt, do = host(synth.TENSOR_Q, Hq, heads), (host(synth.TENSOR_GATE, Hq, heads) if gated else None), \
        host(synth.TENSOR_DOUT, Hq, heads)
    k, v = host(synth.TENSOR_K, Hkv, np.array([kvh])), host(synth.TENSOR_V, Hkv, np.array([kvh]))
    ref = oracle.prefill_layer_backward_rows(q, k, v, gt, L["wq_bits"], L["wk_bits"], do, window=W if gated else None,
                                             rotary_dims=42, base=1e4, eps=1e-6, b=0, kv_head=0, query_rows=qr,
                                             key_rows=kr)
    got = {"dq": to_host_f64(g["dq"][0, qr][:, heads]), "dk": to_host_f64(g["dk"][0, kr, kvh]),
           "dv": to_host_f64(g["dv"][0, kr, kvh])}
    if gated:
        got["dgate"] = to_host_f64(g["dgate"][0, qr][:, heads])
    rms_dv = float(np.sqrt(np.mean(ref["dv"] ** 2)))
    for n, x in got.items():
        r = ref[n]
        d = np.abs(ref[n + "_d16"] - r) if n in ("dq", "dk") else 0.0
        err = np.abs(x - r)
        rms = float(np.sqrt(np.mean(r ** 2)))
        R = rms if rms > 0.01 * rms_dv else rms_dv
        bound = 2 * d + 2.0 ** -7 * np.abs(r) + R / 16
        print(f"backward 16K {'swa' if gated else 'global'} {n}: max_abs {err.max():.3e} mean_abs {err.mean():.3e} "
              f"R {R:.3e} max err/bound {np.max(err / bound):.3f}")
        assert np.all(np.isfinite(x)), n
        assert np.all(err <= bound), f"{n}: max err/bound {np.max(err / bound):.3f}"
        assert err.mean() <= 2 * float(np.mean(d)) + 0.005 * R, f"{n}: mean {err.mean():.3e}"
