"""The C-ABI library on the host: it loads, exports every declared entry point, and rejects malformed
arguments with a status code before touching the GPU (no device is needed for these tests)."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def zg():
    lib = os.path.join(ROOT, "global_attention_gated_amd", "libzgattn.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.build()
    import global_attention_gated_amd as m
    return m


def _declared():
    text = open(os.path.join(ROOT, "include", "zgattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_entry_points_are_exported(zg):
    names = _declared()
    assert {"swa_prefill", "global_prefill", "hybrid_decode_step", "kv_cache_alloc"} <= set(names)
    lib = ctypes.CDLL(zg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(zg.EXPORTED) == set(names)


def test_footprint_closed_form_matches_oracle_and_page(zg):
    for T in (0, 1, 127, 128, 129, 4096, 262144):
        assert zg.footprint_bytes(T) == oracle.kv_footprint_bytes(T)
        assert zg.footprint_bytes(T, global_layers=range(1, 33)) == oracle.kv_footprint_bytes(T, global_layer_ids=range(1, 33))
    assert zg.footprint_bytes(262144, global_layers=range(1, 33)) == 32 * 2**30
    assert round(zg.footprint_bytes(262144) / 2**30, 1) == 5.0
    assert zg.footprint_bytes(1001) - zg.footprint_bytes(1000) == 20480
    assert zg.footprint_bytes(10, batch=3) == 3 * zg.footprint_bytes(10)


def test_workspace_bytes(zg):
    assert zg.workspace_bytes(1, 16384, 8) == 2 * 16384 * 8 * 128 * 2
    # whole 64-key tiles
    assert zg.workspace_bytes(2, 100, 8) == 2 * 2 * 128 * 8 * 128 * 2
    assert zg.workspace_bytes(1, 1, 1) == 2 * 64 * 128 * 2
    assert zg.workspace_bytes(1, 0, 8) == 0


def test_workspace_bytes_with_a_cache(zg):
    """A chunk at pos0 stages the keys its queries see: every earlier position for a global layer (window 0), the
    W - 1 before pos0 for a gated one, in whole 64-key tiles."""
    per_key = 2 * 8 * 128 * 2            # k_hat and v^T, fp16, 8 KV heads
    assert zg.workspace_bytes(1, 16384, 8, pos0=245760) == 262144 * per_key
    assert zg.workspace_bytes(1, 100, 8, pos0=1000) == 1152 * per_key              # 1100 keys -> 18 tiles
    assert zg.workspace_bytes(1, 100, 8, pos0=1000, window=128) == 256 * per_key    # 227 keys -> 4 tiles
    assert zg.workspace_bytes(1, 100, 8, pos0=50, window=128) == 192 * per_key      # keys 0..149
    assert zg.workspace_bytes(2, 100, 8, pos0=0, window=128) == 2 * zg.workspace_bytes(1, 100, 8)
    assert zg._lib.prefill_workspace_bytes_at(1, 10, 8, 128, -1, 0) == 0


def _swa(zg, **over):
    a = dict(q=16, k=16, v=16, gate=16, qw=16, kw=16, out=16, B=1, S=4, Hq=4, Hkv=1, D=128, window=128, R=42,
             base=1e4, eps=1e-6, pos0=0, cache=None, layer=0, ws=16, ws_bytes=1 << 20, stream=None)
    a.update(over)
    return zg._lib.swa_prefill(a["q"], a["k"], a["v"], a["gate"], a["qw"], a["kw"], a["out"], a["B"], a["S"], a["Hq"],
                               a["Hkv"], a["D"], a["window"], a["R"], a["base"], a["eps"], a["pos0"], a["cache"],
                               a["layer"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(D=64), 2), (dict(Hq=6, Hkv=4), 1), (dict(Hq=12, Hkv=1), 2), (dict(window=0), 1), (dict(R=41), 1),
    (dict(R=130), 1), (dict(base=0.0), 1), (dict(eps=-1.0), 1), (dict(pos0=3), 1), (dict(q=None), 1),
    (dict(gate=None), 1), (dict(out=24), 1), (dict(ws=None), 1), (dict(ws_bytes=100), 3), (dict(B=-1), 1),
])
def test_swa_prefill_rejects_bad_arguments(zg, over, status):
    assert _swa(zg, **over) == status
    assert zg._lib.zg_last_error()


def test_noop_sizes_return_ok(zg):
    assert _swa(zg, S=0) == 0
    assert _swa(zg, B=0) == 0


def test_decode_and_cache_reject_bad_arguments(zg):
    lib = zg._lib
    assert lib.hybrid_decode_step(16, 16, 16, 16, 16, 16, 16, None, 32, 42, 1e7, 1e-6, None, None) == 1
    bad = zg._desc(32, [6, 12], 1, 8, 64, 128, 1024)
    h = ctypes.c_void_p()
    assert lib.kv_cache_alloc(ctypes.byref(bad), ctypes.byref(h), None) == 2
    bad = zg._desc(32, [6, 6], 1, 8, 128, 128, 1024)
    assert lib.kv_cache_alloc(ctypes.byref(bad), ctypes.byref(h), None) == 1
    bad = zg._desc(32, [33], 1, 8, 128, 128, 1024)
    assert lib.kv_cache_alloc(ctypes.byref(bad), ctypes.byref(h), None) == 1
    assert lib.kv_cache_free(None) == 0


def test_layer_workspace_bytes_closed_form(zg):
    B, S, Hq, Hkv, D = 2, 300, 32, 8, 128
    act = B * S * (3 * Hq + 2 * Hkv) * D * 2
    act = (act + 255) // 256 * 256
    assert zg.layer_workspace_bytes(B, S, Hq, Hkv, D) == act + zg.workspace_bytes(B, S, Hkv, D)



def test_fp8_layer_workspace_bytes_closed_form(zg):
    B, S, dm, Hq, Hkv, D = 2, 300, 4096, 32, 8, 128
    T = B * S
    a = lambda n: (n + 255) // 256 * 256
    codes = a(T * dm) + a(T * Hq * D) + 2 * a(Hq * D * dm) + 2 * a(Hkv * D * dm) + a(dm * Hq * D)
    assert zg.fp8_layer_workspace_bytes(B, S, dm, Hq, Hkv, D) == zg.layer_workspace_bytes(B, S, Hq, Hkv, D) + codes


def test_fp8_layers_reject_a_null_state(zg):
    args = [16] * 9 + [1, 4, 4096, 4, 1, 128, 128, 42, 1e4, 1e-6, 0, None, 0, None, 256, 1 << 30, None]
    assert zg._lib.gated_swa_layer_fp8(*args) == zg.ZG_EINVAL
    gargs = [16] * 8 + [1, 4, 4096, 4, 1, 128, 42, 1e4, 1e-6, 0, None, 0, None, 256, 1 << 30, None]
    assert zg._lib.global_layer_fp8(*gargs) == zg.ZG_EINVAL
    assert b"null FP8 state" in zg._lib.zg_last_error()

def _layer(zg, **over):
    a = dict(h=16, wq=16, wk=16, wv=16, wg=16, wo=16, qw=16, kw=16, y=16, B=1, S=4, dm=4096, Hq=4, Hkv=1, D=128,
             window=128, R=42, base=1e4, eps=1e-6, pos0=0, cache=None, layer=0, ws=256, ws_bytes=1 << 30, stream=None)
    a.update(over)
    return zg._lib.gated_swa_layer(a["h"], a["wq"], a["wk"], a["wv"], a["wg"], a["wo"], a["qw"], a["kw"], a["y"], a["B"],
                                   a["S"], a["dm"], a["Hq"], a["Hkv"], a["D"], a["window"], a["R"], a["base"], a["eps"],
                                   a["pos0"], a["cache"], a["layer"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(dm=0), 1), (dict(wg=None), 1), (dict(h=24), 1), (dict(ws=None), 1), (dict(ws_bytes=1000), 3),
    # the attention's own arguments are checked before any projection is enqueued
    (dict(window=0), 1), (dict(D=64), 2), (dict(R=41), 1), (dict(pos0=3), 1), (dict(Hq=12, Hkv=1), 2),
])
def test_layer_rejects_bad_arguments_before_enqueueing(zg, over, status):
    assert _layer(zg, **over) == status
    assert zg._lib.zg_last_error()


def test_linear_rejects_bad_arguments(zg):
    lib = zg._lib
    assert lib.linear_bf16(16, 16, 16, 10, 0, 4, None) == 1
    assert lib.linear_bf16(16, 16, 16, -1, 4, 4, None) == 1
    assert lib.linear_bf16(None, 16, 16, 10, 4, 4, None) == 1
    assert lib.linear_bf16(16, 24, 16, 10, 4, 4, None) == 1
    assert lib.linear_bf16(16, 16, 16, 0, 4, 4, None) == 0     # no tokens: no-op
    assert _layer(zg, S=0) == 0


def test_backward_workspace_bytes_closed_form(zg):
    B, S, Hq, Hkv, D = 2, 300, 32, 8, 128
    Sp = (S + 127) // 128 * 128
    a = lambda n: (n + 255) // 256 * 256
    q2, k2, rows = B * Hq * Sp * D * 2, B * Hkv * Sp * D * 2, B * Hq * Sp * 4
    n_blk = B * Hkv * ((S + 31) // 32 + (S + 127) // 128)      # dQ and dK work-groups: dw partials
    want = 4 * a(q2) + 2 * a(rows) + 2 * a(k2) + a(n_blk * D * 4)
    assert zg.backward_workspace_bytes(B, S, Hq, Hkv, D) == want


def _bwd(zg, gated=True, **over):
    a = dict(B=1, S=4, Hq=4, Hkv=1, D=128, W=128, R=42, base=1e4, eps=1e-6, ws=256, ws_bytes=1 << 30, dqw=16, dkw=16,
             ptr=16)
    a.update(over)
    p = a["ptr"]
    if gated:
        return zg._lib.swa_prefill_backward(p, p, p, p, p, p, p, p, p, p, p, p, p, a["dqw"], a["dkw"], a["B"], a["S"],
                                            a["Hq"], a["Hkv"], a["D"], a["W"], a["R"], a["base"], a["eps"], a["ws"],
                                            a["ws_bytes"], None)
    return zg._lib.global_prefill_backward(p, p, p, p, p, p, p, p, p, p, p, a["dqw"], a["dkw"], a["B"], a["S"], a["Hq"],
                                           a["Hkv"], a["D"], a["R"], a["base"], a["eps"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("over,status", [
    (dict(Hq=8, Hkv=1), 2), (dict(D=64), 2), (dict(Hq=6, Hkv=4), 1), (dict(R=43), 1), (dict(eps=-1.0), 1),
    (dict(ptr=None), 1), (dict(dqw=None), 1), (dict(ws_bytes=1024), 3), (dict(ws=None), 1), (dict(ptr=8), 1)])
def test_backward_rejects_bad_arguments_before_enqueueing(zg, gated, over, status):
    assert _bwd(zg, gated, **over) == status, zg._lib.zg_last_error()


def test_swa_backward_rejects_window_zero(zg):
    assert _bwd(zg, True, W=0) == zg.ZG_EINVAL


def test_training_forward_needs_lse(zg):
    p = 16
    rc = zg._lib.swa_prefill_train(p, p, p, p, p, p, p, None, 1, 4, 4, 1, 128, 128, 42, 1e4, 1e-6, 256, 1 << 30, None)
    assert rc == zg.ZG_EINVAL and b"null lse" in zg._lib.zg_last_error()


# ------------------------------------------------------------------------------------------ binding shape checks
# The binding checks every tensor's full shape against q (or the cache) before anything reaches the library; on the
# host these checks run on CPU tensors, which the later device check would refuse anyway.
def _bt(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


def _layer_tensors(B=1, S=8, Hq=4, Hkv=1, D=128):
    return dict(q=_bt(B, S, Hq, D), k=_bt(B, S, Hkv, D), v=_bt(B, S, Hkv, D), gate=_bt(B, S, Hq, D),
                q_norm_w=_bt(D), k_norm_w=_bt(D))


@pytest.mark.parametrize("name,bad", [("k", (1, 7, 1, 128)), ("v", (1, 7, 1, 128)), ("gate", (1, 8, 4, 64)),
                                      ("q_norm_w", (2, 128)), ("k_norm_w", (64,)), ("out", (1, 8, 4, 127))])
def test_binding_rejects_mis_shaped_prefill_tensors(zg, name, bad):
    t = _layer_tensors()
    t[name] = _bt(*bad)
    with pytest.raises(ValueError, match=name):
        zg.swa_prefill(t["q"], t["k"], t["v"], t["gate"], t["q_norm_w"], t["k_norm_w"], t.get("out"))
    if name != "gate":
        with pytest.raises(ValueError, match=name):
            zg.global_prefill(t["q"], t["k"], t["v"], t["q_norm_w"], t["k_norm_w"], t.get("out"))
    with pytest.raises(ValueError, match=name):
        zg.prefill_train(t["q"], t["k"], t["v"], t["gate"], t["q_norm_w"], t["k_norm_w"], out=t.get("out"))


def test_binding_well_shaped_host_tensors_reach_the_device_check(zg):
    t = _layer_tensors()
    with pytest.raises(TypeError, match="CUDA"):
        zg.swa_prefill(t["q"], t["k"], t["v"], t["gate"], t["q_norm_w"], t["k_norm_w"])
    with pytest.raises(ValueError, match="gate is required"):
        zg.swa_prefill(t["q"], t["k"], t["v"], None, t["q_norm_w"], t["k_norm_w"])


def test_binding_rejects_mis_shaped_backward_tensors(zg):
    import torch
    t = _layer_tensors()
    out, dout = _bt(1, 8, 4, 128), _bt(1, 8, 4, 128)
    lse = torch.zeros((1, 4, 8), dtype=torch.float32)
    args = (t["q"], t["k"], t["v"], t["gate"], t["q_norm_w"], t["k_norm_w"], out)
    with pytest.raises(ValueError, match="lse"):
        zg.prefill_backward(*args, torch.zeros((1, 8, 4), dtype=torch.float32), dout)
    with pytest.raises(ValueError, match="dout"):
        zg.prefill_backward(*args, lse, _bt(1, 8, 4, 64))
    with pytest.raises(ValueError, match="dk"):
        zg.prefill_backward(*args, lse, dout, grads={"dk": _bt(1, 8, 4, 128)})
    with pytest.raises(ValueError, match="dq_norm_w"):
        zg.prefill_backward(*args, lse, dout, grads={"dq_norm_w": torch.zeros(64, dtype=torch.float32)})


def test_binding_rejects_decode_tensors_that_do_not_match_the_cache(zg):
    import types
    cache = types.SimpleNamespace(n_layers=3, batch=2, head_dim=128, n_kv_heads=2, handle=None)
    L, B, Hq, Hkv, D = 3, 2, 8, 2, 128
    ok = dict(q=_bt(L, B, Hq, D), k=_bt(L, B, Hkv, D), v=_bt(L, B, Hkv, D), gate=_bt(L, B, Hq, D),
              q_norm_w=_bt(L, D), k_norm_w=_bt(L, D))

    def call(**over):
        a = dict(ok, **over)
        return zg.hybrid_decode_step(a["q"], a["k"], a["v"], a["gate"], a["q_norm_w"], a["k_norm_w"],
                                     a.get("positions", [5, 5]), cache, out=a.get("out"))
    with pytest.raises(ValueError, match="q has shape"):
        call(q=_bt(L, 3, Hq, D))
    # the per-layer norm weights are [L, D] in decode (a [D] vector would be read past its end)
    with pytest.raises(ValueError, match="q_norm_w"):
        call(q_norm_w=_bt(D))
    with pytest.raises(ValueError, match="k has shape"):
        call(k=_bt(L, B, 1, D))
    with pytest.raises(ValueError, match="gate"):
        call(gate=_bt(L, B, Hq + 1, D))
    with pytest.raises(ValueError, match="out"):
        call(out=_bt(L, B, Hq, 64))
    with pytest.raises(ValueError, match="positions"):
        call(positions=[5])
    with pytest.raises(TypeError, match="CUDA"):
        call()


def test_binding_rejects_mis_shaped_layer_tensors(zg):
    B, S, dm, Hq, Hkv, D = 1, 4, 256, 4, 1, 128
    h = _bt(B, S, dm)
    w = dict(w_q=_bt(Hq * D, dm), w_k=_bt(Hkv * D, dm), w_v=_bt(Hkv * D, dm), w_g=_bt(Hq * D, dm),
             w_o=_bt(dm, Hq * D))
    nw = _bt(D)
    for name, bad in (("w_q", (Hq * D, dm + 8)), ("w_k", (Hq * D, dm)), ("w_o", (Hq * D, dm)), ("w_g", (dm, dm))):
        a = dict(w, **{name: _bt(*bad)})
        with pytest.raises(ValueError, match=name):
            zg.gated_swa_layer(h, a["w_q"], a["w_k"], a["w_v"], a["w_g"], a["w_o"], nw, nw, Hq=Hq, Hkv=Hkv)
    with pytest.raises(ValueError, match="y"):
        zg.global_layer(h, w["w_q"], w["w_k"], w["w_v"], w["w_o"], nw, nw, _bt(B, S, dm + 1), Hq=Hq, Hkv=Hkv)
    with pytest.raises(ValueError, match="y has shape"):
        zg.linear_bf16(_bt(3, 256), _bt(128, 256), _bt(3, 64))
    with pytest.raises(ValueError, match="features"):
        zg.linear_bf16(_bt(3, 255), _bt(128, 256))
