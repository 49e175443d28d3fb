"""The allocation-free global prefill (global_prefill_noalloc), through the C ABI, against global_prefill on the same
inputs: two calls in a row, the second smaller (the scratch array keeps the first call's contents), a call against
a KV cache, and a call whose staging exceeds the scratch array (ERANGE before anything is enqueued)."""
import ctypes

import numpy as np
import pytest

from _inputs import Layer, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zg():
    import torch
    assert torch.cuda.is_available()
    import global_attention_gated_amd as m
    return m


def _noalloc(zg, L, out, pos0=0, cache=None, layer=0):
    """One call of the C entry point itself (ctypes), on torch's current stream."""
    import torch
    B, S, Hq, D = L.dq.shape
    Hkv = L.dk.shape[2]
    return zg._lib.global_prefill_noalloc(L.dq.data_ptr(), L.dk.data_ptr(), L.dv.data_ptr(), L.dwq.data_ptr(),
                                          L.dwk.data_ptr(), out.data_ptr(), B, S, Hq, Hkv, D, 42, 1e4, 1e-6, pos0,
                                          None if cache is None else cache.handle, layer,
                                          torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_global_prefill_on_two_calls(zg):
    import torch
    assert zg._lib.global_prefill_noalloc_max_bytes() == 64 << 20
    for seed, (B, S, Hq, Hkv) in ((61, (2, 1000, 8, 2)), (62, (1, 129, 4, 1))):     # the second call is smaller
        L = Layer(seed, 6, B, S, Hq, Hkv, gated=False)
        out = torch.empty_like(L.dq)
        assert _noalloc(zg, L, out) == zg.ZG_OK, zg._lib.zg_last_error()
        ref = zg.global_prefill(L.dq, L.dk, L.dv, L.dwq, L.dwk, rotary_dims=42, rope_base=1e4, eps=1e-6)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host_bits(out), to_host_bits(ref))


def test_noalloc_with_a_cache_matches_global_prefill(zg):
    import torch
    B, Hq, Hkv, S = 1, 8, 2, 300
    ca = zg.KVCache(n_layers=1, global_layers=[1], batch=B, n_kv_heads=Hkv, max_tokens=1024)
    cb = zg.KVCache(n_layers=1, global_layers=[1], batch=B, n_kv_heads=Hkv, max_tokens=1024)
    pos0 = 0
    for c in range(2):
        L = Layer(63, 1, B, S, Hq, Hkv, gated=False, pos0=pos0, S_total=2 * S)
        out = torch.empty_like(L.dq)
        assert _noalloc(zg, L, out, pos0=pos0, cache=ca, layer=1) == zg.ZG_OK, zg._lib.zg_last_error()
        ref = zg.global_prefill(L.dq, L.dk, L.dv, L.dwq, L.dwk, rotary_dims=42, rope_base=1e4, eps=1e-6, pos0=pos0,
                                cache=cb, layer=1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host_bits(out), to_host_bits(ref))
        pos0 += S
    ka, va = ca.read_layer(1)
    kb, vb = cb.read_layer(1)
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    ca.close()
    cb.close()


def test_noalloc_beyond_the_scratch_array_is_erange(zg):
    import torch
    # 8 KV heads x 40,000 keys: 160 MiB of staged tiles against the 64 MiB array
    q = torch.empty((1, 40000, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, 40000, 8, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    rc = zg._lib.global_prefill_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), w.data_ptr(), w.data_ptr(),
                                        q.data_ptr(), 1, 40000, 8, 8, 128, 42, 1e4, 1e-6, 0, None, 0, None)
    assert rc == zg.ZG_ERANGE and b"scratch" in zg._lib.zg_last_error()
