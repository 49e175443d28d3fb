"""Host logic of the schedule sweep (bench.py --schedule-sweep): layer placements, the composition of
measured per-layer times into 32-layer schedules, and the KV footprint of each schedule.

The 5:1 placement and the 32.0 vs 5.0 GiB footprints at 262,144 tokens are the pages' (onedev.kr "How it
works"; jaehun.me "Why the KV Cache Shrinks by 6.4x"); 3:1 and 1:1 are the sweep's own intermediate points.
"""
import os

import pytest

import bench
import oracle

GIB = 2 ** 30
RING_BYTES = 128 * 2 * 8 * 128 * 2          # one SWA layer's full ring: W positions x (K, V) x Hkv x D x bf16


def test_schedule_placements():
    assert bench.schedule_globals("5:1") == (6, 12, 18, 24, 30)
    assert bench.schedule_globals("3:1") == tuple(range(4, 33, 4))
    assert bench.schedule_globals("1:1") == tuple(range(2, 33, 2))
    assert bench.schedule_globals("all-global") == tuple(range(1, 33))
    for name, swa_per_global in (("5:1", 5), ("3:1", 3), ("1:1", 1)):
        g = bench.schedule_globals(name)
        # the last global layer is followed by at most swa_per_global SWA layers, every earlier gap is exact
        gaps = [b - a - 1 for a, b in zip((0,) + g, g)]
        assert set(gaps) == {swa_per_global}, name


def test_compose_sums_measured_layer_times():
    per_layer = {4096: {"swa": 1.0, "global": 10.0}, 262144: {"swa": 64.0, "global": 6400.0}}
    out = bench.compose_schedules(per_layer, lambda S, g: oracle.kv_footprint_bytes(S, global_layer_ids=g))
    r = {name: {x["seq_len"]: x for x in out[name]["by_length"]} for name in bench.SCHEDULES}
    assert r["5:1"][4096]["attention_ms"] == 27 * 1.0 + 5 * 10.0
    assert r["3:1"][4096]["attention_ms"] == 24 * 1.0 + 8 * 10.0
    assert r["1:1"][4096]["attention_ms"] == 16 * 1.0 + 16 * 10.0
    assert r["all-global"][262144]["attention_ms"] == 32 * 6400.0
    assert r["5:1"][262144]["speedup_vs_all_global"] == pytest.approx(32 * 6400.0 / (27 * 64.0 + 5 * 6400.0))
    assert r["all-global"][4096]["speedup_vs_all_global"] == 1.0
    assert r["5:1"][4096]["tokens_per_s"] == pytest.approx(4096 / 0.077)
    # the pages' footprints at 256K: 32.0 GiB for full attention, 5.0 GiB (+ 27 rings) for the 5:1 hybrid
    assert r["all-global"][262144]["kv_cache_bytes"] == 32 * GIB
    assert r["5:1"][262144]["kv_cache_bytes"] == 5 * GIB + 27 * RING_BYTES
    assert r["5:1"][262144]["kv_ratio_all_global"] == pytest.approx(6.4, rel=3e-3)


@pytest.mark.skipif(not os.path.exists(os.path.join(os.path.dirname(bench.__file__), "global_attention_gated_amd",
                                                    "libzgattn.so")), reason="library not built")
def test_library_footprint_matches_oracle_for_every_schedule():
    import global_attention_gated_amd as zg
    for name in bench.SCHEDULES:
        g = bench.schedule_globals(name)
        for S in (1, 127, 128, 129, 4096, 16384, 65536, 262144):
            assert zg.footprint_bytes(S, global_layers=g) == oracle.kv_footprint_bytes(S, global_layer_ids=g), (name, S)
