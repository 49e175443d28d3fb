"""The seeded input generator (CPU side): determinism, stream separation and table shape."""
import numpy as np

import synth


def test_table_is_symmetric_standard_normal_quantiles():
    t = synth.bf16_bits_to_f64(synth.TABLE)
    np.testing.assert_array_equal(t, -t[::-1])
    assert np.all(np.diff(t) >= 0)
    assert abs(t.mean()) < 1e-12 and abs(t.std() - 1.0) < 2e-3


def test_streams_are_deterministic_and_index_addressable():
    a = synth.normal_bf16(1002, 3, synth.TENSOR_Q, (4, 5, 6))
    b = synth.normal_bf16(1002, 3, synth.TENSOR_Q, (4, 5, 6))
    np.testing.assert_array_equal(a, b)
    idx = np.array([0, 7, 119])
    np.testing.assert_array_equal(synth.normal_bf16_at(1002, 3, synth.TENSOR_Q, idx), a.reshape(-1)[idx])
    tail = synth.normal_bf16(1002, 3, synth.TENSOR_Q, (20,), index_offset=100)
    np.testing.assert_array_equal(tail, a.reshape(-1)[100:120])


def test_streams_differ_across_seed_layer_tensor():
    base = synth.normal_bf16(1, 0, 0, (4096,))
    for other in (synth.normal_bf16(2, 0, 0, (4096,)), synth.normal_bf16(1, 1, 0, (4096,)),
                  synth.normal_bf16(1, 0, 1, (4096,))):
        assert np.mean(base == other) < 0.05


def test_norm_weights():
    w = synth.bf16_bits_to_f64(synth.norm_weight_bf16(1002, 0, synth.TENSOR_WQ, 128))
    assert abs(w.mean() - 1.0) < 0.05 and 0.02 < w.std() < 0.2
    np.testing.assert_array_equal(synth.bf16_bits_to_f64(synth.norm_weight_bf16(1, 0, 4, 128, spread=0.0)), 1.0)
