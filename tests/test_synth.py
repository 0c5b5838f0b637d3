"""The seeded input generators: determinism, field ranges, benign scales."""

import numpy as np

import synth


def test_deterministic_and_role_separated():
    a = synth.weights(synth.Q4_K, synth.rng(1, 2, 3, 0), 8, 512)
    b = synth.weights(synth.Q4_K, synth.rng(1, 2, 3, 0), 8, 512)
    c = synth.weights(synth.Q4_K, synth.rng(1, 2, 4, 0), 8, 512)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.shape == (8, 2 * 144) and a.dtype == np.uint8


def _f16_at(blk, off):
    return (blk[..., off].astype(np.uint16) | (blk[..., off + 1].astype(np.uint16) << 8)).view(np.float16)


def test_field_ranges():
    q6 = synth.weights(synth.Q6_K, synth.rng(2), 64, 512).reshape(64, 2, 210)
    sc = q6[..., 192:208].view(np.int8)
    assert sc.min() == -32 and sc.max() == 31
    d6 = _f16_at(q6, 208).astype(np.float64)
    assert np.all(np.isfinite(d6)) and np.all(d6 >= 0) and d6.max() < 2.0 ** -9 * 8
    q8 = synth.weights(synth.Q8_0, synth.rng(3), 64, 1024).reshape(64, 32, 34)
    qv = q8[..., 2:].view(np.int8)
    assert qv.min() >= -127 and qv.max() <= 127
    q4 = synth.weights(synth.Q4_K, synth.rng(4), 64, 512).reshape(64, 2, 144)
    for off in (0, 2):
        d = _f16_at(q4, off).astype(np.float64)
        assert np.all(np.isfinite(d)) and np.all(d >= 0)


def test_integer_mode_sets_unit_scales():
    q4 = synth.weights(synth.Q4_K, synth.rng(5), 4, 256, mode="integer")
    assert q4[0, 0] == 0x00 and q4[0, 1] == 0x3C and q4[0, 2] == 0x00 and q4[0, 3] == 0x3C


def test_activations():
    x = synth.activations(synth.rng(6, role=1), 16, 64)
    v = x.view(np.float16).astype(np.float64)
    assert x.dtype == np.uint16 and abs(v.mean()) < 0.3 and 0.7 < v.std() < 1.3
    xi = synth.activations(synth.rng(6, role=1), 16, 64, mode="integer").view(np.float16)
    assert set(np.unique(xi.astype(np.float64))) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
