"""Seeded generators: deterministic, the stated shapes and laws, packed sizes
consistent with the oracle's own byte count."""
import numpy as np

import oracle
from decode_gemv_elementwise_amd import synth


def test_generators_deterministic_and_seeded():
    a = synth.f32_tiny_256(0)
    b = synth.f32_tiny_256(0)
    c = synth.f32_tiny_256(1)
    assert np.array_equal(a.weights["W"].data, b.weights["W"].data)
    for k in a.vectors:
        assert np.array_equal(a.vectors[k], b.vectors[k])
    assert not np.array_equal(a.weights["W"].data, c.weights["W"].data)


def test_tiny_workload_laws():
    wl = synth.f32_tiny_256(0)
    W = wl.weights["W"].data.view(np.float32)
    assert W.size == 256 * 256
    assert abs(W.std() - 1 / 16) < 0.01 * (1 / 16) * 10
    assert [c.act for c in wl.calls] == list(synth.ACTS)


def test_block_laws_and_sizes():
    rng = np.random.default_rng(0)
    w8 = synth.draw_q8b32(rng, 64, 256, 0.001, 0.01)
    assert w8.codes.min() >= -127 and w8.codes.max() <= 127
    assert 0.001 * 0.999 <= float(w8.scales.min()) and float(w8.scales.max()) <= 0.01 * 1.001
    w4 = synth.draw_q4b32(rng, 64, 256, 0.001, 0.02)
    assert w4.codes.min() == 0 and w4.codes.max() == 15
    for w in (w8, w4):
        assert w.data.size == oracle.weight_bytes(w.fmt, w.N, w.K) == synth.weight_nbytes(w.fmt, w.N, w.K)


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is exactly half-way between bf16 neighbours 1 and 1 + 2^-7: ties to even (1.0)
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], dtype=np.float32)
    bits = synth.bf16_bits_from_f32(vals)
    assert list(bits) == [0x3F80, 0x3F82, 0xC020, 0x0000]


def test_layer_chain_shapes():
    wl = synth.q4b32_decode_layer(0)
    shapes = {k: (w.N, w.K) for k, w in wl.weights.items()}
    assert shapes == {"Wqkv": (6144, 4096), "Wo": (4096, 4096), "Wgate": (14336, 4096),
                      "Wup": (14336, 4096), "Wdown": (4096, 14336), "Wg": (32, 4096)}
    assert [c.act for c in wl.calls] == ["none", "add", "silu", "mul", "add", "sigmoid"]
