"""Seeded input generator: determinism, shapes and the stated distributions."""
import numpy as np

from quantized_moe_decode_affine_amd import synth


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 0.0], dtype=np.float64)
    # 1+2^-8 is halfway between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 -> 1+2^-6 (even mantissa)
    assert list(synth.to_bf16_bits(f)) == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x0000]


def test_q4_matrix_is_deterministic_and_distributed():
    a = synth.q4_matrix(1, 2, 3, 0, 256, 512)
    b = synth.q4_matrix(1, 2, 3, 0, 256, 512)
    c = synth.q4_matrix(1, 2, 3, 1, 256, 512)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    codes, scales, biases = a
    assert codes.shape == (256, 64) and scales.shape == (256, 8) and biases.shape == (256, 8)
    nib = np.stack([(codes >> (4 * i)) & 0xF for i in range(8)]).ravel()
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.85 * nib.size / 16
    s = (scales.astype(np.uint32) << 16).view(np.float32)
    b = (biases.astype(np.uint32) << 16).view(np.float32)
    assert np.all(s >= 0) and 0.012 < s.mean() < 0.020          # |N(0,0.02)| has mean 0.016
    assert np.abs(b + 8 * s).max() < 0.02                       # bias = -8 scale + N(0, 0.002)


def test_layer_shapes_and_shared_expert():
    layer = synth.moe_layer(1, 0, 128, 64, 4, 2, threads=2)
    assert layer.gate.codes.shape == (4, 64, 16) and layer.down.codes.shape == (4, 128, 8)
    assert layer.sh_gate.codes.shape == (1, 64, 16) and layer.router.shape == (4, 128)
    g, u, d = layer.expert(4)
    np.testing.assert_array_equal(g[0], layer.sh_gate.codes[0])
    single = synth.moe_layer(1, 0, 128, 64, 4, 2, threads=1)
    np.testing.assert_array_equal(single.down.codes, layer.down.codes)


def test_fnv1a64_known_values():
    assert synth.fnv1a64(np.array([], dtype=np.int32)) == 0xCBF29CE484222325
    # FNV-1a 64 of the bytes 00 00 00 00
    h = 0xCBF29CE484222325
    for _ in range(4):
        h = ((h ^ 0) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    assert synth.fnv1a64(np.array([0], dtype=np.int32)) == h
    a = np.arange(12, dtype=np.int32).reshape(3, 4)
    assert synth.fnv1a64(a) == synth.fnv1a64(a.ravel())
