"""The shared synthetic-input generator (CPU side): deterministic, windows
agree with whole arrays, distinct streams per key, roughly N(0, sigma)."""

import numpy as np

import synth


def test_deterministic_and_windowed():
    a = synth.cpu_normal_f32(10_000, 0, synth.TAG_MASTER, 0, 0, 0, 0.02)
    b = synth.cpu_normal_f32(10_000, 0, synth.TAG_MASTER, 0, 0, 0, 0.02)
    assert np.array_equal(a, b)
    w = synth.cpu_normal_f32(1000, 0, synth.TAG_MASTER, 0, 0, 4321, 0.02)
    assert np.array_equal(w, a[4321:5321])
    g = synth.cpu_normal_bf16(5000, 0, synth.TAG_GRAD, 3, 2, 0, 1e-3)
    gw = synth.cpu_normal_bf16(100, 0, synth.TAG_GRAD, 3, 2, 777, 1e-3)
    assert np.array_equal(gw, g[777:877])


def test_streams_differ():
    base = synth.cpu_normal_bf16(4096, 0, synth.TAG_GRAD, 1, 0, 0, 1e-3)
    for args in [(1, synth.TAG_GRAD, 1, 0), (0, synth.TAG_GRAD, 2, 0),
                 (0, synth.TAG_GRAD, 1, 1), (0, synth.TAG_MASTER, 1, 0)]:
        other = synth.cpu_normal_bf16(4096, args[0], args[1], args[2],
                                      args[3], 0, 1e-3)
        assert np.mean(other == base) < 0.05


def test_moments():
    x = synth.cpu_normal_f32(1 << 20, 0, synth.TAG_GRAD, 0, 0, 0, 1e-4)
    assert abs(x.mean()) < 3e-7
    assert abs(x.std() / 1e-4 - 1) < 3e-3
    # Irwin-Hall(12) tails: bounded by 6 sigma, fourth moment 2.9 (normal: 3)
    z = x.astype(np.float64) / 1e-4
    assert np.abs(z).max() <= 6.0
    assert abs(np.mean(z ** 4) - 2.9) < 0.05
    v = synth.cpu_normal_f32(4096, 0, synth.TAG_V, 0, 0, 0, 1e-8, absval=True)
    assert (v >= 0).all()
    bits = synth.cpu_normal_bf16(1 << 16, 0, synth.TAG_GRAD, 0, 0, 0, 1e-3)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    assert abs(f.std() / 1e-3 - 1) < 2e-2
