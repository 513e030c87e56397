"""The seeded generator: determinism, regenerable slices, stated distributions."""
import numpy as np

import synth


def test_same_seed_same_bytes_and_slices():
    a = synth.q4_0_matrix(1, "w", 700, 512)
    b = synth.q4_0_matrix(1, "w", 700, 512)
    assert np.array_equal(a, b)
    assert np.array_equal(synth.q4_0_matrix(1, "w", 700, 512, rows=(123, 611)), a[123:611])
    assert not np.array_equal(synth.q4_0_matrix(2, "w", 700, 512), a)
    assert not np.array_equal(synth.q4_0_matrix(1, "w2", 700, 512), a)
    c = synth.q8_0_matrix(1, "e", 300, 256)
    assert np.array_equal(synth.q8_0_matrix(1, "e", 300, 256, rows=(5, 17)), c[5:17])


def test_q4_0_distributions():
    w = synth.q4_0_matrix(3, "dist", 2000, 256).reshape(-1, 18)
    d = w[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    assert d.min() >= 0.005 - 1e-5 and d.max() <= 0.02 + 1e-5
    codes = np.concatenate([w[:, 2:] & 15, w[:, 2:] >> 4]).ravel()
    counts = np.bincount(codes, minlength=16)
    assert counts.min() > 0.9 * codes.size / 16


def test_q8_0_distributions():
    w = synth.q8_0_matrix(3, "dist8", 2000, 256).reshape(-1, 34)
    d = w[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    assert d.min() >= 0.002 - 1e-5 and d.max() <= 0.01 + 1e-5
    q = w[:, 2:].view(np.int8).astype(np.int64)
    assert q.min() == -127 and q.max() == 127


def test_dense_distributions():
    x = synth.normal_f32(4, "x", (3_000_000,))
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    u = synth.uniform_f32(4, "u", (100_000,), 0.8, 1.2)
    assert u.min() >= 0.8 and u.max() <= 1.2
    t = synth.tokens(4, "t", 1000, 151936)
    assert t.min() >= 0 and t.max() < 151936 and t.dtype == np.int32
