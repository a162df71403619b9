"""The seeded input generator: determinism, chunk independence, recipe counts."""
from fractions import Fraction

import numpy as np

from synth import (WORKLOADS, outlier_channels, splitmix64_mix, standard_normal,
                   stream_key, student_t3, uniform53)


def test_splitmix64_published_first_outputs():
    # SplitMix64 seeded with 0: state advances by 0x9E3779B97F4A7C15 before each
    # output; the first outputs of that sequence are widely tabulated.
    states = (np.arange(1, 4, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15))
    got = [int(v) for v in splitmix64_mix(states)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_streams_are_counter_based():
    k = stream_key(0, "t/x")
    a = standard_normal(k, 0, 1001)
    b = np.concatenate([standard_normal(k, 0, 333), standard_normal(k, 333, 668)])
    assert (a == b).all()
    assert (standard_normal(k, 17, 50) == a[17:67]).all()
    u = uniform53(k, 0, 10000)
    assert u.min() > 0 and u.max() < 1
    assert stream_key(0, "t/x") != stream_key(1, "t/x") != stream_key(0, "t/y")


def test_normal_and_t3_moments():
    k = stream_key(0, "t/moments")
    z = standard_normal(k, 0, 400000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    t = student_t3(k, 0, 400000)
    # Student-t(3): variance 3, heavy tails (P(|t| > 5) = 0.0154)
    assert abs(np.mean(np.abs(t) > 5) - 0.0154) < 0.002


def test_outlier_counts_round_half_up():
    k = stream_key(0, "t/ch")
    assert len(outlier_channels(k, 512, Fraction(1, 100))) == 5
    assert len(outlier_channels(k, 4096, Fraction(1, 200))) == 20
    assert len(outlier_channels(k, 11008, Fraction(1, 200))) == 55
    assert len(outlier_channels(k, 4096, Fraction(1, 100))) == 41
    ch = outlier_channels(k, 4096, Fraction(1, 100))
    assert len(set(ch.tolist())) == 41 and ch.min() >= 0 and ch.max() < 4096


def test_workload_tensors_deterministic():
    wl = WORKLOADS["layer-512x256"]
    p = wl.projections[0]
    W1, W2 = wl.weight(p), wl.weight(p)
    assert W1.dtype == np.float32 and W1.shape == (256, 512) and (W1 == W2).all()
    X = wl.acts(p, 4)
    assert X.shape == (4, 512) and X.dtype == np.float32
    # 5 outlier channels scaled x50: those columns dominate the absmax
    big = np.argsort(np.abs(X).max(axis=0))[-5:]
    assert np.abs(X[:, big]).max() > 20 * np.abs(np.delete(X, big, axis=1)).max() / 5
