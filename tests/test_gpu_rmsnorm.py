"""RMS normalisation before the quantiser on the GPU, against the oracle.

The kernels accumulate the mean of squares in fp64 (relative error at most
(K + 2) 2^-53); the oracle rounds the exact mean.  The two agree unless a
row's exact mean lies within that error of an fp32 rounding boundary; for such
a row both roundings are admissible, and the row is checked against the
oracle's result for the one the GPU took (the oracle follows either through
the rest of the path).  Everything after the mean -- X~, x_scale, x_sum,
accumulators -- is then compared exactly.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import bitlinear_oracle as O
from synth import make_acts, make_weight
from tests.gpu_common import assert_equal, check_y, dev, f32_bits, host

pytestmark = pytest.mark.gpu


def _gain(K, name):
    return (1.0 + make_weight(0, name, 1, K, 0.1)[0]).astype(np.float32)


def _acts(M, K, name):
    return make_acts(0, name, M, K, {"outlier_frac": Fraction(1, 100), "outlier_scale": 50.0})


def oracle_rms_quant(X, g, got_xq=None):
    """The oracle's X~, x_scale, x_sum per row, at the admissible rounding of
    the mean of squares that matches the GPU's X~ (the correctly rounded one
    when the row has only that), and the number of rows with two."""
    M, K = X.shape
    cands = O.mean_square_candidates(X, (K + 2) * 2.0 ** -53)
    Xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    xsum = np.empty(M, np.int64)
    for m in range(M):
        options = []
        for c in cands[m]:
            Y, _ = O.rmsnorm(X[m:m + 1], g, ms=[c])
            q, s, t, _ = O.quantize_activations(Y)
            options.append((q[0], s[0], t[0]))
        pick = options[0]
        if got_xq is not None:
            for o in options[1:]:
                if np.array_equal(o[0], got_xq[m]):
                    pick = o
        Xq[m], xs[m], xsum[m] = pick
    return Xq, xs, xsum, sum(len(c) > 1 for c in cands)


RMS_SHAPES = [
    # (M, K): one group of four per thread up to 16 (register rows), 1024
    # threads past 12288 values (register rows up to 32768, then looped), the
    # decode and prefill widths, ragged K
    (1, 16), (3, 64), (2, 1040), (2, 3200), (4, 8192), (1, 12288), (1, 12304), (2, 16384),
    (3, 16400), (2, 28672), (1, 32768), (2, 32784), (1, 65536),
]


@pytest.mark.parametrize("M,K", RMS_SHAPES, ids=[f"M{m}K{k}" for m, k in RMS_SHAPES])
def test_rmsnorm_quant(gpu_lib, M, K):
    X = _acts(M, K, f"test/rms/X{M}x{K}")
    g = _gain(K, f"test/rms/g{K}")
    q, s, t = gpu_lib.bitlinear_rmsnorm_quant(dev(X), dev(g))
    gq = host(q)
    Xq, xs, xsum, amb = oracle_rms_quant(X, g, gq)
    assert_equal(gq, Xq, "X~")
    assert_equal(f32_bits(host(s)), f32_bits(xs), "x_scale")
    assert_equal(host(t).astype(np.int64), xsum, "x_sum")


def test_rmsnorm_quant_special_rows(gpu_lib):
    # a zero row, a constant row, rows of tiny and of huge magnitude (the mean
    # of squares underflows fp32 / needs fp64 range), one spike
    K = 4096
    X = np.zeros((6, K), np.float32)
    X[1] = 3.0
    X[2] = np.float32(1e-25) * _acts(1, K, "test/rms/tiny")[0]
    X[3] = np.float32(1e18) * _acts(1, K, "test/rms/huge")[0]
    X[4, 17] = -5.0
    X[5] = _acts(1, K, "test/rms/plain")[0]
    g = _gain(K, "test/rms/gspecial")
    q, s, t = gpu_lib.bitlinear_rmsnorm_quant(dev(X), dev(g))
    Xq, xs, xsum, _ = oracle_rms_quant(X, g, host(q))
    assert_equal(host(q), Xq, "X~")
    assert_equal(f32_bits(host(s)), f32_bits(xs), "x_scale")
    assert_equal(host(t).astype(np.int64), xsum, "x_sum")
    assert not host(q)[0].any()


FWD_RMS = [
    # (M, N, K): one token fused into the vector-ALU decode (pieces per lane
    # 1, 2, 3), one token past the fused range, several tokens (two launches:
    # normalising quantiser, then the matrix decode or the GEMM)
    (1, 8640, 3200), (1, 77, 192), (1, 3200, 8640), (1, 5, 12288), (1, 9, 12352),
    (4, 100, 4096), (40, 130, 1024),
]


@pytest.mark.parametrize("M,N,K", FWD_RMS, ids=[f"M{m}N{n}K{k}" for m, n, k in FWD_RMS])
def test_forward_rmsnorm(gpu_lib, M, N, K):
    import torch
    W = make_weight(0, f"test/rmsf/W{N}x{K}", N, K, 0.02)
    X = _acts(M, K, f"test/rmsf/X{M}x{K}")
    g = _gain(K, f"test/rmsf/g{K}")
    gamma = O.absmean_gamma(W)
    Wt = O.ternarize(W, gamma)
    P = dev(O.pack_codes(Wt))
    gd = dev(np.array([gamma], np.float32))
    outs = dict(X_q_out=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                x_scale_out=torch.empty(M, dtype=torch.float32, device="cuda"),
                x_sum_out=torch.empty(M, dtype=torch.int32, device="cuda"))
    acc = gpu_lib.bitlinear_forward_rmsnorm(P, gd, dev(X), dev(g), N=N, y_dtype="i32", **outs)
    torch.cuda.synchronize()
    gq = host(outs["X_q_out"])
    Xq, xs, xsum, _ = oracle_rms_quant(X, g, gq)
    assert_equal(gq, Xq, "X~ out")
    assert_equal(f32_bits(host(outs["x_scale_out"])), f32_bits(xs), "x_scale out")
    assert_equal(host(outs["x_sum_out"]).astype(np.int64), xsum, "x_sum out")
    want = O.integer_matmul(Wt, Xq)
    assert_equal(host(acc).astype(np.int64), want, "accumulators")
    # the fused launch and the standalone normalising quantiser sum in the same
    # order: identical codes
    q2, s2, _ = gpu_lib.bitlinear_rmsnorm_quant(dev(X), dev(g))
    assert_equal(host(q2), gq, "standalone vs fused X~")
    # the rescale uses the absmax of the normalised row (an admissible other
    # rounding of the mean moves it by far less than the tolerance)
    _, _, _, beta = O.quantize_activations(O.rmsnorm(X, g)[0])
    for out in ("f32", "bf16"):
        Y = gpu_lib.bitlinear_forward_rmsnorm(P, gd, dev(X), dev(g), N=N, y_dtype=out)
        check_y(Y, O.rescale(want, gamma, beta), out)


RMS_GROUPS = [(1, 4096, (4096, 1024, 1024)), (1, 3200, (3200, 640)), (3, 4096, (512, 200))]


@pytest.mark.parametrize("M,K,Ns", RMS_GROUPS, ids=[f"M{m}K{k}G{len(n)}" for m, k, n in RMS_GROUPS])
def test_forward_rmsnorm_grouped(gpu_lib, M, K, Ns):
    import torch
    X = _acts(M, K, f"test/rmsg/X{M}x{K}")
    g = _gain(K, f"test/rmsg/g{K}")
    Ws = [make_weight(0, f"test/rmsg/W{i}_{n}x{K}", n, K, 0.02) for i, n in enumerate(Ns)]
    gammas = [O.absmean_gamma(W) for W in Ws]
    Wts = [O.ternarize(W, gm) for W, gm in zip(Ws, gammas)]
    Ps = [dev(O.pack_codes(Wt)) for Wt in Wts]
    gds = [dev(np.array([gm], np.float32)) for gm in gammas]
    outs = dict(X_q_out=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                x_scale_out=torch.empty(M, dtype=torch.float32, device="cuda"),
                x_sum_out=torch.empty(M, dtype=torch.int32, device="cuda"))
    accs = gpu_lib.bitlinear_forward_rmsnorm_grouped(Ps, gds, dev(X), dev(g), y_dtype="i32", **outs)
    torch.cuda.synchronize()
    gq = host(outs["X_q_out"])
    Xq, _, _, _ = oracle_rms_quant(X, g, gq)
    assert_equal(gq, Xq, "X~ out")
    for i, (Wt, a) in enumerate(zip(Wts, accs)):
        assert_equal(host(a).astype(np.int64), O.integer_matmul(Wt, Xq), f"accumulators {i}")
