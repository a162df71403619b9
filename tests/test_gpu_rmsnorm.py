"""RMS normalisation before the quantiser on the GPU, against the oracle.

The kernels sum the squares exactly and round the mean once, as the oracle
does, so X~, x_scale, x_sum and the accumulators are compared exactly with
the oracle's single value for every row.
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


def oracle_rms_quant(X, g):
    """The oracle's X~, x_scale and x_sum of the normalised rows."""
    Y, _ = O.rmsnorm(X, g)
    Xq, xs, xsum, _ = O.quantize_activations(Y)
    return Xq, xs, xsum


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
    Xq, xs, xsum = oracle_rms_quant(X, g)
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
    Xq, xs, xsum = oracle_rms_quant(X, g)
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
    Xq, xs, xsum = oracle_rms_quant(X, g)
    assert_equal(gq, Xq, "X~ out")
    assert_equal(f32_bits(host(outs["x_scale_out"])), f32_bits(xs), "x_scale out")
    assert_equal(host(outs["x_sum_out"]).astype(np.int64), xsum, "x_sum out")
    want = O.integer_matmul(Wt, Xq)
    assert_equal(host(acc).astype(np.int64), want, "accumulators")
    # the fused launch and the standalone normalising quantiser give the same
    # codes (both equal the oracle's)
    q2, s2, _ = gpu_lib.bitlinear_rmsnorm_quant(dev(X), dev(g))
    assert_equal(host(q2), gq, "standalone vs fused X~")
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
    Xq, _, _ = oracle_rms_quant(X, g)
    assert_equal(gq, Xq, "X~ out")
    for i, (Wt, a) in enumerate(zip(Wts, accs)):
        assert_equal(host(a).astype(np.int64), O.integer_matmul(Wt, Xq), f"accumulators {i}")


def _exactness_rows(K):
    """Rows whose mean of squares needs the exact sum: a tie between two fp32
    values (to even), the same tie broken by one value 2^60 times smaller
    (below the first summation window, and below any fp64 sum's resolution),
    values spread from subnormals to 2^40 (several windows), subnormals only,
    and one value beside zeros at the bottom of the range."""
    a = np.float32(1.0) + np.float32(2.0 ** -12)
    rows = np.zeros((6, K), np.float32)
    rows[0, : K // 2] = a
    rows[1, : K // 2] = a
    rows[1, K // 2 + 3] = np.float32(2.0 ** -60)
    rng = np.random.default_rng(99)
    e = rng.integers(-149, 41, K)
    rows[2] = (np.where(rng.random(K) < 0.5, -1.0, 1.0) * rng.uniform(1, 2, K) * 2.0 ** e).astype(np.float32)
    rows[3] = (rng.integers(-(1 << 23), 1 << 23, K) * 2.0 ** -149).astype(np.float32)
    rows[4, 7] = np.float32(2.0 ** -149)
    rows[5, : K // 2] = a
    rows[5, K // 2:] = np.float32(2.0 ** -100) * rng.standard_normal(K // 2).astype(np.float32)
    return rows


@pytest.mark.parametrize("K", [64, 4096, 16384, 65536])
def test_rmsnorm_exact_mean_rows(gpu_lib, K):
    # Rows through the first summation window only, and rows that take the
    # further windows (values more than 2^31 below the row's largest), in the
    # register-resident and the looped kernels.
    X = _exactness_rows(K)
    g = _gain(K, f"test/rms/gexact{K}")
    q, s, t = gpu_lib.bitlinear_rmsnorm_quant(dev(X), dev(g))
    Xq, xs, xsum = oracle_rms_quant(X, g)
    assert_equal(host(q), Xq, "X~")
    assert_equal(f32_bits(host(s)), f32_bits(xs), "x_scale")
    assert_equal(host(t).astype(np.int64), xsum, "x_sum")
    ms = O.mean_square(X)
    assert ms[0] != ms[1]          # the tail value decides the rounding


@pytest.mark.parametrize("K", [64, 3200, 12288])
def test_forward_rmsnorm_exact_mean_rows_fused(gpu_lib, K):
    # the same rows through the single-token fused launch (one row at a time)
    import torch
    N = 48
    W = make_weight(0, f"test/rmsx/W{N}x{K}", N, K, 0.02)
    gamma = O.absmean_gamma(W)
    Wt = O.ternarize(W, gamma)
    P = dev(O.pack_codes(Wt))
    gd = dev(np.array([gamma], np.float32))
    g = _gain(K, f"test/rms/gexactf{K}")
    X = _exactness_rows(K)
    assert gpu_lib.forward_kernel("rmsnorm", 1, [N], K) == ("k_decode_dot", True)
    for m in range(X.shape[0]):
        xq = torch.empty((1, K), dtype=torch.int8, device="cuda")
        xs = torch.empty(1, dtype=torch.float32, device="cuda")
        xsum = torch.empty(1, dtype=torch.int32, device="cuda")
        acc = gpu_lib.bitlinear_forward_rmsnorm(P, gd, dev(X[m:m + 1]), dev(g), N=N, y_dtype="i32",
                                                X_q_out=xq, x_scale_out=xs, x_sum_out=xsum)
        torch.cuda.synchronize()
        Xq, s_, t_ = oracle_rms_quant(X[m:m + 1], g)
        assert_equal(host(xq), Xq, f"X~ row {m}")
        assert_equal(f32_bits(host(xs)), f32_bits(s_), f"x_scale row {m}")
        assert_equal(host(xsum).astype(np.int64), t_, f"x_sum row {m}")
        assert_equal(host(acc).astype(np.int64), O.integer_matmul(Wt, Xq), f"accumulators row {m}")
