"""GPU parity of 4-bit activations (A4: values in [-7, 7], one per int8
element, x_scale = beta / 7) against the CPU oracle: the quantiser's
outputs bit-exact, and the projection kernels' accumulators exact and
outputs within tolerance on them."""
import numpy as np
import pytest

from oracle import bitlinear_oracle as O
from synth import make_acts, make_weight
from tests.gpu_common import assert_equal, check_y, dev, f32_bits, host

pytestmark = pytest.mark.gpu

A4_QUANT = [(1, 16), (3, 4096), (2, 4112), (17, 3200), (1, 28672), (2, 65552)]


@pytest.mark.parametrize("M,K", A4_QUANT, ids=[f"M{m}xK{k}" for m, k in A4_QUANT])
def test_quant_a4_parity(gpu_lib, M, K):
    import torch
    X = make_acts(0, f"test/a4/X{M}x{K}", M, K, {"outlier_frac": 0.01, "outlier_scale": 30.0})
    Xq, s, xs = gpu_lib.bitlinear_quant_acts(dev(X), bits=4)
    torch.cuda.synchronize()
    oq, os_, oxs, _ = O.quantize_activations(X, bits=4)
    assert_equal(host(Xq), oq, "X~ (4-bit)")
    assert_equal(f32_bits(host(s)), f32_bits(os_), "x_scale bits")
    assert_equal(host(xs).astype(np.int64), oxs, "x_sum")
    assert np.abs(host(Xq)).max() <= 7


# one token (vector-ALU decode), a few (matrix decode), 8-32 (skinny), > 64 (GEMM)
A4_FWD = [(1, 300, 4096), (4, 129, 1040), (16, 1000, 2048), (32, 257, 4096), (130, 300, 1040)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", A4_FWD, ids=[f"M{m}N{n}K{k}" for m, n, k in A4_FWD])
def test_forward_a4(gpu_lib, M, N, K, out):
    import torch
    W = make_weight(0, f"test/a4/W{N}x{K}", N, K, 0.02)
    X = make_acts(0, f"test/a4/Xf{M}x{K}", M, K, {})
    r = O.bitlinear(W, X, bits=4)
    Wp, g = gpu_lib.bitlinear_pack_weights(dev(W))
    Xq, s, xs = gpu_lib.bitlinear_quant_acts(dev(X), bits=4)
    acc = gpu_lib.bitlinear_forward(Wp, g, Xq, s, xs, N=N, K=K, y_dtype="i32")
    Y = gpu_lib.bitlinear_forward(Wp, g, Xq, s, xs, N=N, K=K, y_dtype=out)
    torch.cuda.synchronize()
    assert_equal(host(Xq), r["Xq"], "X~ (4-bit)")
    assert_equal(host(acc).astype(np.int64), r["acc"], "accumulators")
    check_y(Y, r["y"], out)
    if M <= 16:
        P3, g3 = gpu_lib.bitlinear_pack_weights_base3(dev(W))
        Y3 = gpu_lib.bitlinear_forward_base3(P3, g3, Xq, s, xs, N=N, K=K, y_dtype=out)
        torch.cuda.synchronize()
        check_y(Y3, r["y"], out)
