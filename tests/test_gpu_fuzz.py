"""Seeded shape fuzz of the whole GPU path against the oracle, through the C
ABI.  For each seed three shapes are drawn: M in 1..70 for the first two
(1 for the first draw of an even seed) and 256 or 300 for the third; N
anywhere in 1..3000 (ragged against every tile and row group); K a multiple
of 16 up to 8192 (ragged against the 64-, 128- and 4096-wide steps).
Weights and activations come from the seeded generators.  Packing (gamma
bits, bytes), the quantiser (X~, scale bits, sums), the projection from
quantised activations and from fp32 ones, and the grouped and
multi-projection calls must equal the oracle exactly (accumulators), Y
within the output type's tolerance.  The run stops at the first mismatch
(pytest -x)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import bitlinear_oracle as O
from synth import make_acts, make_weight
from tests.gpu_common import assert_equal, check_y, dev, f32_bits, host

pytestmark = pytest.mark.gpu

DRAWS_PER_SEED = 3


def _draw(rng, seed, d):
    # the last draw of each seed takes a prefill-sized M (the GEMM path), the
    # first draw of an even seed one token (the single-token kernels)
    if d == DRAWS_PER_SEED - 1:
        M = int(rng.choice([256, 300]))
    elif d == 0 and seed % 2 == 0:
        M = 1
    else:
        M = int(rng.integers(1, 71))
    N = int(rng.integers(1, 3001))
    K = 16 * int(rng.integers(1, 513))
    return M, N, K


@pytest.mark.parametrize("seed", range(10))
def test_fuzz_shapes_against_oracle(gpu_lib, seed):
    import torch
    tb = gpu_lib
    rng = np.random.default_rng(1000 + seed)
    for d in range(DRAWS_PER_SEED):
        M, N, K = _draw(rng, seed, d)
        tag = f"fuzz/s{seed}d{d}"
        print(f"fuzz seed {seed} draw {d}: M={M} N={N} K={K}", flush=True)
        W = make_weight(seed, f"{tag}/W", N, K, 0.02)
        X = make_acts(seed, f"{tag}/X", M, K,
                      {"outlier_frac": Fraction(1, 100), "outlier_scale": 50.0})
        r = O.bitlinear(W, X)
        Wp, g = tb.bitlinear_pack_weights(dev(W))
        Xq, s, xs = tb.bitlinear_quant_acts(dev(X))
        torch.cuda.synchronize()
        assert_equal(f32_bits(host(g)), f32_bits(np.array([r["gamma"]])), "gamma")
        assert_equal(host(Wp), r["packed"], "packed bytes")
        assert_equal(host(Xq), r["Xq"], "X~")
        assert_equal(f32_bits(host(s)), f32_bits(r["x_scale"]), "x_scale")
        assert_equal(host(xs).astype(np.int64), r["x_sum"], "x_sum")
        acc = tb.bitlinear_forward(Wp, g, Xq, s, xs, N=N, K=K, y_dtype="i32")
        acc32 = tb.bitlinear_forward_f32(Wp, g, dev(X), N=N, y_dtype="i32")
        y = tb.bitlinear_forward(Wp, g, Xq, s, xs, N=N, K=K, y_dtype="bf16")
        yf = tb.bitlinear_forward_f32(Wp, g, dev(X), N=N, y_dtype="f32")
        torch.cuda.synchronize()
        assert_equal(host(acc).astype(np.int64), r["acc"], "accumulators")
        assert_equal(host(acc32).astype(np.int64), r["acc"], "fp32-in accumulators")
        check_y(y, r["y"], "bf16")
        check_y(yf, r["y"], "f32")
        # the same weights twice as one group (shared X~), and with a second
        # projection of its own input as one multi-projection call
        ga = tb.bitlinear_forward_grouped([Wp, Wp], [g, g], Xq, s, xs, K=K, y_dtype="i32")
        K2 = 16 * int(rng.integers(1, 257))
        W2 = make_weight(seed, f"{tag}/W2", N, K2, 0.02)
        X2 = make_acts(seed, f"{tag}/X2", M, K2, {})
        r2 = O.bitlinear(W2, X2)
        Wp2, g2 = tb.bitlinear_pack_weights(dev(W2))
        mu = tb.bitlinear_forward_f32_multi([Wp, Wp2], [g, g2], [dev(X), dev(X2)], y_dtype="i32")
        torch.cuda.synchronize()
        for i, a in enumerate(ga):
            assert_equal(host(a).astype(np.int64), r["acc"], f"grouped projection {i}")
        assert_equal(host(mu[0]).astype(np.int64), r["acc"], "multi projection 0")
        assert_equal(host(mu[1]).astype(np.int64), r2["acc"], "multi projection 1")
