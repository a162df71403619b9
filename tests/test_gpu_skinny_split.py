"""GPU parity of the K-split skinny projection (one projection, 17-64 tokens,
K >= 2 N, M K > 256 Ki): each split writes exact int32 partial sums and a
second launch adds them and applies the rescale.  Accumulators exact against
the oracle in full, Y within tolerance, and an
unaligned Y (scalar stores in the reduction) byte-identical to an aligned one.
"""
import numpy as np
import pytest

from oracle import bitlinear_oracle as O
from synth import make_acts, make_weight
from tests.gpu_common import assert_equal, check_y, dev, host

pytestmark = pytest.mark.gpu

# (M, N, K): two and four token groups; 4 and 8 row blocks per workgroup;
# ragged N (1000, 999, 8200: the last row group part-empty; 999 also rules
# out vector stores); K ending inside a 512-wide chunk (11008) or 64 into one
# (16448); 2 to 4 splits (3 where 4 would leave a split without a chunk).
SPLIT_SHAPES = [(17, 8200, 16448), (32, 8200, 16448), (33, 999, 8192), (48, 2000, 8192),
                (40, 300, 65536), (64, 8200, 16448), (64, 2000, 4160)]
# 17-32 tokens on up to 512 row blocks with a long K: no split, the token
# halves of the skinny kernel instead (ragged N, K past a 512-wide chunk)
HALVES_SHAPES = [(17, 1000, 16384), (32, 4096, 11008), (24, 64, 65536), (29, 999, 8256)]


def _is_split(M, N, K):
    import ternary_bitlinear_amd as tb
    return (tb.forward_kernel("forward", M, [N], K) == ("k_skinny", False)
            and tb.forward_workspace_bytes(M, N, K) > 0)


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES, ids=[f"M{m}N{n}K{k}" for m, n, k in SPLIT_SHAPES])
def test_split_int32_handbuilt(gpu_lib, M, N, K):
    """Codes packed by the oracle and random int8 activations (x_sum their
    exact row sums): the int32 accumulators must be exact."""
    import torch
    assert _is_split(M, N, K)
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    Wt = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    Xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    xsum = Xq.astype(np.int64).sum(1).astype(np.int32)
    acc = gpu_lib.bitlinear_forward(dev(O.pack_codes(Wt)), dev(np.array([1.0], np.float32)),
                                    dev(Xq), dev(np.ones(M, np.float32)), dev(xsum), N=N, K=K,
                                    y_dtype="i32")
    torch.cuda.synchronize()
    assert_equal(host(acc).astype(np.int64), O.integer_matmul(Wt, Xq), "int32 accumulators")


def test_split_extreme_accumulators(gpu_lib):
    """All weights +-1 and activations +-127 over K = 65536: |acc| = 127 K,
    each split's partial and the total within int32."""
    import torch
    M, N, K = 40, 64, 65536
    assert _is_split(M, N, K)
    Wt = np.ones((N, K), np.int8)
    Wt[1::2] = -1
    Xq = np.full((M, K), 127, np.int8)
    Xq[1::2] = -127
    xsum = Xq.astype(np.int64).sum(1).astype(np.int32)
    acc = gpu_lib.bitlinear_forward(dev(O.pack_codes(Wt)), dev(np.array([1.0], np.float32)),
                                    dev(Xq), dev(np.ones(M, np.float32)), dev(xsum), N=N, K=K,
                                    y_dtype="i32")
    torch.cuda.synchronize()
    assert_equal(host(acc).astype(np.int64), O.integer_matmul(Wt, Xq), "accumulators")


WHOLE = [(48, 1000, 16384), (33, 999, 8192), (40, 300, 65536)]


@pytest.mark.parametrize("out", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("M,N,K", WHOLE, ids=[f"M{m}N{n}K{k}" for m, n, k in WHOLE])
def test_split_whole_path(gpu_lib, M, N, K, out):
    """fp32 W and X through the GPU packer and quantiser, then the split
    projection, against the oracle's whole projection; the fp32 entry point
    (quantiser, then the same projection) gives the same bytes; a Y one
    element past an aligned address gives the same bytes as an aligned one."""
    import torch
    assert _is_split(M, N, K)
    W = make_weight(0, f"test/split/{N}x{K}", N, K, 0.02)
    X = make_acts(0, f"test/split/X{M}x{K}", M, K, {"outlier_frac": 0.005, "outlier_scale": 100.0})
    r = O.bitlinear(W, X)
    Wp, g = gpu_lib.bitlinear_pack_weights(dev(W))
    Xd = dev(X)
    Xq, s, xs = gpu_lib.bitlinear_quant_acts(Xd)
    Y = gpu_lib.bitlinear_forward(Wp, g, Xq, s, xs, N=N, K=K, y_dtype=out)
    Yf = gpu_lib.bitlinear_forward_f32(Wp, g, Xd, N=N, y_dtype=out)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[out]
    buf = torch.zeros(M * N + 1, dtype=tdt, device="cuda")
    Yu = buf[1:].view(M, N)
    gpu_lib.bitlinear_forward(Wp, g, Xq, s, xs, N=N, K=K, y_dtype=out, Y=Yu)
    torch.cuda.synchronize()
    if out == "i32":
        assert_equal(host(Y).astype(np.int64), r["acc"], "int32 accumulators")
    else:
        check_y(Y, r["y"], out)
    assert torch.equal(Y, Yf)
    assert torch.equal(Yu, Y)
    assert buf[0].item() == 0


def test_split_workspace_reuse_and_side_stream(gpu_lib):
    """Two calls sharing one workspace in stream order on a side stream, the
    second with fewer tokens: each result exact (the workspace needs no
    clearing and the second call's splits overwrite what they read)."""
    import torch
    N, K = 2000, 8192
    rng = np.random.default_rng(5)
    Wt = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    Xq = rng.integers(-127, 128, size=(48, K), dtype=np.int8)
    P = dev(O.pack_codes(Wt))
    one = dev(np.array([1.0], np.float32))
    s = torch.cuda.Stream()
    import ternary_bitlinear_amd as tb
    ws = torch.full((tb.forward_workspace_bytes(48, N, K),), 0x7f, dtype=torch.uint8, device="cuda")
    outs = []
    with torch.cuda.stream(s):
        for m in (48, 33):
            assert _is_split(m, N, K)
            xsum = Xq[:m].astype(np.int64).sum(1).astype(np.int32)
            outs.append(gpu_lib.bitlinear_forward(P, one, dev(Xq[:m]), dev(np.ones(m, np.float32)),
                                                  dev(xsum), N=N, K=K, y_dtype="i32",
                                                  workspace=ws, stream=s))
    s.synchronize()
    for m, acc in zip((48, 33), outs):
        assert_equal(host(acc).astype(np.int64), O.integer_matmul(Wt, Xq[:m]), f"M={m}")


@pytest.mark.parametrize("M,N,K", HALVES_SHAPES, ids=[f"M{m}N{n}K{k}" for m, n, k in HALVES_SHAPES])
def test_halves_instead_of_split_int32(gpu_lib, M, N, K):
    """Long-K shapes that the split used to take at 17-32 tokens: the token
    halves, no workspace, and exact int32 accumulators."""
    import torch
    import ternary_bitlinear_amd as tb
    assert tb.forward_kernel("forward", M, [N], K) == ("k_skinny", False)
    assert tb.forward_workspace_bytes(M, N, K) == 0
    rng = np.random.default_rng(M * 7919 + N * 31 + K + 1)
    Wt = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    Xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    xsum = Xq.astype(np.int64).sum(1).astype(np.int32)
    acc = gpu_lib.bitlinear_forward(dev(O.pack_codes(Wt)), dev(np.array([1.0], np.float32)),
                                    dev(Xq), dev(np.ones(M, np.float32)), dev(xsum), N=N, K=K,
                                    y_dtype="i32")
    torch.cuda.synchronize()
    assert_equal(host(acc).astype(np.int64), O.integer_matmul(Wt, Xq), "int32 accumulators")
