"""GPU parity of the base-3 weight format (BLT3-v1) against the CPU oracle.

Bit-exact: gamma, the packed bytes, the bytes rewritten as BLT2-v1 and the
int32 accumulators.  Within tolerance: Y (1e-5 relative for fp32, 1e-2 for
bf16), with outputs of a zero accumulator exactly zero.
"""
import numpy as np
import pytest

from oracle import bitlinear_oracle as O
from synth import WORKLOADS, make_acts, make_weight
from tests.gpu_common import assert_equal, check_y, dev, f32_bits, host

pytestmark = pytest.mark.gpu

# Row lengths: one piece, a piece cut at 16 / 64 weights, several pieces with
# a ragged tail, exactly 64 pieces (one per lane), and rows needing 2, 3, 4
# pieces per lane and two blocks of 256 pieces.
PACK3_SHAPES = [(1, 16), (3, 80), (7, 96), (5, 144), (33, 1040), (64, 3200), (129, 4096),
                (3, 5120), (5, 8640), (2, 11008), (3, 28672)]


@pytest.mark.parametrize("N,K", PACK3_SHAPES, ids=[f"N{n}xK{k}" for n, k in PACK3_SHAPES])
def test_pack3_gaussian(gpu_lib, N, K):
    import torch
    W = make_weight(0, f"test/pack3/{N}x{K}", N, K, 0.02)
    gamma = O.absmean_gamma(W)
    Wt = O.ternarize(W, gamma)
    P3, g = gpu_lib.bitlinear_pack_weights_base3(dev(W))
    P2 = gpu_lib.bitlinear_base3_to_blt2(P3, K)
    torch.cuda.synchronize()
    assert_equal(f32_bits(host(g)), f32_bits([gamma]), "gamma bits")
    assert_equal(host(P3), O.pack_codes_base3(Wt), "BLT3 bytes")
    assert_equal(host(P2), O.pack_codes(Wt), "BLT3 -> BLT2 bytes")


def test_pack3_threshold_neighbours_and_zero_rows(gpu_lib):
    """Weights on and one ulp either side of the +-1/2 decisions, and all-zero
    rows (every digit 1, bytes 0x80)."""
    W = make_weight(0, "test/pack3/thresholds", 16, 240, 0.02)
    W[5] = 0.0
    gamma = O.absmean_gamma(W)
    g = np.float32(gamma + O.EPS)
    for i, side in enumerate((0.5, -0.5)):
        t = np.float32(np.float64(g) * side)
        W[i, :4] = [t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(-np.inf)), -t]
    gamma = O.absmean_gamma(W)
    Wt = O.ternarize(W, gamma)
    P3, gg = gpu_lib.bitlinear_pack_weights_base3(dev(W))
    import torch
    torch.cuda.synchronize()
    assert_equal(f32_bits(host(gg)), f32_bits([gamma]), "gamma bits")
    want = O.pack_codes_base3(Wt)
    assert (want[5] == 0x80).all()
    assert_equal(host(P3), want, "BLT3 bytes")


# (M, N, K): one token on the vector ALU (2 or 4 rows per wave); 2-16 tokens
# on the matrix cores with 1 block of 16 rows per wave, and above 8 tokens 2
# (8192+ rows) or 4 (16384+ rows); ragged N against every block; K with a cut
# last piece, fewer steps than waves, and rows that need several 256-piece
# blocks.
FWD3_SHAPES = [(1, 1, 16), (1, 17, 80), (1, 300, 1040), (1, 8640, 3200), (1, 3200, 8640),
               (1, 100, 20480), (1, 37, 28672), (1, 5, 40960), (2, 33, 96), (3, 129, 4096),
               (4, 1000, 8640), (5, 64, 1040), (8, 257, 4096), (13, 31, 28672), (16, 300, 3200),
               (16, 1, 16), (12, 8200, 1040), (9, 8192, 80), (16, 16400, 336), (10, 16385, 4096)]


@pytest.mark.parametrize("M,N,K", FWD3_SHAPES, ids=[f"M{m}N{n}K{k}" for m, n, k in FWD3_SHAPES])
def test_forward3_int32_handbuilt(gpu_lib, M, N, K):
    """Packed bytes built by the oracle and random int8 activations: the
    accumulators must be exact."""
    import torch
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    Wt = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    Xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    xsum = Xq.astype(np.int64).sum(1).astype(np.int32)
    acc = gpu_lib.bitlinear_forward_base3(dev(O.pack_codes_base3(Wt)),
                                          dev(np.array([1.0], np.float32)), dev(Xq),
                                          dev(np.ones(M, np.float32)), dev(xsum), N=N, K=K,
                                          y_dtype="i32")
    torch.cuda.synchronize()
    assert_equal(host(acc).astype(np.int64), O.integer_matmul(Wt, Xq), "int32 accumulators")


def test_forward3_extreme_accumulators(gpu_lib):
    """All weights +1 (or -1) and all activations +-127: |acc| = 127 K."""
    import torch
    M, N, K = 16, 48, 28672
    Wt = np.ones((N, K), np.int8)
    Wt[1::2] = -1
    Xq = np.full((M, K), 127, np.int8)
    Xq[1::2] = -127
    xsum = Xq.astype(np.int64).sum(1).astype(np.int32)
    acc = gpu_lib.bitlinear_forward_base3(dev(O.pack_codes_base3(Wt)),
                                          dev(np.array([1.0], np.float32)), dev(Xq),
                                          dev(np.ones(M, np.float32)), dev(xsum), N=N, K=K,
                                          y_dtype="i32")
    torch.cuda.synchronize()
    assert_equal(host(acc).astype(np.int64), O.integer_matmul(Wt, Xq), "accumulators")


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 100, 512), (4, 77, 1040), (16, 200, 2048)])
def test_forward3_whole_path(gpu_lib, M, N, K, out):
    """fp32 W and X through the GPU packer, quantiser and base-3 projection
    against the oracle's whole projection."""
    import torch
    W = make_weight(0, f"test/fwd3/{N}x{K}", N, K, 0.02)
    X = make_acts(0, f"test/fwd3/X{M}x{K}", M, K, {})
    r = O.bitlinear(W, X)
    P3, g = gpu_lib.bitlinear_pack_weights_base3(dev(W))
    Xq, s, xs = gpu_lib.bitlinear_quant_acts(dev(X))
    acc = gpu_lib.bitlinear_forward_base3(P3, g, Xq, s, xs, N=N, K=K, y_dtype="i32")
    Y = gpu_lib.bitlinear_forward_base3(P3, g, Xq, s, xs, N=N, K=K, y_dtype=out)
    torch.cuda.synchronize()
    assert_equal(host(acc).astype(np.int64), r["acc"], "accumulators")
    check_y(Y, r["y"], out)


def test_forward3_unaligned_output(gpu_lib):
    """Y one element past an aligned address: the same bytes as an aligned Y."""
    import torch
    M, N, K = 3, 250, 4096
    W = make_weight(0, "test/fwd3u", N, K, 0.02)
    X = make_acts(0, "test/fwd3u/X", M, K, {})
    P3, g = gpu_lib.bitlinear_pack_weights_base3(dev(W))
    Xq, s, xs = gpu_lib.bitlinear_quant_acts(dev(X))
    buf = torch.zeros(M * N + 1, dtype=torch.bfloat16, device="cuda")
    Yu = buf[1:].view(M, N)
    gpu_lib.bitlinear_forward_base3(P3, g, Xq, s, xs, N=N, K=K, y_dtype="bf16", Y=Yu)
    Ya = gpu_lib.bitlinear_forward_base3(P3, g, Xq, s, xs, N=N, K=K, y_dtype="bf16")
    torch.cuda.synchronize()
    assert torch.equal(Yu, Ya)
    assert buf[0].item() == 0


B3_FULL = [("decode-3b", 1), ("decode-7b", 8), ("ffn-70b", 1), ("ffn-70b", 16)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wname,M", B3_FULL, ids=[f"{w}:M{m}" for w, m in B3_FULL])
def test_workload_full_size_base3(gpu_lib, wname, M):
    """Every projection of a decode workload at its real sizes, in the launch
    configuration the bench times: gamma, sampled rows of the packed bytes and
    of the BLT2 rewrite, and the accumulators and outputs of sampled rows,
    against the oracle."""
    import torch
    wl = WORKLOADS[wname]
    for p in wl.projections:
        W = wl.weight(p)
        gamma = O.absmean_gamma(W)
        rows = np.unique(np.concatenate([np.arange(4), p.N - 1 - np.arange(4),
                                         np.random.default_rng(p.N).integers(0, p.N, 24)]))
        Wt = O.ternarize(W[rows], gamma)
        X = wl.acts(p, M)
        oq, os_, oxs, beta = O.quantize_activations(X)
        P3, g = gpu_lib.bitlinear_pack_weights_base3(dev(W))
        del W
        P2 = gpu_lib.bitlinear_base3_to_blt2(P3, p.K)
        Xq, s, xs = gpu_lib.bitlinear_quant_acts(dev(X))
        acc = gpu_lib.bitlinear_forward_base3(P3, g, Xq, s, xs, N=p.N, K=p.K, y_dtype="i32")
        Y = gpu_lib.bitlinear_forward_base3(P3, g, Xq, s, xs, N=p.N, K=p.K, y_dtype=wl.out_dtype)
        torch.cuda.synchronize()
        assert_equal(f32_bits(host(g)), f32_bits([gamma]), f"gamma bits {p.name}")
        idx = torch.as_tensor(rows, device=P3.device)
        assert_equal(host(P3[idx]), O.pack_codes_base3(Wt), f"BLT3 rows {p.name}")
        assert_equal(host(P2[idx]), O.pack_codes(Wt), f"BLT2 rows {p.name}")
        acc_ref = O.integer_matmul(Wt, oq)
        assert_equal(host(acc)[:, rows].astype(np.int64), acc_ref, f"accumulators {p.name}")
        check_y(Y[:, idx], O.rescale(acc_ref, gamma, beta), wl.out_dtype)
        del P3, P2
        torch.cuda.empty_cache()
