"""bitlinear_forward_f32_multi: several projections, each with its own
activations and K, against one bitlinear_forward_f32 per projection (same
bytes) and against the oracle (exact accumulators; Y within the output
type's tolerance), through the C ABI.  Single-token calls run as one
persistent launch over all projections; other shapes fall back to one call
per projection."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import bitlinear_oracle as O
from synth import WORKLOADS, make_acts, make_weight
from tests.gpu_common import assert_equal, check_y, dev, host

pytestmark = pytest.mark.gpu


def _projection(N, K, tag):
    W = make_weight(0, f"test/multi/W{tag}_{N}x{K}", N, K, 0.02)
    gamma = O.absmean_gamma(W)
    Wt = O.ternarize(W, gamma)
    return Wt, gamma


def _run(tb, shapes, M, out, tag, acts=None):
    """shapes: [(N, K)]; returns (multi outputs, single-call outputs, oracle
    accumulators, oracle y)."""
    import torch
    Ps, gs, Xs, accs, ys = [], [], [], [], []
    for i, (N, K) in enumerate(shapes):
        Wt, gamma = _projection(N, K, f"{tag}{i}")
        X = (acts[i] if acts is not None else
             make_acts(0, f"test/multi/X{tag}{i}_{M}x{K}", M, K,
                       {"outlier_frac": Fraction(1, 100), "outlier_scale": 50.0}))
        Xq, _, _, beta = O.quantize_activations(X)
        acc = O.integer_matmul(Wt, Xq)
        Ps.append(dev(O.pack_codes(Wt)))
        gs.append(dev(np.array([gamma], np.float32)))
        Xs.append(dev(X))
        accs.append(acc)
        ys.append(O.rescale(acc, gamma, beta))
    Y = tb.bitlinear_forward_f32_multi(Ps, gs, Xs, Ns=[n for n, _ in shapes], y_dtype=out)
    single = [tb.bitlinear_forward_f32(P, g, X, N=n, y_dtype=out)
              for P, g, X, (n, _) in zip(Ps, gs, Xs, shapes)]
    torch.cuda.synchronize()
    return Y, single, accs, ys


def _bytes(t):
    import torch
    return host(t.view(torch.int16)) if t.dtype == torch.bfloat16 else host(t)


CASES = [
    # (M, [(N, K)]): one launch (M = 1, K % 64 == 0) over 2-4 projections of
    # different K, ragged N (not a multiple of the 4-row groups), a one-row
    # projection, K from 64 to 32768 (the quantiser holds 4, 8 or 16 groups
    # of four per thread); then shapes that fall back to one call each
    (1, [(3000, 512), (77, 2048)]),
    (1, [(1, 64), (130, 4096), (9, 32768)]),
    (1, [(640, 3200), (3200, 640), (5, 128), (1000, 16384)]),
    (1, [(4096, 4096)]),
    (1, [(200, 1040), (300, 512)]),        # K % 64 != 0: one call per projection
    # more tokens: one quantiser launch for every input, then one launch per
    # projection (skinny, decode, GEMM and a K-split projection whose
    # workspace follows the inputs' quantiser regions); two tokens, where a
    # projection may fuse, one call per projection
    (3, [(300, 512), (77, 1024)]),
    (5, [(200, 1040), (300, 528)]),
    (16, [(3000, 1024), (1000, 3008)]),
    (32, [(1024, 11008), (300, 512), (64, 4096)]),
    (40, [(700, 2048), (130, 1040), (2, 64), (513, 320)]),
    (2, [(300, 512), (77, 1040)]),
]


@pytest.mark.parametrize("M,shapes", CASES, ids=[f"M{m}_" + "_".join(f"{n}x{k}" for n, k in s)
                                                 for m, s in CASES])
def test_multi_matches_single_calls_and_oracle(gpu_lib, M, shapes):
    tb = gpu_lib
    Ns, Ks = [n for n, _ in shapes], [k for _, k in shapes]
    one = tb.forward_f32_multi_kernel(M, Ns, Ks) == ("k_stream", True)
    assert one == (M == 1 and all(k % 64 == 0 for k in Ks))
    assert tb.forward_f32_multi_kernel(M, Ns, Ks) in (("k_stream", True), None)
    print(f"multi M{M} {shapes} one launch: {one}", flush=True)
    for out in ("i32", "f32", "bf16"):
        Y, single, accs, ys = _run(tb, shapes, M, out, f"c{len(shapes)}{M}{Ks[0]}")
        for g in range(len(shapes)):
            assert_equal(_bytes(Y[g]), _bytes(single[g]), f"projection {g} ({out}) vs single call")
            if out == "i32":
                assert_equal(host(Y[g]).astype(np.int64), accs[g], f"projection {g} accumulators")
            else:
                check_y(Y[g], ys[g], out)


def test_multi_extreme_and_zero_rows(gpu_lib):
    # +-127 accumulators over K = 32768 (all weights +1 or -1, every
    # activation at the absmax), and a zero activation row (beta = 0 -> 0)
    import torch
    tb = gpu_lib
    K1, K2 = 32768, 4096
    W1 = np.where(np.arange(64 * K1).reshape(64, K1) % 2 == 0, 1.0, -1.0).astype(np.float32)
    W1[::2] = 1.0
    Wt1 = O.ternarize(W1, O.absmean_gamma(W1))
    X1 = np.ones((1, K1), np.float32)
    X2 = np.zeros((1, K2), np.float32)
    Wt2, g2 = _projection(96, K2, "zero")
    Ps = [dev(O.pack_codes(Wt1)), dev(O.pack_codes(Wt2))]
    gs = [dev(np.array([O.absmean_gamma(W1)], np.float32)), dev(np.array([g2], np.float32))]
    Y = tb.bitlinear_forward_f32_multi(Ps, gs, [dev(X1), dev(X2)], y_dtype="i32")
    torch.cuda.synchronize()
    want = O.integer_matmul(Wt1, O.quantize_activations(X1)[0])
    assert np.abs(want).max() == 127 * K1
    assert_equal(host(Y[0]).astype(np.int64), want, "extreme accumulators")
    assert not host(Y[1]).any()


@pytest.mark.parametrize("name", ["decode-3b", "ffn-70b"])
def test_multi_full_size_workloads(gpu_lib, name):
    # every projection of the workload, one token, in one launch, as the
    # bench's step runs it: exact accumulators against the oracle
    import torch
    tb = gpu_lib
    wl = WORKLOADS[name]
    Ps, gs, Xs, want = [], [], [], []
    for p in wl.projections:
        W = wl.weight(p)
        X = wl.acts(p, 1)
        gamma = O.absmean_gamma(W)
        Wt = O.ternarize(W, gamma)
        Xq = O.quantize_activations(X)[0]
        want.append(O.integer_matmul(Wt, Xq))
        Wp, gd = tb.bitlinear_pack_weights(dev(W))
        Ps.append(Wp)
        gs.append(gd)
        Xs.append(dev(X))
        del W, Wt
    Ns = [p.N for p in wl.projections]
    Ks = [p.K for p in wl.projections]
    assert tb.forward_f32_multi_kernel(1, Ns, Ks) == ("k_stream", True)
    Y = tb.bitlinear_forward_f32_multi(Ps, gs, Xs, y_dtype="i32")
    torch.cuda.synchronize()
    for g, w in enumerate(want):
        assert_equal(host(Y[g]).astype(np.int64), w, f"{name} projection {g}")


def test_multi_graph_replays_match_eager(gpu_lib):
    # captured once, replayed three times with eager work on the stream in
    # between: every replay gives the eager call's bytes
    import torch
    tb = gpu_lib
    shapes = [(2048, 1024), (1024, 3072)]
    Ps, gs, Xs = [], [], []
    for i, (N, K) in enumerate(shapes):
        Wt, gamma = _projection(N, K, f"graph{i}")
        Ps.append(dev(O.pack_codes(Wt)))
        gs.append(dev(np.array([gamma], np.float32)))
        Xs.append(dev(make_acts(0, f"test/multi/Xgraph{i}", 1, K, {})))
    eager = [y.clone() for y in tb.bitlinear_forward_f32_multi(Ps, gs, Xs, y_dtype="bf16")]
    s = torch.cuda.Stream()
    Y = [torch.empty_like(y) for y in eager]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tb.bitlinear_forward_f32_multi(Ps, gs, Xs, y_dtype="bf16", Y=Y, stream=s)
    for rep in range(3):
        for y in Y:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(Y, eager):
            assert_equal(_bytes(a), _bytes(b), f"replay {rep}")
        tb.bitlinear_forward_f32_multi(Ps, gs, Xs, y_dtype="bf16")   # eager work between
        torch.cuda.synchronize()
