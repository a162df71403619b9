"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Bit-exact: gamma, packed bytes, X~, x_scale, x_sum and the int32 accumulators.
Within tolerance: Y (1e-5 relative for fp32 out, 1e-2 for bf16), with outputs
of a zero accumulator exactly zero.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import bitlinear_oracle as O
from synth import WORKLOADS, make_acts, make_weight
from tests.gpu_common import assert_equal, check_y, dev, f32_bits, host

pytestmark = pytest.mark.gpu


def run_pack(tb, W):
    Wp, g = tb.bitlinear_pack_weights(dev(W))
    return host(Wp), host(g)


def run_quant(tb, X):
    Xq, s, xs = tb.bitlinear_quant_acts(dev(X))
    return host(Xq), host(s), host(xs)


# --------------------------------------------------------------------------- pack
PACK_SHAPES = [(1, 16), (7, 48), (33, 80), (256, 512), (300, 1040), (129, 4096), (3, 8640)]


@pytest.mark.parametrize("N,K", PACK_SHAPES, ids=[f"N{n}xK{k}" for n, k in PACK_SHAPES])
def test_pack_gaussian(gpu_lib, N, K):
    W = make_weight(0, f"test/pack/{N}x{K}", N, K, 0.02)
    Wp, g = run_pack(gpu_lib, W)
    gamma = O.absmean_gamma(W)
    assert_equal(f32_bits(g), f32_bits([gamma]), "gamma bits")
    assert_equal(Wp, O.pack_codes(O.ternarize(W, gamma)), "packed bytes")


def _special_weights():
    rng = np.random.default_rng(20)
    out = {}
    out["zeros"] = np.zeros((5, 32), np.float32)
    out["const"] = (np.where(rng.random((9, 64)) < 0.5, -1, 1) * np.float32(0.0123)).astype(np.float32)
    # exponents over the whole fp32 range in one tile (exercises the exact slow path)
    mant = rng.random((16, 256)) + 0.5
    expo = rng.integers(-149, 100, size=(16, 256))
    w = (np.ldexp(mant, expo) * np.where(rng.random((16, 256)) < 0.5, -1, 1)).astype(np.float32)
    w[rng.random((16, 256)) < 0.1] = 0.0
    out["wide-exponents"] = w
    out["subnormal-only"] = (np.ldexp(rng.random((4, 64)), -140)).astype(np.float32)
    from scipy.linalg import hadamard
    out["hadamard"] = hadamard(128).astype(np.float32)
    big = make_weight(0, "test/pack/outlier", 64, 512, 0.02)
    big[3, 7] = 3.0e3     # one huge weight: most others fall below the tile window
    out["one-huge"] = big
    return out


SPECIAL = _special_weights()


@pytest.mark.parametrize("name", list(SPECIAL))
def test_pack_special(gpu_lib, name):
    W = SPECIAL[name]
    Wp, g = run_pack(gpu_lib, W)
    gamma = O.absmean_gamma(W)
    assert_equal(f32_bits(g), f32_bits([gamma]), "gamma bits")
    assert_equal(Wp, O.pack_codes(O.ternarize(W, gamma)), "packed bytes")


def test_pack_threshold_neighbours(gpu_lib):
    """Weights placed on and one ulp either side of the +-1/2 decision
    boundaries of z = W / (gamma + eps), for the gamma the matrix itself has."""
    W = make_weight(0, "test/pack/thresholds", 16, 256, 0.02)
    probes = [(r, c) for r in range(2) for c in range(8)]
    for _ in range(20):
        gamma = O.absmean_gamma(W)
        g = np.float32(gamma + O.EPS)
        vals = []
        for side in (0.5, -0.5):
            t = np.float32(np.float64(g) * side)
            vals += [t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(-np.inf)),
                     np.nextafter(np.nextafter(t, np.float32(np.inf)), np.float32(np.inf))]
        for (r, c), v in zip(probes, vals + vals):
            W[r, c] = v
        if O.absmean_gamma(W) == gamma:
            break
    gamma = O.absmean_gamma(W)
    Wt = O.ternarize(W, gamma)
    codes = {int(Wt[r, c]) for (r, c) in probes}
    assert codes == {-1, 0, 1}, "probes must straddle the boundaries"
    Wp, g = run_pack(gpu_lib, W)
    assert_equal(f32_bits(g), f32_bits([gamma]), "gamma bits")
    assert_equal(Wp, O.pack_codes(Wt), "packed bytes")


# --------------------------------------------------------------------------- quant
QUANT_SHAPES = [(1, 16), (3, 48), (5, 512), (64, 4096), (2, 8640), (17, 3200), (300, 128),
                (2, 33280), (1, 131072), (3, 28672),
                # 1024-thread workgroups past 4096 values: 2, 4, 8, 16 groups of
                # four per thread, ragged rows, and the looped variant past 65536
                (1, 4112), (2, 8192), (3, 12304), (4, 16400), (1, 65536), (2, 65552)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES, ids=[f"M{m}xK{k}" for m, k in QUANT_SHAPES])
def test_quant_parity(gpu_lib, M, K):
    from fractions import Fraction
    X = make_acts(0, f"test/quant/{M}x{K}", M, K,
                  {"outlier_frac": Fraction(1, 200), "outlier_scale": 100.0})
    Xq, s, xs = run_quant(gpu_lib, X)
    oq, os_, oxs, _ = O.quantize_activations(X)
    assert_equal(Xq, oq, "X~")
    assert_equal(f32_bits(s), f32_bits(os_), "x_scale bits")
    assert_equal(xs.astype(np.int64), oxs, "x_sum")


def test_quant_edge_rows(gpu_lib):
    K = 32
    rows = []
    rows.append(np.zeros(K, np.float32))                                   # zero token
    b = np.float32(127.0) - np.float32(2.0 ** -17)                          # factor exactly 1
    r = np.zeros(K, np.float32)
    r[:16] = [b, 0.5, -0.5, 2.5, -2.5, np.nextafter(np.float32(0.5), np.float32(0)),
              np.nextafter(np.float32(-0.5), np.float32(-1)), 100.5, -b, 0.0, 63.25, -63.75,
              1.0, -1.0, 126.5, -126.5]
    rows.append(r)
    rows.append(np.full(K, np.float32(1e-40)))                              # subnormal inputs
    rows.append(np.linspace(-3e30, 2e30, K).astype(np.float32))            # huge inputs
    rows.append(-np.abs(np.random.default_rng(3).standard_normal(K)).astype(np.float32))
    rows.append(np.full(K, np.float32(2.5e-3)))                             # absmax near 253 eps
    X = np.stack(rows).astype(np.float32)
    Xq, s, xs = run_quant(gpu_lib, X)
    oq, os_, oxs, _ = O.quantize_activations(X)
    assert_equal(Xq, oq, "X~")
    assert_equal(f32_bits(s), f32_bits(os_), "x_scale bits")
    assert_equal(xs.astype(np.int64), oxs, "x_sum")


# --------------------------------------------------------------------------- forward
FWD_SHAPES = [
    # matrix decode (M <= 16; one token with K > 4096, or K % 64 != 0); the
    # skinny kernel for the rest of M >= 2
    (1, 1, 16), (1, 16, 64), (1, 17, 80), (2, 33, 1040), (5, 129, 512), (16, 300, 4096),
    (7, 64, 8640), (1, 3200, 8640),
    # decode with 2 and 4 row blocks per workgroup (needs >= 256 workgroups), ragged N
    (7, 8200, 80), (13, 16400, 1040), (16, 16384, 272),
    # single token on the vector ALU (K % 64 == 0, K <= 4096): one piece per
    # row, N below and not a multiple of the rows per wave, full rows
    (1, 1, 64), (1, 3, 4096), (1, 1001, 192), (1, 8640, 3200), (1, 11008, 4096),
    # GEMM path (M > 16): ragged tiles and K tails
    (17, 16, 64), (33, 130, 144), (64, 256, 4096), (130, 300, 1040), (300, 129, 128),
    (257, 513, 2048),
    # K split across workgroups (partial sums + reduction): with a K tail, with
    # N % 4 != 0 (scalar partial stores), two row tiles
    (24, 200, 4160), (40, 130, 2064), (100, 64, 8192),
    # skinny kernel (K % 64 == 0; 8-32 tokens, 2-7 on wide outputs, 33-64
    # up to K = 8192): fewer chunks than ring stages, K ending inside a
    # chunk, ragged N in the last workgroup's row blocks, 1 row block of 4
    # waves / 2 of 4 / 4 of 2 per workgroup, 16 / 32 / 64 token groups with
    # ragged M; at 33-64 tokens 1, 2, 3, 4 row blocks of 2 waves and 8 of 1
    # wave (a last workgroup of one row block, K ending inside a chunk,
    # fewer chunks than stages); past K = 8192 the GEMM, K split
    (2, 16384, 8192), (3, 6144, 64), (5, 10000, 128), (8, 100, 64), (9, 1, 128),
    (8, 4099, 4096), (12, 4096, 11008), (16, 16400, 704), (16, 28672, 1024),
    (17, 257, 576), (24, 4096, 11008), (31, 3000, 8192), (32, 6200, 3072),
    (33, 1030, 2048), (48, 11990, 5440), (63, 4100, 4096), (64, 64, 4096), (64, 20, 64),
    (45, 6000, 192), (40, 16000, 1024), (64, 16400, 1088), (37, 20000, 320),
    (40, 5000, 8320),
    # 128 x 256 GEMM tiles (1024+ tokens, 2 x 2 waves): ragged M and N, K
    # tails 16 and 64 wide, and K split two ways (16 tiles) with the tail in
    # the last split
    (1030, 300, 1040), (1024, 520, 4160), (1024, 264, 16448), (1024, 40, 32784),
    # many tiles (several rounds of the chip) with a 16-wide K tail: aligned,
    # then ragged M and N
    (2048, 12288, 272), (1030, 24600, 1040),
]


def _random_operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    Wt = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    Xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    return Wt, Xq


@pytest.mark.parametrize("M,N,K", FWD_SHAPES, ids=[f"M{m}N{n}K{k}" for m, n, k in FWD_SHAPES])
def test_forward_int32_handbuilt(gpu_lib, M, N, K):
    """Packed tensors built by the oracle (bypassing pack_weights) and random int8
    activations: the accumulators must be exact."""
    Wt, Xq = _random_operands(M, N, K, seed=M * 7919 + N * 31 + K)
    P = O.pack_codes(Wt)
    xsum = Xq.astype(np.int64).sum(1).astype(np.int32)
    import torch
    acc = gpu_lib.bitlinear_forward(dev(P), dev(np.array([1.0], np.float32)), dev(Xq),
                                    dev(np.ones(M, np.float32)), dev(xsum), N=N, K=K,
                                    y_dtype="i32")
    torch.cuda.synchronize()
    assert_equal(host(acc).astype(np.int64), O.integer_matmul(Wt, Xq), "int32 accumulators")


def test_forward_extreme_accumulators(gpu_lib):
    """All weights +1 (or -1) and all activations +-127: |acc| = 127 K."""
    M, N, K = 20, 48, 4096
    Wt = np.ones((N, K), np.int8)
    Wt[1::2] = -1
    Xq = np.full((M, K), 127, np.int8)
    Xq[1::2] = -127
    xsum = Xq.astype(np.int64).sum(1).astype(np.int32)
    for m in (M, 3):
        acc = gpu_lib.bitlinear_forward(dev(O.pack_codes(Wt)), dev(np.array([1.0], np.float32)),
                                        dev(Xq[:m]), dev(np.ones(m, np.float32)), dev(xsum[:m]),
                                        N=N, K=K, y_dtype="i32")
        assert_equal(host(acc).astype(np.int64), O.integer_matmul(Wt, Xq[:m]), "accumulators")


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 100, 512), (9, 77, 1040), (48, 200, 2048),
                                   (12, 1000, 3072), (40, 513, 6144)])
def test_forward_rescale(gpu_lib, M, N, K, out):
    W = make_weight(0, f"test/fwd/{N}x{K}", N, K, 0.02)
    X = make_acts(0, f"test/fwd/X{M}x{K}", M, K, {})
    r = O.bitlinear(W, X)
    Y = gpu_lib.bitlinear_forward(dev(r["packed"]), dev(np.array([r["gamma"]], np.float32)),
                                  dev(r["Xq"]), dev(r["x_scale"]),
                                  dev(r["x_sum"].astype(np.int32)), N=N, K=K, y_dtype=out)
    check_y(Y, r["y"], out)


@pytest.mark.parametrize("out", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("M,N,K", [(4, 256, 1024), (96, 256, 1024), (300, 260, 512),
                                   (300, 264, 512), (130, 136, 1040)])
def test_forward_unaligned_output(gpu_lib, M, N, K, out):
    """Y one element past an aligned address (no vector stores possible): the same
    bytes as an aligned Y, and the oracle's values."""
    import torch
    W = make_weight(0, f"test/fwdu/{N}x{K}", N, K, 0.02)
    X = make_acts(0, f"test/fwdu/X{M}x{K}", M, K, {})
    r = O.bitlinear(W, X)
    args = (dev(r["packed"]), dev(np.array([r["gamma"]], np.float32)), dev(r["Xq"]),
            dev(r["x_scale"]), dev(r["x_sum"].astype(np.int32)))
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[out]
    buf = torch.zeros(M * N + 1, dtype=tdt, device="cuda")
    Yu = buf[1:].view(M, N)
    gpu_lib.bitlinear_forward(*args, N=N, K=K, y_dtype=out, Y=Yu)
    Ya = gpu_lib.bitlinear_forward(*args, N=N, K=K, y_dtype=out)
    torch.cuda.synchronize()
    assert torch.equal(Yu, Ya)
    assert buf[0].item() == 0
    if out == "i32":
        assert_equal(host(Ya).astype(np.int64), r["acc"], "int32 accumulators")
    else:
        check_y(Ya, r["y"], out)


def test_forward_deterministic_on_side_stream(gpu_lib):
    import torch
    M, N, K = 40, 300, 1024
    Wt, Xq = _random_operands(M, N, K, seed=5)
    args = (dev(O.pack_codes(Wt)), dev(np.array([0.5], np.float32)), dev(Xq),
            dev(np.full(M, 0.25, np.float32)), dev(Xq.astype(np.int64).sum(1).astype(np.int32)))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = gpu_lib.bitlinear_forward(*args, N=N, K=K, y_dtype="f32", stream=s)
        y2 = gpu_lib.bitlinear_forward(*args, N=N, K=K, y_dtype="f32", stream=s)
    s.synchronize()
    assert torch.equal(y1, y2)


# --------------------------------------------------------------------------- whole path
def _whole_path(tb, W, X, out):
    import torch
    Wp, g = tb.bitlinear_pack_weights(dev(W))
    Xq, s, xs = tb.bitlinear_quant_acts(dev(X))
    N, K = W.shape
    acc = tb.bitlinear_forward(Wp, g, Xq, s, xs, N=N, K=K, y_dtype="i32")
    Y = tb.bitlinear_forward(Wp, g, Xq, s, xs, N=N, K=K, y_dtype=out)
    torch.cuda.synchronize()
    return dict(packed=host(Wp), gamma=host(g), Xq=host(Xq), x_scale=host(s), x_sum=host(xs),
                acc=host(acc), Y=Y)


def _compare_whole(got, W, X, out):
    r = O.bitlinear(W, X)
    assert_equal(f32_bits(got["gamma"]), f32_bits([r["gamma"]]), "gamma bits")
    assert_equal(got["packed"], r["packed"], "packed bytes")
    assert_equal(got["Xq"], r["Xq"], "X~")
    assert_equal(f32_bits(got["x_scale"]), f32_bits(r["x_scale"]), "x_scale bits")
    assert_equal(got["x_sum"].astype(np.int64), r["x_sum"], "x_sum")
    assert_equal(got["acc"].astype(np.int64), r["acc"], "int32 accumulators")
    check_y(got["Y"], r["y"], out)


def test_layer_512x256_fp32(gpu_lib):
    wl = WORKLOADS["layer-512x256"]
    p = wl.projections[0]
    W, X = wl.weight(p), wl.acts(p, 4)
    _compare_whole(_whole_path(gpu_lib, W, X, "f32"), W, X, "f32")


FULL = [(wl.name, p.name) for wl in WORKLOADS.values() if wl.name != "layer-512x256"
        for p in wl.projections]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wname,pname", FULL, ids=[f"{w}:{p}" for w, p in FULL])
def test_workload_full_size(gpu_lib, wname, pname):
    """Every intermediate of the whole path at the workload's real sizes, for
    every token count of the workload, compared in full."""
    wl = WORKLOADS[wname]
    p = next(q for q in wl.projections if q.name == pname)
    W = wl.weight(p)
    gamma = O.absmean_gamma(W)
    Wt = O.ternarize(W, gamma)
    import torch
    Wp, g = gpu_lib.bitlinear_pack_weights(dev(W))
    assert_equal(f32_bits(host(g)), f32_bits([gamma]), "gamma bits")
    assert_equal(host(Wp), O.pack_codes(Wt), "packed bytes")
    for M in wl.tokens:
        X = wl.acts(p, M)
        oq, os_, oxs, beta = O.quantize_activations(X)
        Xq, s, xs = gpu_lib.bitlinear_quant_acts(dev(X))
        assert_equal(host(Xq), oq, f"X~ M={M}")
        assert_equal(f32_bits(host(s)), f32_bits(os_), f"x_scale M={M}")
        assert_equal(host(xs).astype(np.int64), oxs, f"x_sum M={M}")
        acc_ref = O.integer_matmul(Wt, oq)
        acc = gpu_lib.bitlinear_forward(Wp, g, Xq, s, xs, N=p.N, K=p.K, y_dtype="i32")
        assert_equal(host(acc).astype(np.int64), acc_ref, f"accumulators M={M}")
        Y = gpu_lib.bitlinear_forward(Wp, g, Xq, s, xs, N=p.N, K=p.K, y_dtype=wl.out_dtype)
        y_ref = O.rescale(acc_ref, gamma, beta)
        check_y(Y, y_ref, wl.out_dtype)
        # the fused entry point the bench times for decode shapes
        Xd = dev(X)
        accf = gpu_lib.bitlinear_forward_f32(Wp, g, Xd, N=p.N, y_dtype="i32")
        assert_equal(host(accf).astype(np.int64), acc_ref, f"fused accumulators M={M}")
        check_y(gpu_lib.bitlinear_forward_f32(Wp, g, Xd, N=p.N, y_dtype=wl.out_dtype), y_ref,
                wl.out_dtype)
        torch.cuda.synchronize()


GROUPED_FULL = [(wl.name, M) for wl in WORKLOADS.values() if wl.shared_input for M in wl.tokens]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wname,M", GROUPED_FULL, ids=[f"{w}:M{m}" for w, m in GROUPED_FULL])
def test_workload_full_size_grouped(gpu_lib, wname, M):
    """A workload whose projections share their input, at its real sizes, through
    the grouped calls the bench times (one launch for all projections): the
    quantiser's outputs and every projection's accumulators in full against the
    oracle, and the bf16 outputs within tolerance."""
    import torch
    wl = WORKLOADS[wname]
    ps = list(wl.projections)
    K = ps[0].K
    X = wl.acts(ps[0], M)
    oq, os_, oxs, beta = O.quantize_activations(X)
    Wp, gm, refs = [], [], []
    for p in ps:
        W = wl.weight(p)
        gamma = O.absmean_gamma(W)
        Wt = O.ternarize(W, gamma)
        P, g = gpu_lib.bitlinear_pack_weights(dev(W))
        Wp.append(P)
        gm.append(g)
        acc_ref = O.integer_matmul(Wt, oq)
        refs.append((acc_ref, O.rescale(acc_ref, gamma, beta)))
    kw = dict(X_q_out=torch.empty((M, K), dtype=torch.int8, device="cuda"),
              x_scale_out=torch.empty(M, dtype=torch.float32, device="cuda"),
              x_sum_out=torch.empty(M, dtype=torch.int32, device="cuda"))
    Xd = dev(X)
    acc = gpu_lib.bitlinear_forward_f32_grouped(Wp, gm, Xd, y_dtype="i32", **kw)
    Y = gpu_lib.bitlinear_forward_f32_grouped(Wp, gm, Xd, y_dtype=wl.out_dtype)
    torch.cuda.synchronize()
    assert_equal(host(kw["X_q_out"]), oq, "X~")
    assert_equal(f32_bits(host(kw["x_scale_out"])), f32_bits(os_), "x_scale bits")
    assert_equal(host(kw["x_sum_out"]).astype(np.int64), oxs, "x_sum")
    for i, (acc_ref, y_ref) in enumerate(refs):
        assert_equal(host(acc[i]).astype(np.int64), acc_ref, f"accumulators of projection {i}")
        check_y(Y[i], y_ref, wl.out_dtype)
    # the pre-quantised grouped call on the quantiser's outputs
    acc2 = gpu_lib.bitlinear_forward_grouped(Wp, gm, kw["X_q_out"], kw["x_scale_out"],
                                            kw["x_sum_out"], K=K, y_dtype="i32")
    torch.cuda.synchronize()
    for i, (acc_ref, _) in enumerate(refs):
        assert_equal(host(acc2[i]).astype(np.int64), acc_ref, f"pre-quantised projection {i}")


# --------------------------------------------------------------------------- fused quant + forward
FUSED_SHAPES = [
    (1, 1, 16), (1, 40, 80), (2, 33, 1040), (3, 300, 4096), (5, 129, 512), (8, 64, 2048),
    (1, 8640, 3200), (1, 3200, 8640), (1, 64, 28672), (4, 100, 8192),
    # one token, K <= 4096 in steps of 64: quantised inside the vector-ALU decode
    # (row counts that leave a workgroup, and a wave, partly past the end)
    (1, 1, 64), (1, 3, 128), (1, 1001, 192), (1, 4096, 4096), (1, 11008, 4096),
    (1, 5, 4160), (1, 77, 8192), (1, 4096, 11008), (1, 33, 12288), (1, 9, 12352),
    # four pieces per lane, the activations of one piece held at a time
    (1, 1000, 16384), (1, 3, 16320), (1, 300, 14336), (1, 7, 16448),
    # two pieces per lane on 16384+ rows (8 waves per workgroup), the last
    # wave and workgroup partly past the end
    (1, 16390, 4160),
    # the persistent launch (2^25 weights and more): exactly 2^25, a partial
    # last 4-row group, the longest rows it takes
    (1, 2048, 16384), (1, 8193, 4096), (1, 1030, 32768),
    # outside the fused kernel's reach: two launches
    (9, 77, 1040), (16, 300, 4096), (8, 64, 8640), (40, 130, 1024), (2, 50, 40960),
    # two launches with K split across workgroups (workspace needed either
    # way): the skinny kernel's split, the GEMM's
    (48, 200, 8192), (100, 64, 8192),
]


@pytest.mark.parametrize("with_outputs", [True, False], ids=["outs", "noouts"])
@pytest.mark.parametrize("M,N,K", FUSED_SHAPES, ids=[f"M{m}N{n}K{k}" for m, n, k in FUSED_SHAPES])
def test_forward_f32_fused(gpu_lib, M, N, K, with_outputs):
    """Quantisation fused into the projection: the same X~, scales, sums and
    accumulators as the two separate calls, checked against the oracle."""
    import torch
    from fractions import Fraction
    W = make_weight(0, f"test/fused/W{N}x{K}", N, K, 0.02)
    X = make_acts(0, f"test/fused/X{M}x{K}", M, K,
                  {"outlier_frac": Fraction(1, 200), "outlier_scale": 100.0})
    r = O.bitlinear(W, X)
    P = dev(r["packed"])
    g = dev(np.array([r["gamma"]], np.float32))
    Xd = dev(X)
    outs = {}
    if with_outputs:
        outs = dict(X_q_out=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                    x_scale_out=torch.empty(M, dtype=torch.float32, device="cuda"),
                    x_sum_out=torch.empty(M, dtype=torch.int32, device="cuda"))
    acc = gpu_lib.bitlinear_forward_f32(P, g, Xd, N=N, y_dtype="i32", **outs)
    torch.cuda.synchronize()
    assert_equal(host(acc).astype(np.int64), r["acc"], "accumulators")
    if with_outputs:
        assert_equal(host(outs["X_q_out"]), r["Xq"], "X~ out")
        assert_equal(f32_bits(host(outs["x_scale_out"])), f32_bits(r["x_scale"]), "x_scale out")
        assert_equal(host(outs["x_sum_out"]).astype(np.int64), r["x_sum"], "x_sum out")
    for out in ("f32", "bf16"):
        Y = gpu_lib.bitlinear_forward_f32(P, g, Xd, N=N, y_dtype=out, **outs)
        check_y(Y, r["y"], out)


# --------------------------------------------------------------------------- grouped
GROUP_CASES = [
    # (M, K, Ns): one token on the vector ALU, LDS-staged decode, a K that is
    # not a multiple of 64, register-fed decode (X~ beyond the LDS budget),
    # and GEMM shapes run one projection after another (K split on some)
    (1, 4096, (4096, 1024, 1024)),
    (1, 8640, (3200, 3200)),
    (1, 192, (5, 17, 1, 64)),
    (3, 4096, (4096, 1024, 1024)),
    (16, 1040, (300, 17, 64, 129)),
    (16, 8192, (2048, 1040)),
    (40, 12288, (512, 200)),
    (130, 1040, (300, 64)),
    # one skinny launch over the group (workgroups never straddle two
    # projections): 4 row blocks per workgroup, 2 of 4 waves, 1 of 4 waves,
    # 64 tokens (and 40 tokens up to K = 8192)
    (8, 4096, (4096, 4096, 4096)),
    (32, 4096, (4096, 1024, 1024)),
    (20, 2048, (1000, 17, 3, 2000)),
    (64, 1024, (3000, 5000)), (40, 4096, (512, 200)),
]


@pytest.mark.parametrize("M,K,Ns", GROUP_CASES, ids=[f"M{m}K{k}G{len(n)}" for m, k, n in GROUP_CASES])
def test_forward_grouped(gpu_lib, M, K, Ns):
    """Every projection of the group: exact accumulators (oracle), and the same
    output bytes as its own bitlinear_forward call."""
    import torch
    X = make_acts(0, f"test/grp/X{M}x{K}", M, K, {})
    rs = [O.bitlinear(make_weight(0, f"test/grp/W{i}_{n}x{K}", n, K, 0.02), X)
          for i, n in enumerate(Ns)]
    Wp = [dev(r["packed"]) for r in rs]
    gm = [dev(np.array([r["gamma"]], np.float32)) for r in rs]
    xq, xs, xsum = dev(rs[0]["Xq"]), dev(rs[0]["x_scale"]), dev(rs[0]["x_sum"].astype(np.int32))
    acc = gpu_lib.bitlinear_forward_grouped(Wp, gm, xq, xs, xsum, K=K, y_dtype="i32")
    Yb = gpu_lib.bitlinear_forward_grouped(Wp, gm, xq, xs, xsum, K=K, y_dtype="bf16")
    torch.cuda.synchronize()
    for g, r in enumerate(rs):
        assert_equal(host(acc[g]).astype(np.int64), r["acc"], f"accumulators of projection {g}")
        check_y(Yb[g], r["y"], "bf16")
        single = gpu_lib.bitlinear_forward(Wp[g], gm[g], xq, xs, xsum, N=Ns[g], K=K, y_dtype="bf16")
        torch.cuda.synchronize()
        assert torch.equal(single, Yb[g]), f"projection {g} differs from its own call"


@pytest.mark.parametrize("with_outputs", [True, False], ids=["outs", "noouts"])
@pytest.mark.parametrize("M,K,Ns", [(1, 4096, (1024, 512, 512)), (2, 3200, (8640, 64)),
                                    (5, 1040, (300, 17)), (48, 4096, (200, 64)),
                                    (1, 4096, (11008, 4096, 1004))],
                         ids=["fusedM1", "twoM2", "smallM5", "gemmM48", "wideM1"])
def test_forward_f32_grouped(gpu_lib, M, K, Ns, with_outputs):
    """Quantise once, then every projection: the quantiser outputs and each
    projection's accumulators as the oracle's."""
    import torch
    X = make_acts(0, f"test/grpf/X{M}x{K}", M, K, {"outlier_frac": Fraction(1, 100), "outlier_scale": 50.0})
    rs = [O.bitlinear(make_weight(0, f"test/grpf/W{i}_{n}x{K}", n, K, 0.02), X)
          for i, n in enumerate(Ns)]
    Wp = [dev(r["packed"]) for r in rs]
    gm = [dev(np.array([r["gamma"]], np.float32)) for r in rs]
    kw = {}
    if with_outputs:
        kw = dict(X_q_out=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                  x_scale_out=torch.empty(M, dtype=torch.float32, device="cuda"),
                  x_sum_out=torch.empty(M, dtype=torch.int32, device="cuda"))
    acc = gpu_lib.bitlinear_forward_f32_grouped(Wp, gm, dev(X), y_dtype="i32", **kw)
    Y = gpu_lib.bitlinear_forward_f32_grouped(Wp, gm, dev(X), y_dtype="f32")
    torch.cuda.synchronize()
    for g, r in enumerate(rs):
        assert_equal(host(acc[g]).astype(np.int64), r["acc"], f"accumulators of projection {g}")
        check_y(Y[g], r["y"], "f32")
    if with_outputs:
        assert_equal(host(kw["X_q_out"]), rs[0]["Xq"], "X~")
        assert_equal(f32_bits(host(kw["x_scale_out"])), f32_bits(rs[0]["x_scale"]), "x_scale bits")
        assert_equal(host(kw["x_sum_out"]).astype(np.int64), rs[0]["x_sum"], "x_sum")
