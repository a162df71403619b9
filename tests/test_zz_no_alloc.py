"""bitlinear_forward_f32_noalloc (the library's own scratch array as the
workspace) against bitlinear_forward_f32 with a caller workspace, through the
C ABI: identical bytes on two calls in a row, the second smaller, so the
array's leftover contents from the first call must not leak into the second.
"""
import numpy as np
import pytest

from synth import make_acts, make_weight
from tests.gpu_common import assert_equal, dev, host

pytestmark = pytest.mark.gpu

# (M, N, K): quantiser + skinny kernel (quantiser region in the scratch), the
# K-split skinny kernel (partial sums too), the GEMM with a K split, and one
# fused single-token launch (no scratch at all); each followed by a smaller one
CASES = [
    ((40, 3000, 4096), (20, 1000, 2048)),
    ((64, 2048, 12288), (24, 512, 4096)),
    ((96, 1024, 8192), (70, 300, 2048)),
    ((1, 8640, 3200), (1, 77, 192)),
]


def _inputs(M, N, K, tag):
    import torch
    import ternary_bitlinear_amd as tb
    W = make_weight(0, f"test/noalloc/W{tag}{N}x{K}", N, K, 0.02)
    X = make_acts(0, f"test/noalloc/X{tag}{M}x{K}", M, K, {})
    Wp, g = tb.bitlinear_pack_weights(dev(W))
    torch.cuda.synchronize()
    return Wp, g, dev(X)


def _both(tb, Wp, g, X, N, out):
    import torch
    M, K = X.shape
    outs_a = [torch.full((M, K), 77, dtype=torch.int8, device="cuda"),
              torch.zeros(M, dtype=torch.float32, device="cuda"),
              torch.zeros(M, dtype=torch.int32, device="cuda")]
    outs_b = [torch.full((M, K), -5, dtype=torch.int8, device="cuda"),
              torch.ones(M, dtype=torch.float32, device="cuda"),
              torch.ones(M, dtype=torch.int32, device="cuda")]
    ya = tb.bitlinear_forward_f32(Wp, g, X, N=N, y_dtype=out, X_q_out=outs_a[0],
                                  x_scale_out=outs_a[1], x_sum_out=outs_a[2])
    yb = tb.bitlinear_forward_f32_noalloc(Wp, g, X, N=N, y_dtype=out, X_q_out=outs_b[0],
                                          x_scale_out=outs_b[1], x_sum_out=outs_b[2])
    # and without the optional outputs (the quantiser region then holds X~)
    yc = tb.bitlinear_forward_f32_noalloc(Wp, g, X, N=N, y_dtype=out)
    torch.cuda.synchronize()
    return ya, yb, yc, outs_a, outs_b


@pytest.mark.parametrize("big,small", CASES, ids=[f"M{a[0]}N{a[1]}K{a[2]}" for a, _ in CASES])
def test_noalloc_matches_forward_f32(gpu_lib, big, small):
    import torch
    tb = gpu_lib
    print(f"noalloc case {big} then {small}", flush=True)
    for i, (M, N, K) in enumerate((big, small)):
        Wp, g, X = _inputs(M, N, K, f"c{i}")
        for out in ("i32", "bf16", "f32"):
            ya, yb, yc, oa, ob = _both(tb, Wp, g, X, N, out)
            view = (lambda t: host(t.view(torch.int16))) if out == "bf16" else host
            assert_equal(view(yb), view(ya), f"Y ({out}, call {i})")
            assert_equal(view(yc), view(ya), f"Y without outputs ({out}, call {i})")
            for a, b, what in zip(oa, ob, ("X~", "x_scale", "x_sum")):
                assert_equal(host(b), host(a), f"{what} (call {i})")


def test_noalloc_refuses_shapes_beyond_the_array(gpu_lib):
    import torch
    tb = gpu_lib
    M, N, K = 2048, 256, 32768          # quantiser region alone: 64 MiB
    assert tb.forward_f32_workspace_bytes(M, N, K) > tb.NOALLOC_SCRATCH_BYTES
    Wp = torch.zeros((N, K // 4), dtype=torch.uint8, device="cuda")
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    X = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    with pytest.raises(tb.BitLinearError) as e:
        tb.bitlinear_forward_f32_noalloc(Wp, g, X, N=N, y_dtype="bf16")
    assert e.value.status == 7
