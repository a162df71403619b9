"""Projections captured in a HIP graph and replayed, as the bench times them:
every replay, with eager work on the same stream between replays, gives the
same bytes as the eager call.  Covers the fused single-token launch, the
skinny kernel, its K split and the GEMM's (two launches sharing a workspace),
the tiled GEMM, the grouped launch and the RMS-normalised fused launch."""
import numpy as np
import pytest

from synth import make_acts, make_weight
from tests.gpu_common import dev

pytestmark = pytest.mark.gpu

CASES = [("f32", 1, 3200, 8640), ("f32", 16, 4096, 4096), ("f32", 48, 2000, 8192),
         ("f32", 64, 8192, 12288), ("f32", 300, 1040, 1024), ("grouped", 1, 4096, 4096),
         ("rmsnorm", 1, 4096, 4096)]


@pytest.mark.parametrize("kind,M,N,K", CASES, ids=[f"{k}-M{m}N{n}K{kk}" for k, m, n, kk in CASES])
def test_graph_replays_match_eager(gpu_lib, kind, M, N, K):
    import torch
    tb = gpu_lib
    W = make_weight(0, f"test/graph/{N}x{K}", N, K, 0.02)
    X = dev(make_acts(0, f"test/graph/X{M}x{K}", M, K, {}))
    Wp, g = tb.bitlinear_pack_weights(dev(W))
    norm_g = dev(np.linspace(0.5, 1.5, K).astype(np.float32))
    s = torch.cuda.Stream()
    Ns = [N, N // 4, N // 4] if kind == "grouped" else [N]
    Ws = [Wp] + [Wp[: n] for n in Ns[1:]]
    Ys = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for n in Ns]
    if kind == "grouped":
        need = tb.forward_f32_grouped_workspace_bytes(M, Ns, K)
    elif kind == "rmsnorm":
        need = tb.forward_rmsnorm_workspace_bytes(M, N, K)
    else:
        need = tb.forward_f32_workspace_bytes(M, N, K)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def call():
        if kind == "grouped":
            tb.bitlinear_forward_f32_grouped(Ws, [g] * len(Ns), X, Ns=Ns, y_dtype="bf16", Y=Ys,
                                             workspace=ws, stream=s)
        elif kind == "rmsnorm":
            tb.bitlinear_forward_rmsnorm(Wp, g, X, norm_g, N=N, y_dtype="bf16", Y=Ys[0],
                                         workspace=ws, stream=s)
        else:
            tb.bitlinear_forward_f32(Wp, g, X, N=N, y_dtype="bf16", Y=Ys[0], workspace=ws,
                                     stream=s)

    with torch.cuda.stream(s):
        call()
    s.synchronize()
    want = [y.clone() for y in Ys]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call()
    for rep in range(3):
        for y in Ys:
            y.fill_(0)
        with torch.cuda.stream(s):
            torch.neg(X, out=torch.empty_like(X))      # eager work between replays
            graph.replay()
        s.synchronize()
        for y, w in zip(Ys, want):
            assert torch.equal(y, w), f"replay {rep}"
