"""The bench's algorithmic bytes per launch (the numerator of the roofline's
`achieved`), against per-call totals worked out by hand for the workloads'
shapes (MB, two decimals): packed W (N K / 4) + X~ (M K) + per-token scale
and sum + Y (2 M N for bf16).  No GPU."""
import pytest

import bench
from synth import WORKLOADS


def _p(wname, pname):
    return next(q for q in WORKLOADS[wname].projections if q.name == pname)


@pytest.mark.parametrize("wname,pname,M,mb", [
    ("decode-3b", "ffn_up", 1, 6.93),
    ("decode-7b", "ffn_up", 1, 11.30), ("decode-7b", "ffn_up", 8, 11.48),
    ("decode-7b", "ffn_up", 32, 12.11), ("decode-7b", "ffn_up", 64, 12.94),
    ("prefill-7b", "ffn_up", 2048, 64.76),
    ("ffn-70b", "ffn_up", 1, 58.8),
])
def test_alg_bytes_match_the_tables(wname, pname, M, mb):
    P = _p(wname, pname)
    b = bench.alg_bytes(P, M, "bf16")
    assert b == P.N * P.K // 4 + M * P.K + 8 * M + 2 * M * P.N + 4
    assert abs(b / 1e6 - mb) < 0.0105 * max(1.0, mb / 10), (b, mb)


def test_fused_and_grouped_counting():
    P = _p("decode-3b", "ffn_up")
    # fused: fp32 X read in place of X~, x_scale and x_sum
    assert bench.alg_bytes_f32(P, 1, "bf16") - bench.alg_bytes(P, 1, "bf16") == 4 * P.K - P.K - 8
    qkv = list(WORKLOADS["attn-qkv-7b"].projections)
    M = 16
    one = [bench.alg_bytes(Q, M, "bf16") for Q in qkv]
    # a grouped launch reads the shared activations once
    assert bench.launch_alg_bytes(qkv, M, "bf16", False, True) == sum(one) - 2 * (M * 4096 + 8 * M)
    # separate launches: the mean launch
    ffn = list(WORKLOADS["decode-3b"].projections)
    want = sum(bench.alg_bytes_f32(Q, 1, "bf16") for Q in ffn) / 2
    assert bench.launch_alg_bytes(ffn, 1, "bf16", True, False) == want


def test_multi_launch_bytes_ffn70b():
    # one multi-projection launch over both 70B projections, each with its own
    # fp32 activations (one token, bf16 out), worked by hand:
    #   8192 -> 28672: 58 720 256 packed + 32 768 X + 57 344 Y + 4 gamma = 58 810 372
    #   28672 -> 8192: 58 720 256 packed + 114 688 X + 16 384 Y + 4 gamma = 58 851 332
    from synth import WORKLOADS
    shapes = list(WORKLOADS["ffn-70b"].projections)
    assert bench.launch_alg_bytes(shapes, 1, "bf16", True, False, multi=True) == 117_661_704


def test_probe_library_exports_the_bench_probes():
    """The chip-limit probe library the bench loads (built beside the
    BitLinear library by build()) exports every probe the bench calls; no
    probe runs here."""
    import ctypes
    import os
    from ternary_bitlinear_amd.build import PROBES_LIB
    if not os.path.exists(PROBES_LIB):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(PROBES_LIB)
    for name in ("probe_stream_read", "probe_bcast_read", "probe_mfma_loop"):
        assert hasattr(lib, name), name


def test_bench_refuses_more_than_one_gpu():
    """The path runs on one GPU: bench.py exits with a message (status 2)
    before touching any device when asked for more."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
