#!/usr/bin/env python3
"""Throughput of the BitLinear b1.58 projection on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--tokens M]

A step is one pass of the per-token path over one batch of synthetic input:
for every projection of the workload, per-token activation quantisation and
the projection with its fused rescale, through bitlinear_forward_f32 (one
launch for decode shapes, where the quantiser runs in the projection's
prologue; otherwise bitlinear_quant_acts then bitlinear_forward).  Weights are
ternarised and packed once at set-up (bitlinear_pack_weights), as at
inference; that step is timed separately and reported under "rows", as are
the standalone quantiser and the projection on pre-quantised activations.
Packed weights are replicated into enough copies (>= 512 MB per projection)
that successive steps read them from HBM rather than from the 256 MB
Infinity Cache.  Steps are replayed from a HIP graph so that host launch
overhead does not hide the device time.

Prints one JSON line: the whole-step throughput ("value"), the roofline of the
dominant kernel, the CPU oracle timed on a bounded sample, and one entry per
step of the path.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BitLinear GEMV weight GB/s (% HBM peak); prefill int8 TOPS (% MFMA peak)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA
ROTATE_BYTES = 512 << 20     # weight copies rotated per step: beyond the 256 MB MALL
OUT_BYTES = {"f32": 4, "bf16": 2}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode-3b")
    ap.add_argument("--tokens", type=int, default=None, help="M; default: the workload's first")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


class Timer:
    """Device time of work enqueued on one stream, from HIP events on that stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def __call__(self, fn, reps=1):
        t = self.torch
        t.cuda.synchronize()
        a = t.cuda.Event(enable_timing=True)
        b = t.cuda.Event(enable_timing=True)
        a.record(self.stream)
        with t.cuda.stream(self.stream):
            for _ in range(reps):
                fn()
        b.record(self.stream)
        b.synchronize()
        t.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3   # seconds


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ternary_bitlinear_amd as tb
    from synth import WORKLOADS

    wl = WORKLOADS[args.workload]
    M = args.tokens or wl.tokens[0]
    out = wl.out_dtype
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tb.load()
    stream = torch.cuda.Stream()
    timer = Timer(torch, stream)

    # ---------------- set-up: inputs resident in HBM, weights packed once
    projs = []
    for p in wl.projections:
        W = wl.weight(p)
        X = wl.acts(p, M)
        Wd = torch.from_numpy(W).to(dev)
        Wp, g = tb.bitlinear_pack_weights(Wd)
        torch.cuda.synchronize()
        projs.append(dict(p=p, W_host=W, X_host=X, Wd=Wd, Wp=Wp, g=g,
                          X=torch.from_numpy(X).to(dev),
                          Xq=torch.empty((M, p.K), dtype=torch.int8, device=dev),
                          s=torch.empty(M, dtype=torch.float32, device=dev),
                          xs=torch.empty(M, dtype=torch.int32, device=dev),
                          Y=torch.empty((M, p.N), dtype=getattr(torch, {"f32": "float32", "bf16": "bfloat16"}[out]),
                                        device=dev)))
    wbytes_step = sum(q["p"].N * q["p"].K // 4 for q in projs)
    # every projection alone cycles through >= ROTATE_BYTES of copies
    copies = max(1, math.ceil(ROTATE_BYTES / min(q["p"].N * q["p"].K // 4 for q in projs)))
    for q in projs:
        q["Wc"] = [q["Wp"]] + [q["Wp"].clone() for _ in range(copies - 1)]
    torch.cuda.synchronize()

    for q in projs:
        need = tb.forward_f32_workspace_bytes(M, q["p"].N, q["p"].K)
        q["ws"] = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        q["fused"] = need == 0

    def step(r):
        # quantise + project; one launch when the shape fuses, else two
        for q in projs:
            tb.bitlinear_forward_f32(q["Wc"][r % copies], q["g"], q["X"], N=q["p"].N,
                                     y_dtype=out, Y=q["Y"], workspace=q["ws"], stream=stream)

    def graph_of(fn_list):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for fn in fn_list:
                    fn()
        return g

    # ---------------- warm-up (eager, then graph)
    with torch.cuda.stream(stream):
        for r in range(args.warmup):
            step(r)
    torch.cuda.synchronize()
    cycle = min(copies, args.steps)
    g_cycle = graph_of([lambda r=r: step(r) for r in range(cycle)])
    rem = args.steps % cycle
    g_rem = graph_of([lambda r=r: step(r) for r in range(rem)]) if rem else None
    g_cycle.replay()
    torch.cuda.synchronize()

    # ---------------- timed region: exactly K steps
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()

    def timed():
        for _ in range(args.steps // cycle):
            g_cycle.replay()
        if g_rem is not None:
            g_rem.replay()
    elapsed = timer(timed)
    t_wall = time.perf_counter() - t_wall0
    ms_per_step = elapsed / args.steps * 1e3

    prefill = M > 64
    if prefill:
        ops_step = sum(2 * M * q["p"].N * q["p"].K for q in projs)
        value, unit = ops_step / (elapsed / args.steps) / 1e12, "TOP/s"
    else:
        value, unit = wbytes_step / (elapsed / args.steps) / 1e9, "GB/s"

    # ---------------- the dominant kernel: the projection (bitlinear_forward on
    # pre-quantised activations) on the largest projection of the workload
    dom = max(projs, key=lambda q: q["p"].N * q["p"].K)
    P = dom["p"]
    reps = max(1, 2000 // copies) if not prefill else max(1, 200 // copies)
    with torch.cuda.stream(stream):
        tb.bitlinear_quant_acts(dom["X"], dom["Xq"], dom["s"], dom["xs"], stream=stream)

    def fwd_q(r):
        tb.bitlinear_forward(dom["Wc"][r % copies], dom["g"], dom["Xq"], dom["s"], dom["xs"],
                             N=P.N, K=P.K, y_dtype=out, Y=dom["Y"], stream=stream)
    g_fq = graph_of([lambda r=r: fwd_q(r) for r in range(copies)])
    g_fq.replay()
    t_fq = timer(g_fq.replay, reps) / (reps * copies)
    # algorithmic bytes of one launch: packed W, X~, x_scale, x_sum, Y, gamma
    alg_bytes = P.N * P.K // 4 + M * P.K + 8 * M + OUT_BYTES[out] * M * P.N + 4
    kname = "k_decode" if M <= 16 else "k_gemm"
    if prefill:
        achieved = 2 * M * P.N * P.K / t_fq / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS,
                "unit": "TOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4)}
    else:
        achieved = alg_bytes / t_fq / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": None, "kernel": kname, "shape": f"M{M} {P.K}->{P.N}",
                 "us_per_launch": round(t_fq * 1e6, 3), "algorithmic_bytes": alg_bytes,
                 "timing": "HIP events around a graph of back-to-back launches over the "
                           "rotated weight copies, on the launch stream"})
    traffic = load_traffic(kname, P, M)
    if traffic is not None:
        roof["traffic"] = traffic

    # quantise + project as the step runs it (one launch when fused)
    def fwd(r):
        tb.bitlinear_forward_f32(dom["Wc"][r % copies], dom["g"], dom["X"], N=P.N, y_dtype=out,
                                 Y=dom["Y"], workspace=dom["ws"], stream=stream)
    g_fwd = graph_of([lambda r=r: fwd(r) for r in range(copies)])
    g_fwd.replay()
    t_fwd = timer(g_fwd.replay, reps) / (reps * copies)

    # ---------------- every step of the path, timed on its own
    rows = {}
    q0 = projs[0]
    ws = torch.empty(tb.pack_workspace_bytes(q0["p"].N, q0["p"].K), dtype=torch.uint8, device=dev)
    Wp_tmp = torch.empty_like(q0["Wp"])
    g_tmp = torch.empty_like(q0["g"])
    with torch.cuda.stream(stream):
        tb.bitlinear_pack_weights(q0["Wd"], Wp_tmp, g_tmp, ws, stream=stream)
    t_pack = timer(lambda: tb.bitlinear_pack_weights(q0["Wd"], Wp_tmp, g_tmp, ws, stream=stream),
                   5) / 5
    pk_bytes = q0["p"].N * q0["p"].K * 4 + q0["p"].N * q0["p"].K // 4
    rows["pack_weights"] = {"shape": f"{q0['p'].K}->{q0['p'].N}", "us": round(t_pack * 1e6, 2),
                            "GB/s": round(pk_bytes / t_pack / 1e9, 1),
                            "note": "3 launches; reads W twice (exact sum, then codes)"}
    g_q = graph_of([lambda: tb.bitlinear_quant_acts(q0["X"], q0["Xq"], q0["s"], q0["xs"],
                                                     stream=stream)] * 50)
    g_q.replay()
    t_q = timer(g_q.replay, 10) / 500
    q_bytes = M * q0["p"].K * 5 + 8 * M
    rows["quant_acts"] = {"shape": f"M{M} K{q0['p'].K}", "us": round(t_q * 1e6, 3),
                          "GB/s": round(q_bytes / t_q / 1e9, 1)}
    rows["forward" + ("_gemm" if M > 16 else "_decode")] = {
        "shape": roof["shape"], "us": roof["us_per_launch"],
        ("TOP/s" if prefill else "GB/s"): roof["achieved"],
        "epilogue": f"gamma*beta rescale fused, {out} out"}
    f32_bytes = P.N * P.K // 4 + 4 * M * P.K + OUT_BYTES[out] * M * P.N + 4
    rows["forward_f32"] = {"shape": roof["shape"], "us": round(t_fwd * 1e6, 3),
                           "fused": dom["fused"],
                           ("TOP/s" if prefill else "GB/s"): round(
                               (2 * M * P.N * P.K / t_fwd / 1e12) if prefill
                               else f32_bytes / t_fwd / 1e9, 2 if prefill else 1)}

    # ---------------- CPU oracle on a bounded sample of the same step
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(projs, M, args.cpu_seconds, wbytes_step, prefill)

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": M,
                   "projections": [f"{q['p'].K}->{q['p'].N}" for q in projs],
                   "out": out, "weight_copies": copies, "seed": wl.seed, "graph": True},
        "roofline": roof, "cpu_baseline": cpu, "rows": rows,
        "wall_s_timed": round(t_wall, 3),
    }
    print(json.dumps(line), flush=True)


def load_traffic(kernel, P, M):
    """HBM bytes per launch from committed rocprofv3 counter summaries
    (profiles/traffic.json), when they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    import hashlib
    with open(path) as f:
        data = json.load(f)
    src = os.path.join(ROOT, "ternary_bitlinear_amd", "csrc", "forward.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    key = f"{kernel} M{M} {P.K}->{P.N}"
    ent = data.get(key)
    if not ent or ent.get("source_sha256_16") != digest:
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(projs, M, seconds, wbytes_step, prefill):
    """The oracle's per-step work (quantise, integer product, rescale) for every
    projection, repeated on the host for about `seconds`."""
    import numpy as np
    from oracle import bitlinear_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    prep = []
    for q in projs:
        gamma = O.absmean_gamma(q["W_host"])
        prep.append((O.ternarize(q["W_host"], gamma), gamma, q["X_host"]))

    def one_step():
        for Wt, gamma, X in prep:
            Xq, _, _, beta = O.quantize_activations(X)
            O.rescale(O.integer_matmul(Wt, Xq), gamma, beta)
    n = 0
    t0 = time.perf_counter()
    while True:
        one_step()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or (n >= 1 and el * (n + 1) / n > 3 * seconds):
            break
    per = el / n
    if prefill:
        ops = sum(2 * M * q["p"].N * q["p"].K for q in projs)
        v, unit = ops / per / 1e12, "TOP/s"
    else:
        v, unit = wbytes_step / per / 1e9, "GB/s"
    return {"value": round(v, 6), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{n} full steps of the same workload ({el:.1f} s)",
            "ms_per_step": round(per * 1e3, 3)}


if __name__ == "__main__":
    main()
