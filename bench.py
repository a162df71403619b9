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
step of the path.  The dominant kernel is the step's own launch where the step
is nothing but fused launches (decode shapes), else the projection on
pre-quantised activations (bitlinear_forward), which is also reported as a row
in both cases.
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
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: at least 200 steps and "
                         "0.5 s, so the GPU clocks have ramped up; the count is reported)")
    ap.add_argument("--workload", default="decode-3b")
    ap.add_argument("--tokens", type=int, default=None, help="M; default: the workload's first")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run one plain copy of known size, then bitlinear_forward once per "
                         "projection and weight copy, and exit (for rocprofv3 --pmc runs)")
    ap.add_argument("--probe-reps", type=int, default=1,
                    help="with --traffic-probe: launches per weight copy (for a kernel trace)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn the FETCH_SIZE and WRITE_SIZE counter runs of "
                         "--traffic-probe into profiles/traffic.json")
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
    if args.traffic_from:
        traffic_from(args)
        return
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
    grouped = wl.shared_input
    if grouped:
        # every projection reads one X (and, after quantisation, one X~)
        for q in projs[1:]:
            for key in ("X", "Xq", "s", "xs"):
                q[key] = projs[0][key]
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
    Ns = [q["p"].N for q in projs]
    g_need = tb.forward_f32_grouped_workspace_bytes(M, Ns, projs[0]["p"].K) if grouped else 0
    ws_group = torch.empty(max(g_need, 16), dtype=torch.uint8, device=dev)

    def step_separate(r):
        # quantise + project; one launch when the shape fuses, else two
        for q in projs:
            tb.bitlinear_forward_f32(q["Wc"][r % copies], q["g"], q["X"], N=q["p"].N,
                                     y_dtype=out, Y=q["Y"], workspace=q["ws"], stream=stream)

    def step_grouped(r):
        # quantise once, then every projection in one launch (decode shapes)
        tb.bitlinear_forward_f32_grouped([q["Wc"][r % copies] for q in projs],
                                         [q["g"] for q in projs], projs[0]["X"], Ns=Ns,
                                         y_dtype=out, Y=[q["Y"] for q in projs],
                                         workspace=ws_group, stream=stream)

    step = step_grouped if grouped else step_separate
    fused_step = step_is_fused(tb, [q["p"] for q in projs], M, grouped)

    if args.traffic_probe:
        traffic_probe(tb, torch, projs, M, out, copies, stream, dev, wl, grouped,
                      step if fused_step else None, reps=args.probe_reps)
        return

    def graph_of(fn_list):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for fn in fn_list:
                    fn()
        return g

    # ---------------- warm-up: eager steps, then the step graph replayed (by
    # default until 0.5 s have passed, so that the clocks have ramped up)
    w_eager = min(args.warmup, 200) if args.warmup is not None else 200
    with torch.cuda.stream(stream):
        for r in range(w_eager):
            step(r)
    torch.cuda.synchronize()
    cycle = min(copies, args.steps)
    g_cycle = graph_of([lambda r=r: step(r) for r in range(cycle)])
    rem = args.steps % cycle
    g_rem = graph_of([lambda r=r: step(r) for r in range(rem)]) if rem else None
    warmup = w_eager
    t_w0 = time.perf_counter()
    while True:
        if args.warmup is not None:
            if warmup >= args.warmup:
                break
            if args.warmup - warmup < cycle:      # exactly W: finish eagerly
                with torch.cuda.stream(stream):
                    for r in range(args.warmup - warmup):
                        step(r)
                warmup = args.warmup
                break
        elif time.perf_counter() - t_w0 >= 0.5:
            break
        g_cycle.replay()
        warmup += cycle
        torch.cuda.synchronize()
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

    # ---------------- the dominant kernel.  The projection on pre-quantised
    # activations (bitlinear_forward) over every projection of the workload,
    # back to back over the rotated weight copies; when the step is nothing but
    # fused launches (decode shapes), the step's own launch is the dominant
    # kernel and is timed the same way.
    with torch.cuda.stream(stream):
        for q in projs:
            tb.bitlinear_quant_acts(q["X"], q["Xq"], q["s"], q["xs"], stream=stream)
    proj_roof, _ = roofline(tb, torch, timer, graph_of, projs, M, out, copies, prefill, stream,
                            grouped)
    roof = proj_roof
    if fused_step:
        roof, _ = roofline(tb, torch, timer, graph_of, projs, M, out, copies, prefill, stream,
                           grouped, fused_step=step)
    dom = max(projs, key=lambda q: q["p"].N * q["p"].K)
    P = dom["p"]

    # quantise + project as the step runs it (one launch when fused)
    def fwd(r):
        tb.bitlinear_forward_f32(dom["Wc"][r % copies], dom["g"], dom["X"], N=P.N, y_dtype=out,
                                 Y=dom["Y"], workspace=dom["ws"], stream=stream)
    g_fwd = graph_of([lambda r=r: fwd(r) for r in range(copies)])
    g_fwd.replay()
    reps = max(1, (2000 if not prefill else 200) // copies)
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
                            "frac_of_hbm": round(pk_bytes / t_pack / 1e9 / HBM_PEAK_GBS, 4),
                            "note": "3 launches; reads W twice (exact sum, then codes); bytes "
                                    "counted once: 4NK read + NK/4 written"}
    g_q = graph_of([lambda: tb.bitlinear_quant_acts(q0["X"], q0["Xq"], q0["s"], q0["xs"],
                                                     stream=stream)] * 50)
    g_q.replay()
    t_q = timer(g_q.replay, 10) / 500
    q_bytes = M * q0["p"].K * 5 + 8 * M
    rows["quant_acts"] = {"shape": f"M{M} K{q0['p'].K}", "us": round(t_q * 1e6, 3),
                          "GB/s": round(q_bytes / t_q / 1e9, 1),
                          "frac_of_hbm": round(q_bytes / t_q / 1e9 / HBM_PEAK_GBS, 4)}
    rows["forward"] = {
        "shape": proj_roof["shape"], "kernel": proj_roof["kernel"],
        "us": proj_roof["us_per_launch"],
        ("TOP/s" if prefill else "GB/s"): proj_roof["achieved"],
        "entry_point": proj_roof["entry_point"],
        "epilogue": f"gamma*beta rescale fused, {out} out"}
    if prefill:
        rows["vendor_int8_mm"] = vendor_int8_mm(tb, torch, timer, stream, dom, M)
    f32_bytes = P.N * P.K // 4 + 4 * M * P.K + OUT_BYTES[out] * M * P.N + 4
    rows["forward_f32"] = {"shape": f"M{M} {P.K}->{P.N}", "us": round(t_fwd * 1e6, 3),
                           "fused": dom["fused"],
                           ("TOP/s" if prefill else "GB/s"): round(
                               (2 * M * P.N * P.K / t_fwd / 1e12) if prefill
                               else f32_bytes / t_fwd / 1e9, 2 if prefill else 1)}
    # the same launch with warm caches: one weight copy replayed back to back,
    # so the packed weights stay in the 256 MB MALL (and partly in L2); for
    # context only, every other number here reads the weights from HBM
    g_warm = graph_of([lambda: fwd(0)] * min(copies, 64))
    g_warm.replay()
    t_warm = timer(g_warm.replay, reps) / (reps * min(copies, 64))
    rows["forward_f32_warm_cache"] = {"shape": f"M{M} {P.K}->{P.N}", "us": round(t_warm * 1e6, 3),
                                      "note": "one weight copy, cache-resident: not an HBM number"}
    del g_warm

    # base-3 weights (1.6 bits per weight, up to 16 tokens): each projection
    # on the same quantised activations in both formats, back to back over
    # >= 512 MB of weight copies, in one process
    if M <= 16:
        b3 = {"us": [], "us_blt2": [], "bytes": []}
        for q in projs:
            N_, K_ = q["p"].N, q["p"].K
            P3, g3 = tb.bitlinear_pack_weights_base3(q["Wd"])
            c3 = max(1, math.ceil(ROTATE_BYTES / P3.numel()))
            W3 = [P3] + [P3.clone() for _ in range(c3 - 1)]
            torch.cuda.synchronize()

            def f3(r, q=q, W3=W3, g3=g3, N_=N_, K_=K_):
                tb.bitlinear_forward_base3(W3[r], g3, q["Xq"], q["s"], q["xs"], N=N_, K=K_,
                                           y_dtype=out, Y=q["Y"], stream=stream)

            def f2(r, q=q, N_=N_, K_=K_):
                tb.bitlinear_forward(q["Wc"][r % copies], q["g"], q["Xq"], q["s"], q["xs"],
                                     N=N_, K=K_, y_dtype=out, Y=q["Y"], stream=stream)
            for key, fn, n_c in (("us", f3, c3), ("us_blt2", f2, copies)):
                gq = graph_of([lambda r=r, fn=fn: fn(r) for r in range(n_c)])
                gq.replay()
                rq = max(1, 2000 // n_c)
                b3[key].append(timer(gq.replay, rq) / (rq * n_c))
                del gq
            b3["bytes"].append(P3.numel() + M * K_ + 8 * M + OUT_BYTES[out] * M * N_ + 4)
            del W3, P3
            torch.cuda.empty_cache()
        t3 = sum(b3["us"]) / len(b3["us"])
        rows["forward_base3"] = {
            "shape": f"M{M} " + ", ".join(f"{q['p'].K}->{q['p'].N}" for q in projs),
            "format": "BLT3-v1 (5 weights per byte)", "entry_point": "bitlinear_forward_base3",
            "us": round(t3 * 1e6, 3),
            "us_per_projection": [round(t * 1e6, 3) for t in b3["us"]],
            "blt2_us_per_projection": [round(t * 1e6, 3) for t in b3["us_blt2"]],
            "GB/s": round(sum(b3["bytes"]) / len(b3["bytes"]) / t3 / 1e9, 1)}
        ws3 = torch.empty(tb.pack_workspace_bytes(q0["p"].N, q0["p"].K), dtype=torch.uint8,
                          device=dev)
        P3_tmp = torch.empty((q0["p"].N, 16 * -(-q0["p"].K // 80)), dtype=torch.uint8, device=dev)
        with torch.cuda.stream(stream):
            tb.bitlinear_pack_weights_base3(q0["Wd"], P3_tmp, g_tmp, ws3, stream=stream)
        t_pack3 = timer(lambda: tb.bitlinear_pack_weights_base3(q0["Wd"], P3_tmp, g_tmp, ws3,
                                                                stream=stream), 5) / 5
        rows["pack_weights_base3"] = {"shape": f"{q0['p'].K}->{q0['p'].N}",
                                      "us": round(t_pack3 * 1e6, 2)}
        del P3_tmp, ws3

    # RMS normalisation in front of the quantiser (the step before the
    # projection): the normalising quantiser alone, and fused into the
    # projection as the dominant projection would run it
    from synth import make_weight
    norm_g = torch.from_numpy((1.0 + make_weight(wl.seed, "bench/norm_g", 1, q0["p"].K, 0.1)[0])
                              .astype(np.float32)).to(dev)
    g_rq = graph_of([lambda: tb.bitlinear_rmsnorm_quant(q0["X"], norm_g, q0["Xq"], q0["s"],
                                                         q0["xs"], stream=stream)] * 50)
    g_rq.replay()
    t_rq = timer(g_rq.replay, 10) / 500
    rq_bytes = M * q0["p"].K * 5 + 4 * q0["p"].K + 8 * M
    rows["rmsnorm_quant"] = {"shape": f"M{M} K{q0['p'].K}", "us": round(t_rq * 1e6, 3),
                             "GB/s": round(rq_bytes / t_rq / 1e9, 1),
                             "frac_of_hbm": round(rq_bytes / t_rq / 1e9 / HBM_PEAK_GBS, 4)}
    gd = dom["p"].K
    dom_norm_g = norm_g if gd == q0["p"].K else torch.from_numpy(
        (1.0 + make_weight(wl.seed, "bench/norm_g", 1, gd, 0.1)[0]).astype(np.float32)).to(dev)
    rn_need = tb.forward_rmsnorm_workspace_bytes(M, P.N, P.K)
    rn_ws = torch.empty(max(rn_need, 16), dtype=torch.uint8, device=dev)

    def fwd_rms(r):
        tb.bitlinear_forward_rmsnorm(dom["Wc"][r % copies], dom["g"], dom["X"], dom_norm_g, N=P.N,
                                     y_dtype=out, Y=dom["Y"], workspace=rn_ws, stream=stream)
    g_fr = graph_of([lambda r=r: fwd_rms(r) for r in range(copies)])
    g_fr.replay()
    t_fr = timer(g_fr.replay, reps) / (reps * copies)
    rows["forward_rmsnorm"] = {"shape": f"M{M} {P.K}->{P.N}", "us": round(t_fr * 1e6, 3),
                               "fused": rn_need == 0,
                               ("TOP/s" if prefill else "GB/s"): round(
                                   (2 * M * P.N * P.K / t_fr / 1e12) if prefill
                                   else (f32_bytes + 4 * P.K) / t_fr / 1e9, 2 if prefill else 1)}

    if grouped:
        # the same step as one call per projection, for comparison
        g_sep = graph_of([lambda r=r: step_separate(r) for r in range(cycle)])
        g_sep.replay()
        t_sep = timer(g_sep.replay, max(1, 2000 // cycle)) / (max(1, 2000 // cycle) * cycle)
        rows["step_separate_calls"] = {"us": round(t_sep * 1e6, 3),
                                       "note": "one bitlinear_forward_f32 per projection"}
        rows["step_grouped"] = {"us": round(ms_per_step * 1e3, 3),
                                "note": "one bitlinear_forward_f32_grouped"}
        gn_need = tb.forward_rmsnorm_grouped_workspace_bytes(M, Ns, projs[0]["p"].K)
        gn_ws = torch.empty(max(gn_need, 16), dtype=torch.uint8, device=dev)

        def step_grouped_rms(r):
            tb.bitlinear_forward_rmsnorm_grouped([q["Wc"][r % copies] for q in projs],
                                                 [q["g"] for q in projs], projs[0]["X"], norm_g,
                                                 Ns=Ns, y_dtype=out, Y=[q["Y"] for q in projs],
                                                 workspace=gn_ws, stream=stream)
        g_gr = graph_of([lambda r=r: step_grouped_rms(r) for r in range(cycle)])
        g_gr.replay()
        t_gr = timer(g_gr.replay, max(1, 2000 // cycle)) / (max(1, 2000 // cycle) * cycle)
        rows["step_grouped_rmsnorm"] = {"us": round(t_gr * 1e6, 3), "fused": gn_need == 0,
                                        "note": "one bitlinear_forward_rmsnorm_grouped: RMS "
                                                "normalisation, quantiser and every projection"}

    # ---------------- CPU oracle on a bounded sample of the same step
    cpu = None
    if not args.no_cpu_baseline:
        # the timed step once more, its outputs for the oracle leg to check
        with torch.cuda.stream(stream):
            step(0)
        stream.synchronize()
        y_gpu = [q["Y"].float().cpu().numpy() for q in projs]
        cpu = cpu_baseline(projs, M, args.cpu_seconds, wbytes_step, prefill, grouped, y_gpu,
                           out)

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": M,
                   "projections": [f"{q['p'].K}->{q['p'].N}" for q in projs],
                   "out": out, "weight_copies": copies, "seed": wl.seed, "graph": True},
        "roofline": roof, "cpu_baseline": cpu, "rows": rows,
        # tokens through every projection of the step (one layer) per second
        "tokens_per_s": round(M / (elapsed / args.steps), 1),
        "wall_s_timed": round(t_wall, 3),
    }
    print(json.dumps(line), flush=True)


def alg_bytes(P, M, out):
    """Algorithmic bytes of one projection launch: packed W, X~, x_scale and
    x_sum, Y, gamma."""
    return P.N * P.K // 4 + M * P.K + 8 * M + OUT_BYTES[out] * M * P.N + 4


def alg_bytes_f32(P, M, out):
    """Algorithmic bytes of one fused launch (quantiser in the prologue):
    packed W, fp32 X, Y, gamma."""
    return P.N * P.K // 4 + 4 * M * P.K + OUT_BYTES[out] * M * P.N + 4


def vendor_int8_mm(tb, torch, timer, stream, q, M):
    """The vendor's int8 GEMM (torch._int_mm, hipBLASLt underneath) on the same
    operands as the projection: X~ [M][K] and W~ unpacked to int8 [N][K] (four
    times the packed bytes), given as the transposed right operand, its faster
    layout here.  It calibrates the MFMA fraction on this chip with these
    value distributions; it is not part of the path.  Its int32 product must
    equal the projection's raw accumulators."""
    P = q["p"]
    N, K = P.N, P.K
    if not hasattr(torch, "_int_mm"):
        return {"note": "torch._int_mm not available"}
    with torch.cuda.stream(stream):
        # BLT2-v1: byte i of word g holds k = 16 g + 4 j + i at bits 2j..2j+1
        b = q["Wp"].view(N, K // 16, 1, 4).to(torch.int16)
        sh = torch.arange(0, 8, 2, device=b.device, dtype=torch.int16).view(1, 1, 4, 1)
        Wt8 = (((b >> sh) & 3) - 1).to(torch.int8).reshape(N, K).contiguous()
        del b
        acc_v = torch._int_mm(q["Xq"], Wt8.t())
    acc = tb.bitlinear_forward(q["Wp"], q["g"], q["Xq"], q["s"], q["xs"], N=N, K=K,
                               y_dtype="i32", stream=stream)
    stream.synchronize()
    same = bool(torch.equal(acc, acc_v))
    del acc, acc_v
    reps = 20
    timer(lambda: torch._int_mm(q["Xq"], Wt8.t()), 3)
    t = timer(lambda: torch._int_mm(q["Xq"], Wt8.t()), reps) / reps
    del Wt8
    torch.cuda.empty_cache()
    tops = 2 * M * N * K / t / 1e12
    return {"shape": f"M{M} {K}->{N}", "us": round(t * 1e6, 2), "TOP/s": round(tops, 1),
            "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
            "equals_forward_accumulators": same,
            "note": "torch._int_mm on W~ unpacked to int8 (4x the bytes), one weight copy: "
                    "calibration, not the path"}


def launch_alg_bytes(shapes, M, out, fused, grouped):
    """Algorithmic bytes per launch of the dominant kernel: one grouped launch
    reads the shared activations once; separate launches are averaged."""
    f = alg_bytes_f32 if fused else alg_bytes
    shared = 4 * M * shapes[0].K if fused else M * shapes[0].K + 8 * M
    if grouped:
        return sum(f(P, M, out) for P in shapes) - (len(shapes) - 1) * shared
    return sum(f(P, M, out) for P in shapes) / len(shapes)


def step_is_fused(tb, shapes, M, grouped):
    """True when every launch of the step is the fused projection (no
    separate quantiser launch): its workspace query is then 0."""
    if M > 16:
        return False
    if grouped:
        return tb.forward_f32_grouped_workspace_bytes(M, [P.N for P in shapes], shapes[0].K) == 0
    return all(tb.forward_f32_workspace_bytes(M, P.N, P.K) == 0 for P in shapes)


# Kernel names as the library reports them (bitlinear_forward_kernel), and the
# symbols they appear under in a profile.
KERNEL_SYMBOLS = {"k_decode_dot": ("k_decode_dot",), "k_decode": ("k_decode_lds", "k_decode_reg"),
                  "k_skinny": ("k_skinny",), "k_gemm": ("k_gemm",)}


def step_kernels(tb, shapes, M, grouped, fused):
    """The kernel(s) the step's projection launches run, '+'-joined when the
    projections of a step differ."""
    entry = "f32" if fused else "forward"
    if grouped:
        names = {tb.forward_kernel(entry, M, [P.N for P in shapes], shapes[0].K)[0]}
    else:
        names = {tb.forward_kernel(entry, M, [P.N], P.K)[0] for P in shapes}
    return "+".join(sorted(names))


def kernel_matches(kernels, name):
    """True when a profiled kernel name is one of `kernels` ('+'-joined)."""
    return any(sym + "<" in name for k in kernels.split("+") for sym in KERNEL_SYMBOLS[k])


def roofline(tb, torch, timer, graph_of, projs, M, out, copies, prefill, stream, grouped=False,
             fused_step=None):
    """Average launch of the dominant kernel, timed with HIP events on the
    launch stream around a graph of back-to-back launches over the rotated
    weight copies.  With fused_step (the step's own function, every launch of
    which is one fused bitlinear_forward_f32[_grouped]) that kernel is the
    step's; otherwise it is bitlinear_forward (or one bitlinear_forward_grouped
    over all projections, when they share their input) on pre-quantised
    activations."""
    fused = fused_step is not None

    def fwd_all(r):
        if fused:
            fused_step(r)
            return
        if grouped:
            tb.bitlinear_forward_grouped([q["Wc"][r % copies] for q in projs],
                                         [q["g"] for q in projs], projs[0]["Xq"], projs[0]["s"],
                                         projs[0]["xs"], Ns=[q["p"].N for q in projs],
                                         K=projs[0]["p"].K, y_dtype=out, Y=[q["Y"] for q in projs],
                                         stream=stream)
            return
        for q in projs:
            tb.bitlinear_forward(q["Wc"][r % copies], q["g"], q["Xq"], q["s"], q["xs"],
                                 N=q["p"].N, K=q["p"].K, y_dtype=out, Y=q["Y"], stream=stream)
    g = graph_of([lambda r=r: fwd_all(r) for r in range(copies)])
    g.replay()
    per_replay = 1 if grouped else len(projs)
    launches_per_replay = copies * per_replay
    # the replays in ROOF_GROUPS timed groups; the median group's mean launch
    # is reported, with the spread of the group means
    reps = max(1, (4000 if not prefill else 200) // (launches_per_replay * ROOF_GROUPS))
    per_group = sorted(timer(g.replay, reps) / (reps * launches_per_replay)
                       for _ in range(ROOF_GROUPS))
    n_launch = ROOF_GROUPS * reps * launches_per_replay
    t_launch = per_group[ROOF_GROUPS // 2]
    shapes = [q["p"] for q in projs]
    bytes_launch = launch_alg_bytes(shapes, M, out, fused, grouped)
    ops_launch = sum(2 * M * P.N * P.K for P in shapes) / (1 if grouped else len(shapes))
    if prefill:
        achieved = ops_launch / t_launch / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS,
                "unit": "TOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4)}
    else:
        achieved = bytes_launch / t_launch / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    api = ("bitlinear_forward_f32" if fused else "bitlinear_forward") + ("_grouped" if grouped else "")
    kern = step_kernels(tb, shapes, M, grouped, fused)
    roof.update({
        "traffic": load_traffic(kern, projs, M, out, fused),
        "kernel": kern, "entry_point": api,
        "shape": f"M{M} " + ", ".join(f"{P.K}->{P.N}" for P in shapes),
        "us_per_launch": round(t_launch * 1e6, 3), "launches_timed": n_launch,
        "us_per_launch_min_max": [round(per_group[0] * 1e6, 3), round(per_group[-1] * 1e6, 3)],
        "algorithmic_bytes_per_launch": int(bytes_launch),
        "ops_per_launch": int(ops_launch),
        "grouped": grouped, "fused_quantiser": fused,
        "timing": f"HIP events on the launch stream around replays of a graph of back-to-back "
                  f"{api} launches ("
                  + ("all projections in one, " if grouped else "every projection, ")
                  + f"rotated weight copies), in {ROOF_GROUPS} timed groups: the median "
                  "group's mean launch"})
    return roof, t_launch


CAL_BYTES = 256 << 20        # the calibration copy reads and writes this many bytes
ROOF_GROUPS = 9              # timed groups of the roofline's graph replays


def traffic_probe(tb, torch, projs, M, out, copies, stream, dev, wl, grouped=False,
                  fused_step=None, reps=1):
    """One elementwise copy of CAL_BYTES (torch.neg on int32: reads and writes
    CAL_BYTES), then the dominant kernel `reps` times per weight copy: the
    step's own fused launches when it has nothing else (fused_step), else
    bitlinear_forward once per projection (or bitlinear_forward_grouped once)."""
    src = torch.ones(CAL_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    with torch.cuda.stream(stream):
        if fused_step is None:
            for q in projs:
                tb.bitlinear_quant_acts(q["X"], q["Xq"], q["s"], q["xs"], stream=stream)
    torch.cuda.synchronize()

    def launch(r):
        if fused_step is not None:
            fused_step(r)
        elif grouped:
            tb.bitlinear_forward_grouped([q["Wc"][r % copies] for q in projs],
                                         [q["g"] for q in projs], projs[0]["Xq"],
                                         projs[0]["s"], projs[0]["xs"],
                                         Ns=[q["p"].N for q in projs], K=projs[0]["p"].K,
                                         y_dtype=out, Y=[q["Y"] for q in projs], stream=stream)
        else:
            for q in projs:
                tb.bitlinear_forward(q["Wc"][r % copies], q["g"], q["Xq"], q["s"], q["xs"],
                                     N=q["p"].N, K=q["p"].K, y_dtype=out, Y=q["Y"],
                                     stream=stream)
    if reps > 1:
        # back to back as the bench times them: one graph over the weight
        # copies, replayed `reps` times
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for r in range(copies):
                    launch(r)
        for _ in range(reps):
            g.replay()
    else:
        with torch.cuda.stream(stream):
            for r in range(copies):
                launch(r)
    torch.cuda.synchronize()
    shapes = [q["p"] for q in projs]
    kern = step_kernels(tb, shapes, M, grouped, fused_step is not None)
    print(json.dumps({"traffic_probe": traffic_key(kern, shapes, M, out, fused_step is not None),
                      "workload": wl.name, "calibration_bytes": CAL_BYTES,
                      "launches": copies * reps * (1 if grouped else len(projs))}), flush=True)


def _counters(d, name):
    """{dispatch id: (kernel name, value)} of one counter from a rocprofv3 csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    res = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != name:
                    continue
                k = (fn, r["Dispatch_Id"])
                kn, v = res.get(k, (r["Kernel_Name"], 0.0))
                res[k] = (kn, v + float(r["Counter_Value"]))
    return res


def traffic_from(args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the probe's launches, each
    scaled by known bytes / counter for the calibration copy, into
    profiles/traffic.json and a text summary beside it."""
    from synth import WORKLOADS
    wl = WORKLOADS[args.workload]
    M = args.tokens or wl.tokens[0]
    shapes = list(wl.projections)
    import ternary_bitlinear_amd as tb   # size queries only: no GPU
    tb.load()
    fused = step_is_fused(tb, shapes, M, wl.shared_input)
    fam = step_kernels(tb, shapes, M, wl.shared_input, fused)
    key = traffic_key(fam, shapes, M, wl.out_dtype, fused)
    out = {}
    for what, d, cname in (("fetch", args.traffic_from[0], "FETCH_SIZE"),
                           ("write", args.traffic_from[1], "WRITE_SIZE")):
        c = _counters(d, cname)
        cal = [v for kn, v in c.values() if "neg" in kn.lower()]
        ker = [v for kn, v in c.values() if kernel_matches(fam, kn)]
        # a projection with K split across workgroups is two dispatches
        red = [v for kn, v in c.values() if "k_splitk_reduce" in kn]
        if len(cal) != 1 or not ker:
            raise SystemExit(f"{d}: expected one calibration copy and >= 1 {fam} dispatch, "
                             f"found {len(cal)} and {len(ker)}")
        factor = CAL_BYTES / (cal[0] * 1024.0)
        kib = (sum(ker) + sum(red)) / len(ker)
        out[what] = {"counter": cname, "calibration_kib": cal[0], "factor": round(factor, 5),
                     "kernel_kib_per_dispatch": round(kib, 2), "dispatches": len(ker),
                     "reduce_dispatches": len(red),
                     "bytes_per_launch": kib * 1024.0 * factor}
    alg = launch_alg_bytes(shapes, M, wl.out_dtype, fused, wl.shared_input)
    total = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    ent = {"bytes_per_launch": int(total), "algorithmic_bytes_per_launch": int(alg),
           "ratio_to_algorithmic": round(total / alg, 4),
           "fetch": out["fetch"], "write": out["write"],
           "source_sha256_16": forward_source_digest(),
           "commands": [f"rocprofv3 --pmc {c} -d <dir> -o pmc --output-format csv -- "
                        f"python3 bench.py --traffic-probe --workload {wl.name} --tokens {M}"
                        for c in ("FETCH_SIZE", "WRITE_SIZE")]}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {"entries": {}}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data.setdefault("entries", {})[key] = ent
    data["note"] = ("HBM bytes per launch of the dominant kernel (bitlinear_forward's, or the "
                    "fused bitlinear_forward_f32's where the key says f32-fused): rocprofv3 "
                    "FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by CAL_BYTES / "
                    "the same counter on one torch.neg copy of CAL_BYTES int32 bytes in the "
                    "same run.")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({key: ent}))


def traffic_key(kernel, shapes, M, out, fused=False):
    """shapes: the workload's projections (objects with K and N)."""
    return (f"{kernel}{' f32-fused' if fused else ''} M{M} "
            + ",".join(f"{P.K}->{P.N}" for P in shapes) + f" {out}")


def forward_source_digest():
    """Digest of the sources the projection kernels are compiled from."""
    import hashlib
    h = hashlib.sha256()
    for name in ("forward.hip", "common.hpp"):
        h.update(open(os.path.join(ROOT, "ternary_bitlinear_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel, projs, M, out, fused=False):
    """HBM bytes per launch (read + written) from profiles/traffic.json, when the
    counters there were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get("entries", {}).get(traffic_key(kernel, [q["p"] for q in projs], M, out, fused))
    if not ent or ent.get("source_sha256_16") != forward_source_digest():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(projs, M, seconds, wbytes_step, prefill, grouped, y_gpu, out):
    """The oracle's per-step work (quantise, integer product, rescale) for every
    projection, repeated on the host for about `seconds`; its last step's
    outputs are compared element by element with the GPU step's (y_gpu):
    |y - y_oracle| <= tol |y_oracle| (1e-5 fp32, 1e-2 bf16), and exactly 0
    where the accumulator is 0."""
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
        # a grouped step feeds every projection the first one's activations
        X = projs[0]["X_host"] if grouped else q["X_host"]
        prep.append((O.ternarize(q["W_host"], gamma), gamma, X))

    def one_step():
        ys = []
        for Wt, gamma, X in prep:
            Xq, _, _, beta = O.quantize_activations(X)
            ys.append(O.rescale(O.integer_matmul(Wt, Xq), gamma, beta))
        return ys
    n = 0
    t0 = time.perf_counter()
    while True:
        ys = one_step()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or (n >= 1 and el * (n + 1) / n > 3 * seconds):
            break
    per = el / n
    macs = sum(M * q["p"].N * q["p"].K for q in projs)
    if prefill:
        v, unit = 2 * macs / per / 1e12, "TOP/s"
    else:
        v, unit = wbytes_step / per / 1e9, "GB/s"
    # the same step on one thread (decode shapes only: a prefill step takes
    # tens of seconds there), for about a third of the time
    single = None
    if not prefill:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                n1, t1 = 0, time.perf_counter()
                while True:
                    one_step()
                    n1 += 1
                    e1 = time.perf_counter() - t1
                    if e1 >= seconds / 3:
                        break
            single = {"value": round(wbytes_step / (e1 / n1) / 1e9, 6), "unit": "GB/s",
                      "ms_per_step": round(e1 / n1 * 1e3, 3), "sample": f"{n1} steps ({e1:.1f} s)"}
        except Exception:  # pragma: no cover
            single = None
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    tol = {"f32": 1e-5, "bf16": 1e-2}[out]
    bad = 0
    for y, yg in zip(ys, y_gpu):
        zero = y == 0
        bad += int((yg[zero] != 0).sum())
        bad += int((np.abs(yg - y) > tol * np.abs(y))[~zero].sum())
    return {"value": round(v, 6), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{n} full steps of the same workload ({el:.1f} s)",
            "ms_per_step": round(per * 1e3, 3),
            "gmac_per_s": round(macs / per / 1e9, 3),
            "cpu_model": cpu_model, "nproc": os.cpu_count(),
            "single_core": single,
            "timed_outputs_checked": int(sum(y.size for y in ys)),
            "timed_outputs_mismatched": bad,
            "timed_outputs_tolerance": f"{tol:g} relative ({out}); exact 0 for a zero accumulator"}


if __name__ == "__main__":
    main()
