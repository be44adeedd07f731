"""Timeline of the single-token chain (router -> gate/up -> down) at decode40.

Loads the timestamp build (libmoe_stamps.so; csrc/stamps.hpp), captures the
40-layer decode40 step as the bench does (one HIP graph, same layers, same
inputs), replays it, and prints in Markdown when each phase of the last layer
happened, relative to the first router workgroup's start: per kernel the
earliest, median and latest workgroup; for gate/up also per slot (the slot-s
workgroups run s+1 top-k rounds); and the gaps between kernels. The stamps
that wait for loads change wave 0's schedule, so the chain under this build
is somewhat slower than the plain library's; its event time is printed too.

With --gemm WORKLOAD... it instead runs each workload's layer eagerly and
prints how the grouped GEMM's waves spend their shader-clock cycles (DMA
wait, barrier, issue + compute, pass set-up, ...), summed over every wave of
the timed launches, for the gate/up and the down kernel.

Build on any host with hipcc, then run from the repository root on one GPU:
    python -m routed_expert_quantized_amd.build --stamps
    python -m routed_expert_quantized_amd.timeline [--replays N]
    python -m routed_expert_quantized_amd.timeline --gemm prefill8k prefill batched_int4
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COLS = 1024  # kStampCols


# k_gemm_dma's phase sums (g_stamps_gemm columns)
GEMM_PHASES = {"dma_wait": 0, "barrier": 1, "issue_compute": 2, "total": 3, "waves": 4, "pass_setup": 5,
               "prologue": 6, "trailing_wait": 7, "epilogue": 8}


def gemm_split(names, runs, rq, bench, synth, torch, L) -> None:
    L.moe_stamps_read_gemm.argtypes = [ctypes.c_void_p]
    print("# Grouped GEMM: where the waves' cycles go\n")
    print("Command (from the repository root, on one MI355X):\n")
    print("```\npython -m routed_expert_quantized_amd.build --stamps\n"
          f"python -m routed_expert_quantized_amd.timeline --gemm {' '.join(names)} --runs {runs}\n```\n")
    print(f"Timestamp build. Per workload: two layers, four warm-up calls, then {runs} calls of the layer whose "
          "waves' shader-clock cycles are summed by phase over every wave of the gate/up and down launches "
          "(fractions of the summed wave time). 'other' is the rest: tile set-up, the grid-stride loop and the "
          "kernel's start and end.\n")
    print("| workload | kernel | waves per launch | DMA wait | trailing wait | barrier | issue + compute | "
          "pass set-up | prologue | epilogue | other |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for name in names:
        w = synth.WORKLOADS[name]
        pools, routers = bench.build_layers(w, 2, 0, rq, synth, torch)
        xs = [bench.to_dev(synth.draw_step_x(w, 0, s), w.xtype, torch) for s in range(2)]
        ws = rq.Workspace()
        ws.get(rq.moe_workspace_bytes(w.T, w.E, w.H, w.I, w.k, w.scheme))
        y = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")

        def run(n):
            for i in range(n):
                rq.moe_layer_forward(xs[i % 2], routers[i % 2], pools[i % 2], w.k, rq.MOE_FLAG_RENORM, ws=ws,
                                     out=y, return_routing=False)

        run(4)
        torch.cuda.synchronize()
        if L.moe_stamps_zero_gemm() != 0:
            raise SystemExit("clearing the GEMM stamps failed")
        run(runs)
        torch.cuda.synchronize()
        g = np.zeros((2, 16), np.uint64)
        if L.moe_stamps_read_gemm(g.ctypes.data) != 0:
            raise SystemExit("reading the GEMM stamps failed")
        for mode, kname in ((0, "gate/up"), (1, "down")):
            v = {k: int(g[mode][i]) for k, i in GEMM_PHASES.items()}
            tot = max(v["total"], 1)
            parts = [v[k] for k in ("dma_wait", "trailing_wait", "barrier", "issue_compute", "pass_setup",
                                    "prologue", "epilogue")]
            other = tot - sum(parts)
            cells = " | ".join(f"{100.0 * p / tot:.1f}%" for p in parts + [other])
            print(f"| {name} | {kname} | {v['waves'] // runs} | {cells} |")
        del pools, routers, ws
        torch.cuda.empty_cache()


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--replays", type=int, default=8)
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--gemm", nargs="+", default=None, metavar="WORKLOAD")
    ap.add_argument("--runs", type=int, default=8)
    args = ap.parse_args()
    sys.path.insert(0, ROOT)
    import torch

    import routed_expert_quantized_amd as rq
    rq.LIB_PATH = os.path.join(PKG, "libmoe_stamps.so")
    if not os.path.exists(rq.LIB_PATH):
        raise SystemExit(f"{rq.LIB_PATH} is missing: python -m routed_expert_quantized_amd.build --stamps")
    import bench
    import synth
    L = rq.lib()
    if args.gemm:
        for name in args.gemm:
            if name not in synth.WORKLOADS or synth.WORKLOADS[name].T == 1:
                raise SystemExit(f"--gemm takes workloads with more than one token, not {name}")
        gemm_split(args.gemm, args.runs, rq, bench, synth, torch, L)
        return
    for fn in (L.moe_stamps_read_route, L.moe_stamps_read_decode):
        fn.argtypes = [ctypes.c_void_p]
        fn.restype = ctypes.c_int
    L.moe_stamps_clock_khz.restype = ctypes.c_int

    w = synth.WORKLOADS["decode40"]
    NL = args.layers
    pools, routers = bench.build_layers(w, NL, 0, rq, synth, torch)
    xs = [bench.to_dev(synth.draw_step_x(w, 0, s), w.xtype, torch) for s in range(16)]
    xbuf = torch.empty_like(xs[0])
    ys = [torch.empty((1, w.H), dtype=torch.float32, device="cuda") for _ in range(NL)]
    ws = rq.Workspace()
    ws.get(rq.moe_workspace_bytes(1, w.E, w.H, w.I, w.k, w.scheme))

    def run():
        for l in range(NL):
            rq.moe_layer_forward(xbuf, routers[l], pools[l], w.k, rq.MOE_FLAG_RENORM, ws=ws, out=ys[l],
                                 return_routing=False)

    xbuf.copy_(xs[0])
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    khz = L.moe_stamps_clock_khz()
    if khz <= 0:
        raise SystemExit("could not read the stamps' clock rate")
    us_per_tick = 1000.0 / khz

    r = np.zeros((2, COLS), np.uint64)
    d = np.zeros((8, COLS), np.uint64)
    runs = []
    for rep in range(args.replays + 2):
        xbuf.copy_(xs[rep % len(xs)])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        if L.moe_stamps_read_route(r.ctypes.data) != 0 or L.moe_stamps_read_decode(d.ctypes.data) != 0:
            raise SystemExit("reading the stamps failed")
        if rep >= 2:
            runs.append((e0.elapsed_time(e1) * 1000.0 / NL, r.copy(), d.copy()))

    # the last layer's stamps: every workgroup of each grid writes its entry
    nr = int(np.count_nonzero(runs[0][1][0]))
    ngu = int(np.count_nonzero(runs[0][2][0]))
    ndn = int(np.count_nonzero(runs[0][2][4]))
    bps = ngu // w.k
    phases = {}

    def put(name, vals):
        phases.setdefault(name, []).append(vals)

    for _, rr, dd in runs:
        base = int(rr[0, :nr].min())
        f = lambda a: (a.astype(np.int64) - base) * us_per_tick
        R = [f(rr[i, :nr]) for i in range(2)]
        G = [f(dd[i, :ngu]) for i in range(4)]
        D = [f(dd[4 + i, :ndn]) for i in range(4)]
        for name, a in (("router: start", R[0]), ("router: end", R[1]),
                        ("gate/up: start", G[0]), ("gate/up: routing known", G[1]),
                        ("gate/up: weight loads landed", G[2]), ("gate/up: end", G[3]),
                        ("down: start", D[0]), ("down: routing read", D[1]),
                        ("down: weight loads landed", D[2]), ("down: end", D[3])):
            put(name, (a.min(), float(np.median(a)), a.max()))
        for s in range(w.k):
            sl = slice(s * bps, (s + 1) * bps)
            put(f"slot {s}", (float(np.median(G[1][sl])), float(np.median(G[2][sl])), G[3][sl].max()))
        put("gaps", (G[0].min() - R[1].max(), D[0].min() - G[3].max(), D[3].max()))

    med = lambda name, i: statistics.median(v[i] for v in phases[name])
    ev = statistics.median(t for t, _, _ in runs)
    print(f"# Single-token chain timeline: decode40 (T=1, H={w.H}, E={w.E}, top-{w.k}, I={w.I}, sym8, x fp16)\n")
    print("Command (from the repository root, on one MI355X):\n")
    print("```\npython -m routed_expert_quantized_amd.build --stamps\n"
          f"python -m routed_expert_quantized_amd.timeline --replays {args.replays} --layers {NL}\n```\n")
    print(f"Timestamp build, {NL}-layer graph, {len(runs)} replays; the last layer of each replay, medians over "
          f"replays. Counter {khz} kHz. Event time of this build: {ev:.2f} us per layer. Workgroups: router {nr}, "
          f"gate/up {ngu} ({bps} per slot; the routing publisher is not stamped), down {ndn}.\n")
    print("| phase (us from the first router start) | earliest workgroup | median | latest |")
    print("|---|---|---|---|")
    for name in ("router: start", "router: end", "gate/up: start", "gate/up: routing known",
                 "gate/up: weight loads landed", "gate/up: end", "down: start", "down: routing read",
                 "down: weight loads landed", "down: end"):
        print(f"| {name} | {med(name, 0):.2f} | {med(name, 1):.2f} | {med(name, 2):.2f} |")
    print("\n| gate/up slot | routing known (median) | loads landed (median) | end (latest) |")
    print("|---|---|---|---|")
    for s in range(w.k):
        print(f"| {s} | {med(f'slot {s}', 0):.2f} | {med(f'slot {s}', 1):.2f} | {med(f'slot {s}', 2):.2f} |")
    print(f"\nGaps: router end -> gate/up start {med('gaps', 0):.2f} us, gate/up end -> down start "
          f"{med('gaps', 1):.2f} us; the layer's span {med('gaps', 2):.2f} us.")


if __name__ == "__main__":
    main()
