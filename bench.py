#!/usr/bin/env python3
"""Benchmark of the routed, block-quantized MoE expert layer on one MI355X.

Default workload (decode40): single-token decode through 40 stacked MoE
layers, H=2048, E=256, top-8, I=512, sym8 experts with fp16 block scales, x
fp16, fresh activations on each of 512 steps. A step is one token through
all 40 layers: per layer, router, gathered gate/up + SwiGLU, per-slot down and
gate-weighted combine. Each step is a captured HIP graph. Inputs and all
40 layers' weights (34 GB) are resident in HBM before timing starts.

Prints one JSON line: the contract fields, plus the dominant kernel's
roofline (live HIP-event durations) and the CPU oracle's rate on a bounded
sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode40]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE-layer decode tokens/s + achieved HBM GB/s on routed bytes (1 MI355X)"


# sources that define each path's dominant kernel; a stored counter reading is
# used only while these files are unchanged
KERNEL_SOURCES = {"gather": ("k_decode.hip", "common.hpp"),
                  "gemm": ("k_gemm.hip", "common.hpp")}


def kernel_source_sha(path: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[path]:
        with open(os.path.join(ROOT, "routed_expert_quantized_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode40")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copies", type=int, default=8, help="layer copies cycled for single-layer workloads")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--timer-steps", type=int, default=16, help="steps of the per-kernel event timing pass")
    ap.add_argument("--k", type=int, default=None,
                    help="override the workload's top-k (for the bytes-read-versus-k counter sweep)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run a plain fp32 copy kernel over this many MiB (counter calibration)")
    ap.add_argument("--no-prerouter", action="store_true", help="skip the prerouted (prediction-as-routing) step")
    ap.add_argument("--no-lora", action="store_true", help="skip the quantized linear with a LoRA delta")
    ap.add_argument("--path", choices=["auto", "gather", "gemm"], default="auto",
                    help="expert path: the library's choice, the gathered matvec or the grouped MFMA GEMM")
    ap.add_argument("--secondary", default=",".join(SECONDARY),
                    help="after decode40, these workloads are measured too and reported under 'workloads' "
                         "(comma-separated, or 'none')")
    return ap.parse_args()


def expert_bytes(w) -> int:
    per_block = 32 if w.scheme == 0 else 16
    return 3 * w.H * w.I // 32 * (per_block + 2)


def gate_up_bytes(w) -> int:
    per_block = 32 if w.scheme == 0 else 16
    return 2 * w.I * w.H // 32 * (per_block + 2)


def dtype_name(w, gemm: bool) -> str:
    """The arithmetic each stage of the timed path runs in."""
    if gemm:
        xt = "bf16" if w.xtype == 2 else "f16"
        return (f"gate/up {xt} x raw codes on the matrix cores, f32 per-block scale; h f16 (tile exponent); "
                f"down f16 x raw codes, f32; f32 router, combine")
    if w.T > 1:
        return "f32 (grouped matvec)"
    gu = "f16xf16->f32 (v_dot2)" if w.xtype == 1 else "f32"
    down = "f16xf16->f32 (v_dot2, fp16 h)" if w.I <= 1024 else "f32"
    return f"gate/up {gu}; down {down}; f32 router, combine"


def miss_policies(w, xs, router, pool, rq, torch) -> dict:
    """Expert-cache miss policies replayed (moe_miss_replay) over the routing of
    the workload's distinct tokens, in order, through one layer's router: a
    quarter of the experts resident, as on the pages. Fetched bytes count the
    synchronous fetches and background admissions at the expert's packed size.
    Also times moe_stage_experts filling a stack of that many slots from the
    pool (HBM to HBM; the pages fetch from SSD or host memory instead)."""
    import numpy as np
    idx, gate = [], []
    for x in xs:
        i, g = rq.moe_route(x, router, w.k, rq.MOE_FLAG_RENORM)
        idx.append(i.cpu().numpy())
        gate.append(g.cpu().numpy())
    idx, gate = np.concatenate(idx), np.concatenate(gate)
    C = max(w.k, w.E // 4)
    out = {"tokens": int(idx.shape[0]), "capacity": C, "expert_bytes": expert_bytes(w)}
    for name, pol, beta in (("fetch_all", rq.MOE_MISS_FETCH_ALL, 0.0), ("quality_first", rq.MOE_MISS_RULE, 0.5),
                            ("speed_first", rq.MOE_MISS_FIRST_CHOICE, 0.5)):
        t0 = time.perf_counter()
        m, sync, bg, _ = rq.moe_miss_replay(idx, gate, w.E, C, pol, 0.15, beta)
        dt = time.perf_counter() - t0
        fetched = float(np.mean(sync + bg))
        out[name] = {"mean_m": round(float(np.mean(m)), 5), "max_m": round(float(np.max(m)), 5),
                     "sync_fetches_per_token": round(float(np.mean(sync)), 4),
                     "bg_fetches_per_token": round(float(np.mean(bg)), 4),
                     "fetched_bytes_per_token": int(round(fetched * expert_bytes(w))),
                     "replay_us_per_token": round(dt * 1e6 / idx.shape[0], 3)}
    out["fetch_all_hit_rate"] = round(1.0 - out["fetch_all"]["sync_fetches_per_token"] / w.k, 4)
    stack = rq.empty_stack(pool, C)
    experts = torch.randperm(w.E, device="cuda")[:C].to(torch.int32)
    slots = torch.arange(C, device="cuda", dtype=torch.int32)
    rq.moe_stage_experts(pool, stack, experts, slots)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(8):
        rq.moe_stage_experts(pool, stack, experts, slots)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 8
    nbytes = C * expert_bytes(w)
    out["stage_all_slots"] = {"bytes": nbytes, "us": round(us, 2),
                              "gbps_copied": round(nbytes / (us * 1e-6) / 1e9, 1)}
    del stack
    return out


def flag_step(w, xs, nl, pools, routers, ws, K, W, flags, rq, torch) -> dict:
    """The headline's layers with other flags (the single-token path with fp32
    h): the same pools, routers and inputs, one HIP graph of the nl layers."""
    xbuf = torch.empty_like(xs[0])
    ys = [torch.empty((w.T, w.H), dtype=torch.float32, device="cuda") for _ in range(nl)]
    nx = xs.shape[0]

    def run():
        for l in range(nl):
            rq.moe_layer_forward(xbuf, routers[l], pools[l], w.k, rq.MOE_FLAG_RENORM | flags, ws=ws, out=ys[l],
                                 return_routing=False)

    xbuf.copy_(xs[0])
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for s in range(W):
        xbuf.copy_(xs[s % nx])
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(K):
        xbuf.copy_(xs[(W + s) % nx])
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (K * nl)
    del g
    return {"us_per_layer": round(us, 3), "flags": int(flags), "layers": nl, "steps": K}


def staged_step(w, xs, nl, pools, routers, ws, K, W, path_flag, rq, torch) -> dict:
    """The layer on resident stacks behind slot tables (moe_layer_forward_staged):
    every layer's E experts copied into a stack in a random slot order, so the
    routing, the bytes and the outputs are the pool layer's and the difference
    is the slot-table lookup. Timed as one HIP graph of the nl layers."""
    stacks, tables = [], []
    for l in range(nl):
        st = rq.empty_stack(pools[l], w.E)
        experts = torch.arange(w.E, dtype=torch.int32, device="cuda")
        slots = torch.randperm(w.E, device="cuda").to(torch.int32)
        rq.moe_stage_experts(pools[l], st, experts, slots)
        slot_of = torch.empty(w.E, dtype=torch.int32, device="cuda")
        slot_of[experts.long()] = slots
        stacks.append(st)
        tables.append(slot_of)
    xbuf = torch.empty_like(xs[0])
    ys = [torch.empty((w.T, w.H), dtype=torch.float32, device="cuda") for _ in range(nl)]
    nx = xs.shape[0]

    def run():
        for l in range(nl):
            rq.moe_layer_forward_staged(xbuf, routers[l], stacks[l], tables[l], w.k, rq.MOE_FLAG_RENORM | path_flag,
                                        ws=ws, out=ys[l], return_routing=False)

    xbuf.copy_(xs[0])
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for s in range(W):
        xbuf.copy_(xs[s % nx])
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(K):
        xbuf.copy_(xs[(W + s) % nx])
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (K * nl)
    del g, stacks, tables
    torch.cuda.empty_cache()
    return {"us_per_layer": round(us, 3), "slots": w.E, "layers": nl, "steps": K}


def prerouted_step(w, xs, nl, pools, routers, ws, seed, K, W, path_flag, rq, synth, torch) -> dict:
    """Prediction as routing: layer 0 runs its router; every later layer runs its
    experts (moe_experts_from_logits) on the logits that the previous layer's
    prerouter head predicted one token earlier. Each layer but the last then runs
    its head (moe_prerouter_forward, logits only) on the layer input and its own
    routing at this token and the previous one. No other router runs. Heads are
    seeded random weights (F = synth.PREROUTER_F). Timed twice, each as HIP
    graphs (one per parity of the step, for the double-buffered routing): with
    separate expert and head calls, then with moe_prerouted_layer_forward, which
    runs the head's rows inside the expert launches for one token."""
    import numpy as np
    F, T, k = synth.PREROUTER_F, w.T, w.k
    heads = []
    for l in range(nl - 1):
        d = synth.draw_prerouter(seed, w.wid, l, w.H, w.E, F, w.router_std)
        # fc1 and the residual path in one allocation, the residual rows right
        # after fc1's, so a batch runs their products as one launch
        D = w.H + 2 * w.E
        w1l = torch.from_numpy(np.concatenate([d["w1"].ravel(), d["wl"].ravel()])).cuda()
        heads.append(rq.Prerouter(w1l[:F * D].view(F, D), torch.from_numpy(d["b1"]).cuda(),
                                  torch.from_numpy(d["w2"]).cuda(), torch.from_numpy(d["b2"]).cuda(),
                                  w1l[F * D:].view(w.E, D)))
    # per layer, two generations of the predicted logits and of the routing taken
    lgs = [[torch.empty((T, w.E), dtype=torch.float32, device="cuda") for _ in range(2)] for _ in range(nl)]
    idxs = [[torch.empty((T, k), dtype=torch.int32, device="cuda") for _ in range(2)] for _ in range(nl)]
    gates = [torch.empty((T, k), dtype=torch.float32, device="cuda") for _ in range(nl)]
    hws = rq.Workspace()
    hws.get(rq.moe_prerouter_workspace_bytes(T, w.E, F))
    xbuf = torch.empty_like(xs[0])
    xbuf.copy_(xs[0])
    for l in range(nl):  # starting predictions: the router's logits, via a warm-start head
        for g in range(2):
            i, _ = rq.moe_route(xs[0], routers[l], k, rq.MOE_FLAG_RENORM)
            idxs[l][g].copy_(i)
    for l in range(1, nl):
        D = w.H + 2 * w.E
        wl = torch.zeros((w.E, D), dtype=torch.float32, device="cuda")
        wl[:, :w.H] = routers[l]
        warm = rq.Prerouter(torch.zeros((F, D), dtype=torch.float32, device="cuda"), None,
                            torch.zeros((w.E, F), dtype=torch.float32, device="cuda"), None, wl)
        for g in range(2):
            rq.moe_prerouter_forward(xs[0], warm, None, None, k, ws=hws, logits_out=lgs[l][g], topk=False)
    torch.cuda.synchronize()
    ys = [torch.empty((T, w.H), dtype=torch.float32, device="cuda") for _ in range(nl)]
    def run(gen, fused):
        cur, other = gen % 2, 1 - gen % 2
        for l in range(nl):
            if l == 0:
                rq.moe_layer_forward(xbuf, routers[0], pools[0], k, rq.MOE_FLAG_RENORM | path_flag, ws=ws,
                                     out=ys[0], routing_out=(idxs[0][cur], gates[0]))
            elif fused:
                # experts on the predicted logits and the next layer's head, together
                head = heads[l] if l + 1 < nl else None
                rq.moe_prerouted_layer_forward(xbuf, lgs[l][cur], pools[l], k, head, idxs[l][other], idxs[l][cur],
                                               lgs[l + 1][other] if head is not None else None,
                                               flags=rq.MOE_FLAG_RENORM | path_flag, gate_out=gates[l], ws=ws,
                                               out=ys[l])
                continue
            else:
                rq.moe_experts_from_logits(xbuf, lgs[l][cur], pools[l], k, rq.MOE_FLAG_RENORM | path_flag, ws=ws,
                                           out=ys[l], routing_out=(idxs[l][cur], gates[l]))
            if l + 1 < nl:
                rq.moe_prerouter_forward(xbuf, heads[l], idxs[l][cur], idxs[l][other], k, ws=hws,
                                         logits_out=lgs[l + 1][other], topk=False)

    for gen in range(2):
        run(gen, False)
        run(gen, True)
    torch.cuda.synchronize()
    nx = xs.shape[0]
    out = {}
    for fused in (False, True):
        graphs = []
        for gen in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run(gen, fused)
            graphs.append(g)
        torch.cuda.synchronize()

        def step(s):
            xbuf.copy_(xs[s % nx])
            graphs[s % 2].replay()

        for s in range(W):
            step(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(K):
            step(W + s)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        out["fused" if fused else "separate_calls"] = {"us_per_layer": round(ms * 1e3 / (K * nl), 3),
                                                       "step_tokens_per_s": round(T / (ms * 1e-3 / K), 1)}
        del graphs
    # experts the predicted routing touches per layer (the head is random, so it
    # lacks the workload's popularity and reuse structure)
    uniq = [len(torch.unique(idxs[l][0])) for l in range(1, nl)]
    out["unique_experts_per_layer"] = round(float(np.mean(uniq)), 2)
    # head kernels alone, per launch (eager): stage 1 (fc1 + GELU, residual
    # path), stage 2 (fc2); the top-k runs inside the next layer's expert call
    with rq.KernelTimer(rq.MOE_KERNEL_HEAD, 2 * (nl - 1) * 4 + 8) as t:
        for s in range(4):
            xbuf.copy_(xs[s % nx])
            run(s, False)
    torch.cuda.synchronize()
    s1_us = float(np.mean(t.ms[0::2])) * 1e3
    s2_us = float(np.mean(t.ms[1::2])) * 1e3
    xb = T * w.H * (4 if w.xtype == 0 else 2)
    H, E = w.H, w.E
    # algorithmic bytes: stage 1 reads the hidden columns of fc1 and of the
    # residual path, 2k routed entries per row, biases, x and the routing ids,
    # and writes fc1's outputs and the partial logits; stage 2 reads fc2,
    # fc1's outputs and the partials and writes the logits
    ids = 4 * T * 2 * k
    s1_bytes = 4 * ((F + E) * H + 2 * k * (F + E) + F + E) + xb + ids + 4 * T * (F + E)
    s2_bytes = 4 * (E * F + T * F + 2 * T * E)
    s1 = "stage1_fc1_residual" if T < 16 else "stage1_epilogue"  # from 16 tokens the products run on the router's MFMA kernel
    res = {"F": F, "layers": nl, "heads": nl - 1, "steps": K, **out,
           "head_kernel_us": {s1: round(s1_us, 3), "stage2_fc2": round(s2_us, 3)},
           "head_bytes": {"stage2_fc2": s2_bytes},
           "head_gbps": {"stage2_fc2": round(s2_bytes / (s2_us * 1e-6) / 1e9, 1)}}
    if T < 16:
        res["head_bytes"][s1] = s1_bytes
        res["head_gbps"][s1] = round(s1_bytes / (s1_us * 1e-6) / 1e9, 1)
    return res


def lora_linear(w, seed, rq, synth, torch) -> dict:
    """Unmerged LoRA delta on a block-quantized projection (moe_qlinear_lora_forward):
    an H x H matrix in the workload's codec at the workload's T, rank 16, scale
    alpha / r = 2. Calls chain over enough distinct weight copies to exceed the
    256 MB MALL, captured in a HIP graph; timed with the delta and without it."""
    import numpy as np
    T, N, K, r = w.T, w.H, w.H, 16
    g = synth.rng(seed, w.wid, 0, 0, 3000)
    W = torch.from_numpy((g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32)).cuda()
    codes, scales = rq.moe_quantize(W, w.scheme)
    del W
    wbytes = codes.numel() + scales.numel() * 2
    copies = max(8, -(-(512 << 20) // wbytes))
    qws = [rq.QWeight(N, K, w.scheme, codes.clone(), scales.clone()) for _ in range(copies)]
    A = torch.from_numpy((g.standard_normal((r, K), dtype=np.float32) / np.float32(np.sqrt(K))).astype(np.float32)).cuda()
    B = torch.from_numpy((g.standard_normal((N, r), dtype=np.float32) * np.float32(0.05)).astype(np.float32)).cuda()
    x = to_dev(synth.encode_x(synth.draw_x(g, T, K), w.xtype), w.xtype, torch)
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    ws = rq.Workspace()
    ws.get(rq.lib().moe_qlinear_lora_workspace_bytes(T, r))
    out = {"N": N, "K": K, "r": r, "T": T, "copies": copies, "weight_bytes": wbytes}
    for name, a, b in (("base", None, None), ("with_lora", A, B)):
        def run():
            for q in qws:
                rq.moe_qlinear_lora_forward(x, q, a, b, 2.0, ws=ws, out=y)
        run()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            run()
        gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 8
        e0.record()
        for _ in range(reps):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
        nbytes = wbytes + T * K * (4 if w.xtype == 0 else 2) + T * N * 4 + (4 * (r * K + N * r + 2 * T * r) if a is not None else 0)
        out[name] = {"us_per_call": round(us, 3), "bytes": nbytes, "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del gr
    with rq.KernelTimer(rq.MOE_KERNEL_LORA, 2 * 16 + 4) as t:
        for q in qws[:16]:
            rq.moe_qlinear_lora_forward(x, q, A, B, 2.0, ws=ws, out=y)
    torch.cuda.synchronize()
    out["kernel_us"] = {"lora_a": round(float(np.mean(t.ms[0::2])) * 1e3, 3),
                        "qlinear_lora": round(float(np.mean(t.ms[1::2])) * 1e3, 3)}
    out["lora_overhead"] = round(out["with_lora"]["us_per_call"] / out["base"]["us_per_call"] - 1.0, 4)
    del qws
    return out


def stream_ceiling(nbytes: int, rq, torch) -> dict:
    """A plain streaming read of one layer's routed bytes (moe_stream_read), as
    back-to-back launches in a HIP graph over distinct buffers that together far
    exceed the 256 MB MALL: the bandwidth a kernel moving that many bytes can
    reach on this GPU, next to the HBM peak."""
    nb = (nbytes + 15) // 16 * 16
    nbuf = max(2, min(64, -(-(2 << 30) // nb)))
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    reps = max(2, 256 // nbuf)

    def run():
        for b in bufs:
            rq.moe_stream_read(b, nb)

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * nbuf)
    del g, bufs
    gbps = nb / (us * 1e-6) / 1e9
    return {"bytes": nb, "us_per_read": round(us, 3), "gbps": round(gbps, 1),
            "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4), "buffers": nbuf}


def build_layers(w, nl, seed, rq, synth, torch):
    """nl layers of device experts (quantised on the device) and host-drawn routers."""
    pools, routers = [], []
    for l in range(nl):
        E, H, I = w.E, w.H, w.I
        cbh = H if w.scheme == 0 else H // 2
        cbi = I if w.scheme == 0 else I // 2
        wgu = torch.empty((E, 2 * I, cbh), dtype=torch.uint8, device="cuda")
        sgu = torch.empty((E, 2 * I, H // 32), dtype=torch.int16, device="cuda")
        wd = torch.empty((E, H, cbi), dtype=torch.uint8, device="cuda")
        sd = torch.empty((E, H, I // 32), dtype=torch.int16, device="cuda")
        chunk = max(1, (256 << 20) // (3 * H * I * 4))
        for e0, a, b in synth.torch_expert_chunks(w, seed, l, chunk, "cuda"):
            c = a.shape[0]
            ca, sa = rq.moe_quantize(a, w.scheme)
            cb, sb = rq.moe_quantize(b, w.scheme)
            wgu[e0:e0 + c], sgu[e0:e0 + c], wd[e0:e0 + c], sd[e0:e0 + c] = ca, sa, cb, sb
            del a, b, ca, sa, cb, sb
        pools.append(rq.Experts(E, H, I, w.scheme, wgu, sgu, wd, sd))
        li = synth.draw_layer(w, seed=seed, layer=l, T=1, with_experts=False)
        routers.append(torch.from_numpy(li.R).cuda())
        if (l + 1) % 10 == 0:
            log(f"  built {l + 1}/{nl} layers")
    torch.cuda.synchronize()
    return pools, routers


def to_dev(x, xtype, torch):
    import numpy as np
    if xtype == 2:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def cpu_baseline(w, seed, seconds, threads=None):
    """The oracle, timed on this host on a bounded sample: one token per layer
    for successive layers of the same workload (router + gathered experts).
    Expert draws and quantisation happen before the clock starts. `threads`
    sets the oracle's OpenMP threads for this measurement (None: all)."""
    import numpy as np
    import oracle
    import synth
    n_sample = min(w.layers, 8) if w.T == 1 else 2
    t_sample = min(w.T, 16)
    samples = []
    for l in range(n_sample):
        li = synth.draw_layer(w, seed=seed, layer=l, T=1, with_experts=False)
        x = np.ascontiguousarray(synth.draw_step_x(w, seed, l)[:t_sample])
        idx, _ = oracle.route(x, li.R, w.k, bf16=w.xtype == synth.BF16)
        used = np.unique(idx)
        wgu, wd = synth.draw_experts(seed, w.wid, l, used, w.H, w.I, w.weight_std)
        samples.append((x, li.R, oracle.quantize_experts(wgu, wd, w.scheme), {int(e): i for i, e in enumerate(used)}))
    all_threads = oracle.num_threads()
    if threads is not None:
        oracle.set_num_threads(threads)
    try:
        used_threads = oracle.num_threads()
        t0 = time.perf_counter()
        n_tok = 0
        n_layers = 0
        while True:
            for x, R, ex, m in samples:
                idx, gate = oracle.route(x, R, w.k, bf16=w.xtype == synth.BF16)
                cidx = np.vectorize(lambda e: m[int(e)])(idx).astype(np.int32)
                oracle.gather_forward(x, ex, cidx, gate, bf16=w.xtype == synth.BF16)
                n_tok += x.shape[0]
                n_layers += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(all_threads)
    return {"value": n_tok / dt, "unit": "tokens/s (per layer)", "cores": used_threads, "kind": "oracle",
            "sample": f"{len(samples)} layers x {t_sample} token(s) of {w.name}, {n_layers} layer calls in {dt:.1f} s "
                      f"(fp64 oracle: router + gathered experts; weight draws and quantisation untimed)"}


def host_info() -> dict:
    """The host the CPU baseline ran on: logical CPUs, the ones this process may
    use, and the CPU model."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def dense_over_read(w, seed, seconds) -> dict:
    """The oracle's gathered forward (only the k routed experts) against its dense
    form (all E experts evaluated, non-routed gates zero) on one token of one
    layer: the host-side cost of reading every expert instead of the routed
    ones. Codes are random bytes and scales a constant: the timing does not
    depend on the values, and drawing and quantising every expert of a large
    layer would take longer than the measurement."""
    import numpy as np
    import oracle
    import synth
    g = np.random.default_rng(seed)
    cb = 1 if w.scheme == synth.SYM8 else 2
    E, H, I = w.E, w.H, w.I
    ex = oracle.Experts(E, H, I, w.scheme, g.integers(0, 256, (E, 2 * I, H // cb), dtype=np.uint8),
                        np.full((E, 2 * I, H // 32), 0x2000, dtype=np.uint16),
                        g.integers(0, 256, (E, H, I // cb), dtype=np.uint8),
                        np.full((E, H, I // 32), 0x2000, dtype=np.uint16))
    li = synth.draw_layer(w, seed=seed, layer=0, T=1, with_experts=False)
    x = np.ascontiguousarray(synth.draw_step_x(w, seed, 0)[:1])
    bf16 = w.xtype == synth.BF16
    idx, gate = oracle.route(x, li.R, w.k, bf16=bf16)
    gfull = np.zeros((1, E), dtype=np.float32)
    gfull[0, idx[0]] = gate[0]

    def rate(fn):
        fn()
        t0, n = time.perf_counter(), 0
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        return (time.perf_counter() - t0) / n

    t_gather = rate(lambda: oracle.gather_forward(x, ex, idx, gate, bf16=bf16))
    t_dense = rate(lambda: oracle.dense_forward(x, ex, gfull, bf16=bf16))
    return {"E": E, "k": w.k, "gathered_ms_per_token": round(t_gather * 1e3, 3),
            "dense_ms_per_token": round(t_dense * 1e3, 3), "dense_over_gathered": round(t_dense / t_gather, 2),
            "E_over_k": round(E / w.k, 2)}


def trace_kernel_us(wname: str, sha: str) -> dict | None:
    """Average kernel durations from the committed rocprofv3 kernel trace of this
    workload (profiles/kernel_trace_<workload>.md), when it was taken on the
    current kernel sources (its "kernel source sha" line matches). The table
    lists kernels by total time, so of several instantiations of one kernel
    (the staged top-k, other tunings of the GEMM) the workload's main one comes
    first and is the one taken."""
    p = os.path.join(ROOT, "profiles", f"kernel_trace_{wname}.md")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        text = f.read()
    if f"kernel source sha: {sha}" not in text:
        return None
    out = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.split("|")]
        if len(cells) < 6 or not cells[1].startswith("`"):
            continue
        name = cells[1].strip("`")
        try:
            avg = float(cells[3])
        except ValueError:
            continue
        for key, pat in (("route_logits", "k_logits_"), ("topk", "k_topk<"), ("group", "k_group_"),
                         ("combine", "k_combine<"), ("gate_up", "k_gate_up_t1<"), ("down", "k_down_t1_slots<"),
                         ("down", "k_down_t1<")):
            if pat in name:
                out.setdefault(key, avg)
        if "k_gemm_dma<" in name or "k_gemm_grouped<" in name:
            targs = name[name.index("<") + 1:].split(",")
            mode = targs[2].strip() if len(targs) > 2 else ""
            out.setdefault("gemm_gate_up" if mode == "0" else "gemm_down", avg)
    return out or None


SECONDARY = ("batched_int4", "large_int4", "prefill", "prefill8k")


def run_workload(w, args, K, W, rq, synth, torch, headline: bool) -> dict:
    """Builds the workload's layers in HBM, times K steps (HIP graphs), then the
    dominant kernel's launches with events, the streaming-read reference and, for
    the headline, the rows beyond the layer. Frees its buffers before returning."""
    import numpy as np
    multi = w.layers > 1
    nl = w.layers if multi else args.copies
    log(f"workload {w.name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} scheme={w.scheme} layers={nl}")
    t_setup = time.perf_counter()
    pools, routers = build_layers(w, nl, args.seed, rq, synth, torch)
    nx = w.steps if w.steps > 1 else 8
    xs = torch.stack([to_dev(synth.draw_step_x(w, args.seed, s), w.xtype, torch) for s in range(nx)])
    xbuf = torch.empty_like(xs[0])
    ys = [torch.empty((w.T, w.H), dtype=torch.float32, device="cuda") for _ in range(nl)]
    ws = rq.Workspace()
    ws.get(rq.moe_workspace_bytes(w.T, w.E, w.H, w.I, w.k, w.scheme))
    log(f"setup {time.perf_counter() - t_setup:.1f} s, pool "
        f"{sum(p.w_gate_up.numel() + p.w_down.numel() for p in pools) / 1e9:.1f} GB codes")

    layers_per_step = nl if multi else 1
    path_flag = {"auto": 0, "gather": rq.MOE_FLAG_PATH_GATHER, "gemm": rq.MOE_FLAG_PATH_GEMM}[args.path]
    # the library's own choice (kept in step with moe_api.cpp): the GEMM path for
    # T > 1 with 16-bit activations
    gemm = args.path == "gemm" or (args.path == "auto" and w.T > 1 and w.xtype != synth.F32)

    def run_layers(step):
        ls = range(nl) if multi else [step % nl]
        for l in ls:
            rq.moe_layer_forward(xbuf, routers[l], pools[l], w.k, rq.MOE_FLAG_RENORM | path_flag, ws=ws,
                                 out=ys[l], return_routing=False)

    # eager warm-up (also checks every call succeeds)
    xbuf.copy_(xs[0])
    for s in range(2):
        run_layers(s)
    torch.cuda.synchronize()

    graphs = []
    if not args.no_graph:
        ngraph = 1 if multi else nl
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        torch.cuda.current_stream().wait_stream(side)
        for gi in range(ngraph):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_layers(gi)
            graphs.append(g)
        torch.cuda.synchronize()

    def step(s):
        xbuf.copy_(xs[s % nx])
        if graphs:
            graphs[0 if multi else s % nl].replay()
        else:
            run_layers(s)

    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for s in range(K):
        step(W + s)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    elapsed_ms = ev0.elapsed_time(ev1)
    log(f"timed {K} steps: {elapsed_ms:.2f} ms (wall {wall * 1e3:.2f} ms)")

    # realized unique experts per layer call (routing recomputed after the clock stops)
    uniq_counts = []
    for s in range(min(K, 64)):
        ss = W + s
        x = xs[ss % nx]
        for l in (range(nl) if multi else [ss % nl]):
            idx, _ = rq.moe_route(x, routers[l], w.k, rq.MOE_FLAG_RENORM)
            uniq_counts.append(len(torch.unique(idx)))
    uniq_mean = float(np.mean(uniq_counts))
    layer_calls = K * layers_per_step
    t_layer_s = elapsed_ms * 1e-3 / layer_calls
    routed_bytes = uniq_mean * expert_bytes(w)
    routed_gbps = routed_bytes / t_layer_s / 1e9
    tokens_per_s_layer = w.T / t_layer_s

    # per-kernel durations: eager pass with HIP events around every launch
    # Each timing step is queued behind a long streaming read (about 1 ms), so
    # its launches reach the GPU back to back, as in the graph, rather than one
    # by one with the host's launch gaps in between.
    spacer = torch.empty(8 << 30, dtype=torch.uint8, device="cuda")

    def timed_kernel(kid, n_steps):
        torch.cuda.synchronize()
        with rq.KernelTimer(kid, n_steps * layers_per_step + 8) as t:
            for s in range(n_steps):
                rq.moe_stream_read(spacer)
                xbuf.copy_(xs[s % nx])
                run_layers(s)
        torch.cuda.synchronize()
        return float(np.mean(t.ms)) * 1e3 if t.ms else None  # microseconds

    kids = {"route_logits": rq.MOE_KERNEL_ROUTE_LOGITS}
    if w.T > 1:
        kids.update(topk=rq.MOE_KERNEL_TOPK, group=rq.MOE_KERNEL_GROUP, combine=rq.MOE_KERNEL_COMBINE)
    if gemm:
        kids.update(gemm_gate_up=rq.MOE_KERNEL_GEMM_GATE_UP, gemm_down=rq.MOE_KERNEL_GEMM_DOWN)
        dom = "gemm_gate_up"
    else:
        kids.update(gate_up=rq.MOE_KERNEL_GATE_UP, down=rq.MOE_KERNEL_DOWN)
        dom = "gate_up"
    kern_us = {name: timed_kernel(kid, args.timer_steps) for name, kid in kids.items()}
    del spacer
    gu_us = kern_us[dom]
    # algorithmic bytes of one launch of the dominant kernel (gate/up stage):
    # routed gate/up codes + scales, the activations, and the SwiGLU output
    # (fp32 on the matvec path, fp16 on the GEMM path); single token: + router logits
    xbytes = w.T * w.H * (4 if w.xtype == 0 else 2)
    hbytes = w.T * w.k * w.I * (2 if gemm else 4)
    gu_alg = uniq_mean * gate_up_bytes(w) + xbytes + hbytes + (w.E * 4 if (w.T == 1 and not gemm) else 0)
    kname = ("grouped MFMA GEMM gate/up + SwiGLU" if gemm else
             "gathered gate/up + SwiGLU" + (" (with the top-k)" if w.T == 1 else " (grouped)"))
    achieved = gu_alg / (gu_us * 1e-6) / 1e9
    gu_flops = 2.0 * w.T * w.k * 2 * w.I * w.H
    mfma_tflops = gu_flops / (gu_us * 1e-6) / 1e12

    ceiling = stream_ceiling(int(round(routed_bytes)), rq, torch)
    extras = {}
    if headline and w.T <= 64:
        extras["miss_policies"] = miss_policies(w, [xs[i] for i in range(nx)], routers[0], pools[0], rq, torch)
        if w.T == 1:
            log("fp32 h ...")
            extras["h_fp32"] = flag_step(w, xs, nl, pools, routers, ws, K, W, path_flag | rq.MOE_FLAG_H_FP32, rq, torch)
            extras["h_fp32"]["default_us_per_layer"] = round(t_layer_s * 1e6, 3)
            log("staged layer ...")
            st = staged_step(w, xs, nl, pools, routers, ws, K, W, path_flag, rq, torch)
            st["routed_us_per_layer"] = round(t_layer_s * 1e6, 3)
            extras["staged"] = st
        if not args.no_prerouter:
            log("prerouted step ...")
            pre = prerouted_step(w, xs, nl, pools, routers, ws, args.seed, K, W, path_flag, rq, synth, torch)
            pre["routed_us_per_layer"] = round(t_layer_s * 1e6, 3)
            extras["prerouted"] = pre
        if not args.no_lora:
            log("quantized linear with LoRA ...")
            extras["lora_linear"] = lora_linear(w, args.seed, rq, synth, torch)

    traffic = None
    tf = os.path.join(ROOT, "profiles", f"traffic_{dom}_{w.name}.json")
    sha = kernel_source_sha("gemm" if gemm else "gather")
    if os.path.exists(tf) and args.k is None:
        with open(tf) as f:
            tj = json.load(f)
        if tj.get("kernel_source_sha") == sha:
            traffic = tj.get("bytes_per_launch")
    trace = trace_kernel_us(w.name, sha)

    res = {
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "k": w.k, "I": w.I,
                   "codec": "sym8" if w.scheme == 0 else "int4",
                   "x": {0: "f32", 1: "f16", 2: "bf16"}[w.xtype], "layers_per_step": layers_per_step,
                   "layer_copies": nl, "fresh_x": nx, "graph": not args.no_graph,
                   "path": "gemm" if gemm else "gather"},
        "dtype": dtype_name(w, gemm),
        "steps": K, "warmup": W,
        "ms_per_step": round(elapsed_ms / K, 5),
        "tokens_per_s_per_layer": round(tokens_per_s_layer, 1),
        "us_per_layer": round(t_layer_s * 1e6, 3),
        "step_tokens_per_s": round(w.T / (elapsed_ms * 1e-3 / K), 1),
        "routed_bytes_per_layer": int(routed_bytes),
        "unique_experts_per_layer": round(uniq_mean, 2),
        "routed_hbm_gbps": round(routed_gbps, 1),
        "routed_hbm_frac": round(routed_gbps / HBM_PEAK_GBPS, 4),
        "stream_read_ceiling": {**ceiling, "layer_vs_ceiling": round(routed_gbps / ceiling["gbps"], 4)},
        **extras,
        "kernel_us": {n: round(v, 3) for n, v in kern_us.items()},
        "kernel_trace_us": trace,
        "roofline": {"kernel": kname, "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(gu_alg), "avg_launch_us": round(gu_us, 3),
                     **({"avg_launch_us_trace": round(trace[dom], 3)} if trace and dom in trace else {}),
                     **({"mfma_tflops": round(mfma_tflops, 1), "mfma_peak_tflops": 2500.0,
                         "mfma_frac": round(mfma_tflops / 2500.0, 4)} if gemm else {})},
        "kernel_source_sha": sha,
    }
    del graphs, pools, routers, xs, ys, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the layer is built and measured on a single MI355X "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch

    import routed_expert_quantized_amd as rq
    import synth

    w = synth.WORKLOADS[args.workload]
    if args.k is not None:
        w = dataclasses.replace(w, k=args.k)
    K = args.steps if args.steps is not None else (512 if w.T == 1 else 64)
    W = args.warmup if args.warmup is not None else 32
    rq.lib()
    head = run_workload(w, args, K, W, rq, synth, torch, headline=True)
    secondary = {}
    names = [] if args.secondary == "none" or args.workload != "decode40" or args.k is not None else \
        [n for n in args.secondary.split(",") if n]
    for name in names:
        sw = synth.WORKLOADS[name]
        # the same step count as the headline, at most 64 (a step is one layer call
        # for single-layer workloads, 60 layer calls at large_int4)
        secondary[name] = run_workload(sw, args, min(K, 64), min(W, 16), rq, synth, torch, headline=False)

    result = {
        "metric": METRIC,
        "value": head["tokens_per_s_per_layer"],
        "unit": "tokens/s per MoE layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        **{k: v for k, v in head.items() if k not in ("config", "dtype", "steps", "warmup", "ms_per_step")},
    }
    if secondary:
        result["workloads"] = secondary
    if args.calib_copy_mib:
        # a plain elementwise copy of known size (negation: a kernel nothing else
        # here launches): its FETCH_SIZE / WRITE_SIZE per dispatch give the factor
        # between counter units and bytes moved
        n = args.calib_copy_mib << 18
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = n * 4
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cb = cpu_baseline(w, args.seed, args.cpu_seconds)
        cb["host"] = host_info()
        one = cpu_baseline(w, args.seed, args.cpu_seconds / 3, threads=1)
        cb["one_thread"] = {"value": one["value"], "cores": one["cores"], "sample": one["sample"]}
        if args.workload == "decode40" and args.k is None:
            cb["dense_all_experts"] = {n: dense_over_read(synth.WORKLOADS[n], args.seed, 1.0)
                                       for n in ("tiny", "decode40")}
        result["cpu_baseline"] = cb
        for name, r in secondary.items():
            r["cpu_baseline"] = cpu_baseline(synth.WORKLOADS[name], args.seed, args.cpu_seconds / 3)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
