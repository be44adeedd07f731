"""GPU test helpers: device expert pools built from the seeded draws.

Each side quantises the same fp32 draws itself: the GPU with moe_quantize, the
oracle with its own quantiser. Experts that no token routes to get NaN scales,
so any read of an unrouted expert would turn the output into NaN.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import routed_expert_quantized_amd as rq
import synth

NAN_F16 = 0x7E00


def device_pool(w: synth.Workload, seed: int, layer: int, experts, device="cuda", nan_fill=True) -> rq.Experts:
    """Device experts where only `experts` hold quantised draws; the rest have NaN scales."""
    E, H, I = w.E, w.H, w.I
    cbh = H if w.scheme == synth.SYM8 else H // 2
    cbi = I if w.scheme == synth.SYM8 else I // 2
    fill = NAN_F16 if nan_fill else 0
    wgu = torch.full((E, 2 * I, cbh), 0x5A, dtype=torch.uint8, device=device)
    sgu = torch.full((E, 2 * I, H // 32), fill, dtype=torch.int16, device=device)
    wd = torch.full((E, H, cbi), 0x5A, dtype=torch.uint8, device=device)
    sd = torch.full((E, H, I // 32), fill, dtype=torch.int16, device=device)
    for e in experts:
        a, b = synth.draw_expert(seed, w.wid, layer, int(e), H, I, w.weight_std)
        ca, sa = rq.moe_quantize(torch.from_numpy(a).to(device), w.scheme)
        cb, sb = rq.moe_quantize(torch.from_numpy(b).to(device), w.scheme)
        wgu[e], sgu[e], wd[e], sd[e] = ca, sa, cb, sb
    return rq.Experts(E, H, I, w.scheme, wgu, sgu, wd, sd)


def oracle_compact(w: synth.Workload, seed: int, layer: int, experts) -> tuple[oracle.Experts, dict]:
    """Oracle experts holding only `experts` (compact ids), and the id map."""
    experts = [int(e) for e in experts]
    wgu, wd = synth.draw_experts(seed, w.wid, layer, experts, w.H, w.I, w.weight_std)
    ex = oracle.quantize_experts(wgu, wd, w.scheme)
    return ex, {e: i for i, e in enumerate(experts)}


def remap(idx: np.ndarray, m: dict) -> np.ndarray:
    return np.vectorize(lambda e: m[int(e)])(idx).astype(np.int32)


def to_dev_x(x: np.ndarray, xtype: int, device="cuda") -> torch.Tensor:
    if xtype == synth.F32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    if xtype == synth.F16:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
