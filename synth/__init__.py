"""Seeded synthetic inputs for the routed, block-quantized MoE expert layer.

This module only draws random numbers and lays them out. It holds none of the
layer's arithmetic (no routing, quantisation, projection or combine), so the
oracle and the GPU library can both be fed from it without sharing code.

Workloads (shapes and distributions of the pages' models):
  tiny          T=1,    H=256,  E=16,  k=4,  I=128,  sym8, x fp32
  decode40      T=1,    H=2048, E=256, k=8,  I=512,  sym8, x fp16, 40 stacked layers
  batched_int4  T=64,   H=2048, E=512, k=10, I=512,  int4, x fp16, Zipf(1.1) expert popularity
  prefill       T=2048, H=2048, E=256, k=8,  I=512,  sym8, x bf16
  large_int4    T=16,   H=4096, E=512, k=10, I=1024, int4, x fp16, 60 layers, 27% token reuse
  prefill8k     T=8192, H=2048, E=256, k=8,  I=512,  sym8, x bf16 (supplementary: ~256
                assignments per expert, where the grouped GEMM is bound by the matrix cores)

The 256-expert top-8, d_model 2048, 40-layer shape is the 35B-A3B model of
"QwenのMoEルーターを観測してホットエキスパートを先読みしても速くならなかった"
(lilting.ch), section "検証環境" (test environment). Its observation that about
60% of experts are hit per layer over a generation (section
"35B-A3Bでのエキスパート観測") sets the batched_int4 popularity skew.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SYM8, INT4 = 0, 1
F32, F16, BF16 = 0, 1, 2

# Zipf(1.1) popularity strength for batched_int4, in logit units per unit of
# ln(popularity). Chosen by tests/golden/calibrate_zipf.py, which bisects on the
# oracle's router so that ~60% of the 512 experts are hit by 64 tokens.
ZIPF_BETA_BATCHED = 0.62

_WORKLOAD_IDS = {"tiny": 0, "decode40": 1, "batched_int4": 2, "prefill": 3, "large_int4": 4, "prefill8k": 5}


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    scheme: int
    xtype: int
    layers: int = 1
    router_std: float = 0.05
    weight_std: float = 0.02
    zipf_s: float = 0.0
    zipf_beta: float = 0.0
    reuse_p: float = 0.0
    steps: int = 1
    notes: str = field(default="", compare=False)

    @property
    def wid(self) -> int:
        return _WORKLOAD_IDS.get(self.name, 99)


WORKLOADS = {
    "tiny": Workload("tiny", T=1, H=256, E=16, k=4, I=128, scheme=SYM8, xtype=F32),
    "decode40": Workload("decode40", T=1, H=2048, E=256, k=8, I=512, scheme=SYM8, xtype=F16,
                         layers=40, steps=512),
    "batched_int4": Workload("batched_int4", T=64, H=2048, E=512, k=10, I=512, scheme=INT4, xtype=F16,
                             zipf_s=1.1, zipf_beta=ZIPF_BETA_BATCHED),
    "prefill": Workload("prefill", T=2048, H=2048, E=256, k=8, I=512, scheme=SYM8, xtype=BF16),
    "large_int4": Workload("large_int4", T=16, H=4096, E=512, k=10, I=1024, scheme=INT4, xtype=F16,
                           layers=60, router_std=4096 ** -0.5, reuse_p=0.27),
    "prefill8k": Workload("prefill8k", T=8192, H=2048, E=256, k=8, I=512, scheme=SYM8, xtype=BF16),
}


def rng(seed: int, workload: int, layer: int = 0, step: int = 0, stream: int = 0) -> np.random.Generator:
    """Independent PCG64 stream per (seed, workload, layer, step, stream)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, workload, layer, step, stream])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even) and return the 16-bit patterns.
    Inputs are finite draws; NaN handling is not needed here."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def encode_x(x32: np.ndarray, xtype: int) -> np.ndarray:
    """Store fp32 draws in the activation type: fp32, fp16 (numpy RNE) or bf16 bits."""
    if xtype == F32:
        return np.ascontiguousarray(x32, dtype=np.float32)
    if xtype == F16:
        return np.ascontiguousarray(x32.astype(np.float16))
    return f32_to_bf16_bits(x32)


def draw_x(g: np.random.Generator, T: int, H: int) -> np.ndarray:
    return g.standard_normal((T, H), dtype=np.float32)


def draw_router(g: np.random.Generator, E: int, H: int, std: float) -> np.ndarray:
    return (g.standard_normal((E, H), dtype=np.float32) * np.float32(std)).astype(np.float32)


def draw_expert(seed: int, workload: int, layer: int, e: int, H: int, I: int, std: float):
    """fp32 weights of expert e from its own stream: gate/up [2I][H] (gate rows
    first), down [H][I]. Any subset of experts can be drawn on its own."""
    g = rng(seed, workload, layer, 0, 1000 + e)
    wgu = (g.standard_normal((2 * I, H), dtype=np.float32) * np.float32(std)).astype(np.float32)
    wd = (g.standard_normal((H, I), dtype=np.float32) * np.float32(std)).astype(np.float32)
    return wgu, wd


def draw_experts(seed: int, workload: int, layer: int, experts, H: int, I: int, std: float):
    """Stacked fp32 weights of the listed experts: [n][2I][H] and [n][H][I]."""
    experts = list(experts)
    wgu = np.empty((len(experts), 2 * I, H), dtype=np.float32)
    wd = np.empty((len(experts), H, I), dtype=np.float32)
    for i, e in enumerate(experts):
        wgu[i], wd[i] = draw_expert(seed, workload, layer, e, H, I, std)
    return wgu, wd


def zipf_log_popularity(g: np.random.Generator, E: int, s: float) -> np.ndarray:
    """ln p_e for a Zipf(s) popularity over a seeded random ranking of the experts."""
    ranks = g.permutation(E) + 1
    logp = -s * np.log(ranks.astype(np.float64))
    logp -= np.log(np.exp(logp).sum())
    return logp


def apply_zipf_bias(x32: np.ndarray, R: np.ndarray, logp: np.ndarray, beta: float) -> None:
    """Fold a per-expert logit bias beta*ln p_e into a constant input channel:
    x[:, H-1] = 1 and R[:, H-1] += beta*ln p_e (in place)."""
    x32[:, -1] = 1.0
    R[:, -1] = (R[:, -1].astype(np.float64) + beta * logp).astype(np.float32)


def apply_reuse(x32: np.ndarray, g: np.random.Generator, p: float) -> np.ndarray:
    """With probability p, token t (t >= 1) repeats token t-1 exactly, so it
    reuses the previous token's top-k set. Returns the boolean reuse mask."""
    mask = np.zeros(x32.shape[0], dtype=bool)
    if x32.shape[0] > 1:
        mask[1:] = g.random(x32.shape[0] - 1) < p
    for t in range(1, x32.shape[0]):
        if mask[t]:
            x32[t] = x32[t - 1]
    return mask


@dataclass
class LayerInputs:
    """One layer's fp32 draws (weights not yet quantised) and activation."""
    x32: np.ndarray          # [T][H] fp32 draws
    x: np.ndarray            # [T][H] in the workload's activation type
    R: np.ndarray            # [E][H] fp32
    w_gate_up: np.ndarray    # [E][2I][H] fp32
    w_down: np.ndarray       # [E][H][I] fp32
    reuse: np.ndarray | None = None


def draw_layer(w: Workload, seed: int = 0, layer: int = 0, T: int | None = None,
               with_experts: bool = True) -> LayerInputs:
    """Draw one layer of a workload on the host. T overrides the token count."""
    T = w.T if T is None else T
    gx = rng(seed, w.wid, layer, 0, 0)
    gr = rng(seed, w.wid, layer, 0, 1)
    x32 = draw_x(gx, T, w.H)
    R = draw_router(gr, w.E, w.H, w.router_std)
    if w.zipf_s > 0:
        logp = zipf_log_popularity(rng(seed, w.wid, layer, 0, 3), w.E, w.zipf_s)
        apply_zipf_bias(x32, R, logp, w.zipf_beta)
    reuse = None
    if w.reuse_p > 0:
        reuse = apply_reuse(x32, rng(seed, w.wid, layer, 0, 4), w.reuse_p)
    if with_experts:
        wgu, wd = draw_experts(seed, w.wid, layer, range(w.E), w.H, w.I, w.weight_std)
    else:
        wgu = wd = None
    return LayerInputs(x32, encode_x(x32, w.xtype), R, wgu, wd, reuse)


def redraw_tokens(x32: np.ndarray, tokens, seed: int, workload: int, layer: int, attempt: int,
                  const_channel: bool) -> None:
    """Replace the listed tokens with fresh N(0,1) draws from a stream keyed by attempt."""
    g = rng(seed, workload, layer, 1 + attempt, 5)
    for t in tokens:
        x32[t] = g.standard_normal(x32.shape[1], dtype=np.float32)
        if const_channel:
            x32[t, -1] = 1.0


def draw_routing(g: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    """[T][k] int32 expert ids, distinct within each token, uniform."""
    return np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32).reshape(T, k)


# Prerouter head width (fc1 outputs). The pages give the input width (H + 2E)
# but not this one; the measured head takes F = E.
PREROUTER_F = 256


def draw_prerouter(seed: int, workload: int, layer: int, H: int, E: int, F: int, router_std: float,
                   bias: bool = True) -> dict:
    """fp32 prerouter head weights in the layout [F][H+2E] (fc1), [E][F] (fc2),
    [E][H+2E] (linear residual path). The residual path's hidden columns are a
    router draw (the warm start from the next layer's router); the rest are
    Gaussian, scaled by fan-in. Biases are None when bias is False."""
    g = rng(seed, workload, layer, 0, 2000)
    D = H + 2 * E
    std1 = np.float32(1.0 / np.sqrt(D))
    w1 = (g.standard_normal((F, D), dtype=np.float32) * std1).astype(np.float32)
    b1 = (g.standard_normal(F, dtype=np.float32) * np.float32(0.1)).astype(np.float32) if bias else None
    w2 = (g.standard_normal((E, F), dtype=np.float32) * np.float32(0.5 / np.sqrt(F))).astype(np.float32)
    b2 = (g.standard_normal(E, dtype=np.float32) * np.float32(0.1)).astype(np.float32) if bias else None
    wl = np.empty((E, D), dtype=np.float32)
    wl[:, :H] = draw_router(g, E, H, router_std)
    wl[:, H:] = g.standard_normal((E, 2 * E), dtype=np.float32) * np.float32(0.5)
    return {"w1": w1, "b1": b1, "w2": w2, "b2": b2, "wl": wl}


def draw_step_x(w: Workload, seed: int, step: int, T: int | None = None) -> np.ndarray:
    """Activations of one decode/prefill step, with the workload's structure
    (constant channel under a popularity skew, token reuse), encoded."""
    T = w.T if T is None else T
    x32 = draw_x(rng(seed, w.wid, 100000 + step, 0, 0), T, w.H)
    if w.zipf_s > 0:
        x32[:, -1] = 1.0
    if w.reuse_p > 0:
        apply_reuse(x32, rng(seed, w.wid, 100000 + step, 0, 4), w.reuse_p)
    return encode_x(x32, w.xtype)


def torch_expert_chunks(w: Workload, seed: int, layer: int, chunk: int, device):
    """Device fp32 draws of a layer's experts, `chunk` experts at a time, from a
    seeded torch generator on the device: yields (e0, w_gate_up [c][2I][H], w_down [c][H][I])."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + w.wid * 7919 + layer) & 0x7FFFFFFFFFFFFFFF)
    for e0 in range(0, w.E, chunk):
        c = min(chunk, w.E - e0)
        wgu = torch.randn((c, 2 * w.I, w.H), generator=g, device=device, dtype=torch.float32).mul_(w.weight_std)
        wd = torch.randn((c, w.H, w.I), generator=g, device=device, dtype=torch.float32).mul_(w.weight_std)
        yield e0, wgu, wd
