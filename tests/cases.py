"""Test-side helpers: parity tolerance, logit-gap enforcement, quantised cases.

Test infrastructure. Uses the oracle (for the logit-gap rule) and the seeded
generator; never the GPU library.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

# Parity contract of the layer: indices bit-exact, gates within 1e-5 absolute,
# outputs within 1e-3 of the output norm, per token.
GATE_ATOL = 1e-5
Y_REL_NORM = 1e-3
LOGIT_GAP = 1e-3


def rel_norm_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max over tokens of max_i |y - ref| / ||ref||_2 (rows = tokens, last axis = H)."""
    y = np.asarray(y, dtype=np.float64).reshape(-1, ref.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.abs(y - r).max(axis=1)
    den = np.linalg.norm(r, axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if len(num) else 0.0


def rel_inf_err(y: np.ndarray, ref: np.ndarray) -> float:
    """Stricter reading: max |y - ref| / max |ref| per token."""
    y = np.asarray(y, dtype=np.float64).reshape(-1, ref.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.abs(y - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if len(num) else 0.0


def gap_failures(x: np.ndarray, R: np.ndarray, k: int, bf16: bool) -> np.ndarray:
    """Tokens whose top k+1 fp64 logits are not separated by >= LOGIT_GAP."""
    lg = oracle.logits(x, R, bf16=bf16)
    E = R.shape[0]
    m = min(k + 1, E)
    top = -np.sort(-lg, axis=1)[:, :m]
    gaps = top[:, :-1] - top[:, 1:] if m > 1 else np.full((lg.shape[0], 1), np.inf)
    return np.nonzero((gaps < LOGIT_GAP).any(axis=1))[0]


def enforce_gap(w: synth.Workload, li: synth.LayerInputs, seed: int, layer: int, k: int | None = None,
                max_attempts: int = 64) -> synth.LayerInputs:
    """Redraw tokens until every token's routing decision has margin >= LOGIT_GAP.

    A token that repeats its predecessor (token reuse) is re-copied after its
    source is redrawn, so reuse chains keep sharing one top-k set."""
    k = w.k if k is None else k
    bf16 = w.xtype == synth.BF16
    const_channel = w.zipf_s > 0
    for attempt in range(max_attempts):
        bad = gap_failures(li.x, li.R, k, bf16)
        if len(bad) == 0:
            return li
        roots = set()
        for t in bad:
            t = int(t)
            while li.reuse is not None and li.reuse[t]:
                t -= 1
            roots.add(t)
        synth.redraw_tokens(li.x32, sorted(roots), seed, w.wid, layer, attempt, const_channel)
        if li.reuse is not None:
            for t in range(1, li.x32.shape[0]):
                if li.reuse[t]:
                    li.x32[t] = li.x32[t - 1]
        li.x = synth.encode_x(li.x32, w.xtype)
    raise RuntimeError(f"logit gap not reached after {max_attempts} attempts for {w.name}")


def oracle_experts(li: synth.LayerInputs, scheme: int) -> oracle.Experts:
    return oracle.quantize_experts(li.w_gate_up, li.w_down, scheme)
