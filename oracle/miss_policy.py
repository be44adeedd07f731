"""Test infrastructure: the plain, slow reference of the expert-cache miss policies.

Only tests/, smoke() and bench.py's CPU baseline load this module; the library's
own replay (moe_miss_replay) shares no code with it.

"Which Expert Misses Are Worth Waiting For? Substitution and Caching for
Mixture-of-Experts Inference on a Consumer GPU" (gist.science), section 手法
(method): about a quarter of each layer's experts are resident; a routed expert
that is not resident is either fetched synchronously or substituted by a
resident one; the substituted gate mass m of a token is the sum of the
normalised gates of its substituted experts. Policies: fetch every miss; the
0.15 rule (fetch a miss that is the router's first choice or has gate >= 0.15,
substitute the rest); the first-choice rule (fetch only first-choice misses);
background admission (accumulate each expert's substituted gate mass and admit
it once the sum reaches a threshold, 0.5 in the pages' selected policies).
Section 主な貢献と知見 (findings), item 5: the selected policies pair a rule with
frequency-based eviction and background admission at beta = 0.5.

Readings where the page is silent (each one is a plain choice):
  - one cache per layer, capacity C slots, k <= C <= E, initially empty;
  - an expert's frequency counts every token that selected it (hit or miss),
    counted for all k selections of a token before its slots are decided;
  - an admission into a full cache evicts the resident expert with the lowest
    frequency, the lower id on ties, never one the current token selected;
  - slots are decided in slot order (descending gate); a synchronous fetch is
    resident at once; background admissions follow the token's decisions, in
    slot order, and an admission (of either kind) resets the accumulator;
  - m is the sum of the substituted slots' gates, the renormalised top-k gates.
"""
from __future__ import annotations

import numpy as np

FETCH_ALL, RULE, FIRST_CHOICE = 0, 1, 2


def replay(idx: np.ndarray, gate: np.ndarray, E: int, capacity: int, policy: int,
           threshold: float = 0.15, beta: float = 0.0):
    """Replay the routing of T tokens (idx/gate [T][k], slot order) through the
    cache. Returns (m [T] float64, sync [T] int, bg [T] int, resident [E] bool)."""
    idx = np.asarray(idx, dtype=np.int64)
    gate = np.asarray(gate, dtype=np.float64)
    T, k = idx.shape
    if not (1 <= k <= capacity <= E):
        raise ValueError("need 1 <= k <= capacity <= E")
    resident: set[int] = set()
    freq = [0] * E
    acc = [0.0] * E
    m = np.zeros(T)
    sync = np.zeros(T, dtype=np.int64)
    bg = np.zeros(T, dtype=np.int64)

    def admit(e: int, chosen: set[int]) -> None:
        if len(resident) >= capacity:
            victim = min((v for v in resident if v not in chosen), key=lambda v: (freq[v], v))
            resident.remove(victim)
        resident.add(e)
        acc[e] = 0.0

    for t in range(T):
        chosen = {int(e) for e in idx[t]}
        for e in idx[t]:
            freq[int(e)] += 1
        substituted = []
        for s in range(k):
            e, g = int(idx[t, s]), float(gate[t, s])
            if e in resident:
                continue
            fetch = (policy == FETCH_ALL or (policy == RULE and (s == 0 or g >= threshold))
                     or (policy == FIRST_CHOICE and s == 0))
            if fetch:
                admit(e, chosen)
                sync[t] += 1
            else:
                m[t] += g
                substituted.append((e, g))
        if beta > 0.0:
            for e, g in substituted:
                acc[e] += g
                if acc[e] >= beta:
                    admit(e, chosen)
                    bg[t] += 1
    res = np.zeros(E, dtype=bool)
    res[list(resident)] = True
    return m, sync, bg, res
