"""Calibrate the Zipf(1.1) popularity strength of the batched_int4 workload.

The 35B-A3B observation in "QwenのMoEルーターを観測してホットエキスパートを先読みしても
速くならなかった" (lilting.ch, section "35B-A3Bでのエキスパート観測") is that about 60%
of a layer's experts are hit over a generation, far fewer than uniform routing
would hit. This script bisects on beta (logit bias = beta * ln p_e) so that 64
tokens routed top-10 over 512 experts hit 60% of them on average over layers
0..7 at seed 0, using only the oracle's router. It writes zipf_beta.json; the
generator's ZIPF_BETA_BATCHED constant is that value rounded to two digits.

Run: python tests/golden/calibrate_zipf.py
"""
import dataclasses
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

TARGET = 0.60
LAYERS = 8


def hit_fraction(beta: float) -> float:
    w = dataclasses.replace(synth.WORKLOADS["batched_int4"], zipf_beta=beta)
    fr = []
    for layer in range(LAYERS):
        li = synth.draw_layer(w, seed=0, layer=layer, with_experts=False)
        idx, _ = oracle.route(li.x, li.R, w.k)
        fr.append(len(np.unique(idx)) / w.E)
    return float(np.mean(fr))


def main():
    lo, hi = 0.0, 2.0
    for _ in range(16):
        mid = (lo + hi) / 2
        if hit_fraction(mid) > TARGET:
            lo = mid
        else:
            hi = mid
    beta = (lo + hi) / 2
    out = {"beta": beta, "hit_fraction": hit_fraction(beta), "hit_fraction_beta0": hit_fraction(0.0),
           "target": TARGET, "layers": LAYERS, "seed": 0}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_beta.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()
