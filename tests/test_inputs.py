"""The seeded generator: determinism, activation encodings and the workload
shapes it is asked to reproduce (expert popularity skew, token reuse)."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests.cases import enforce_gap, gap_failures

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_draws_are_deterministic_and_streams_independent():
    w = synth.WORKLOADS["tiny"]
    a = synth.draw_layer(w, seed=0)
    b = synth.draw_layer(w, seed=0)
    c = synth.draw_layer(w, seed=0, layer=1)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w_gate_up, b.w_gate_up)
    assert not np.array_equal(a.x, c.x)
    assert a.w_gate_up.shape == (16, 256, 256) and a.w_down.shape == (16, 256, 128)


def test_bf16_encoding_matches_torch_round_to_nearest_even():
    torch = pytest.importorskip("torch")
    v = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    v[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(v), ref)


def test_zipf_calibration_hits_about_sixty_percent():
    with open(os.path.join(GOLDEN, "zipf_beta.json")) as f:
        cal = json.load(f)
    assert abs(cal["beta"] - synth.ZIPF_BETA_BATCHED) < 0.01
    w = synth.WORKLOADS["batched_int4"]
    fr = []
    for layer in range(2):
        li = synth.draw_layer(w, seed=0, layer=layer, with_experts=False)
        idx, _ = oracle.route(li.x, li.R, w.k)
        fr.append(len(np.unique(idx)) / w.E)
    assert 0.55 <= np.mean(fr) <= 0.65
    # without the skew, routing spreads wider (uniform would hit ~72%)
    assert cal["hit_fraction_beta0"] > 0.7


def test_token_reuse_shares_previous_top_k_set():
    w = synth.WORKLOADS["large_int4"]
    li = synth.draw_layer(w, seed=0, with_experts=False, T=400)
    assert 0.2 <= li.reuse.mean() <= 0.34
    idx, _ = oracle.route(li.x, li.R, w.k)
    for t in np.nonzero(li.reuse)[0]:
        assert set(idx[t]) == set(idx[t - 1])


def test_gap_enforcement_reaches_margin():
    w = synth.WORKLOADS["tiny"]
    li = enforce_gap(w, synth.draw_layer(w, seed=0, T=64), seed=0, layer=0)
    assert len(gap_failures(li.x, li.R, w.k, False)) == 0
