"""The library's miss-policy replay (moe_miss_replay, host C++) against the
reference in oracle/miss_policy.py: identical decisions and substituted mass on
the hand-worked sequence and on seeded routings."""
import json
import os

import numpy as np
import pytest

import routed_expert_quantized_amd as rq
from oracle import miss_policy as mp

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(rq.LIB_PATH):
        from routed_expert_quantized_amd import build
        build.build()


def _routings(seed, T, E, k, reuse):
    g = np.random.default_rng(seed)
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float32)
    for t in range(T):
        idx[t] = g.permutation(idx[t - 1]) if t and g.random() < reuse else g.choice(E, size=k, replace=False)
        w = np.sort(g.random(k))[::-1] + 1e-3
        gate[t] = (w / w.sum()).astype(np.float32)
    return idx, gate


def _same(idx, gate, E, C, policy, thr, beta):
    m, sync, bg, res = rq.moe_miss_replay(idx, gate, E, C, policy, thr, beta)
    rm, rsync, rbg, rres = mp.replay(idx, gate.astype(np.float64), E, C, policy, float(np.float32(thr)), float(np.float32(beta)))
    assert np.array_equal(sync, rsync) and np.array_equal(bg, rbg) and np.array_equal(res, rres)
    assert np.array_equal(m, rm.astype(np.float32))


def test_hand_worked_sequence():
    with open(os.path.join(HERE, "golden", "miss_policy.json")) as f:
        gd = json.load(f)
    idx = np.array(gd["idx"], dtype=np.int32)
    gate = np.array(gd["gate"], dtype=np.float32)
    for r in gd["runs"]:
        m, sync, bg, res = rq.moe_miss_replay(idx, gate, gd["E"], gd["capacity"], r["policy"], gd["threshold"], r["beta"])
        assert np.allclose(m, r["m"], atol=1e-6)
        assert sync.tolist() == r["sync"] and bg.tolist() == r["bg"]
        assert sorted(np.nonzero(res)[0].tolist()) == r["resident"]


@pytest.mark.parametrize("policy", [rq.MOE_MISS_FETCH_ALL, rq.MOE_MISS_RULE, rq.MOE_MISS_FIRST_CHOICE])
@pytest.mark.parametrize("beta", [0.0, 0.5, 0.2])
@pytest.mark.parametrize("E,k,C,reuse", [(24, 4, 6, 0.3), (64, 8, 16, 0.27), (512, 10, 128, 0.27), (10, 3, 10, 0.5)])
def test_matches_reference(policy, beta, E, k, C, reuse):
    idx, gate = _routings(E + k + C, 400, E, k, reuse)
    _same(idx, gate, E, C, policy, 0.15, beta)


def test_validation():
    idx = np.array([[0, 1]], dtype=np.int32)
    gate = np.array([[0.6, 0.4]], dtype=np.float32)
    with pytest.raises(rq.MoeError):
        rq.moe_miss_replay(idx, gate, 4, 1, rq.MOE_MISS_RULE)          # capacity < k
    with pytest.raises(rq.MoeError):
        rq.moe_miss_replay(np.array([[0, 4]], dtype=np.int32), gate, 4, 2, rq.MOE_MISS_RULE)  # id out of range
    with pytest.raises(rq.MoeError):
        rq.moe_miss_replay(np.array([[1, 1]], dtype=np.int32), gate, 4, 2, rq.MOE_MISS_RULE)  # repeated id
    with pytest.raises(rq.MoeError):
        rq.moe_miss_replay(idx, gate, 4, 2, 7)                          # unknown policy
    m, sync, bg, res = rq.moe_miss_replay(np.zeros((0, 2), dtype=np.int32), np.zeros((0, 2), dtype=np.float32), 4, 2,
                                          rq.MOE_MISS_RULE)
    assert m.shape == (0,) and not res.any()
