"""Pins of the miss-policy reference (oracle/miss_policy.py): a hand-worked
sequence, and invariants that follow from the rules on random routings."""
import json
import os

import numpy as np
import pytest

from oracle import miss_policy as mp

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    with open(os.path.join(HERE, "golden", "miss_policy.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("run", range(3))
def test_hand_worked_sequence(run):
    gd = _golden()
    r = gd["runs"][run]
    m, sync, bg, res = mp.replay(np.array(gd["idx"]), np.array(gd["gate"]), gd["E"], gd["capacity"], r["policy"],
                                 gd["threshold"], r["beta"])
    assert np.allclose(m, r["m"], atol=1e-12)
    assert sync.tolist() == r["sync"]
    assert bg.tolist() == r["bg"]
    assert sorted(np.nonzero(res)[0].tolist()) == r["resident"]


def _routings(seed, T, E, k, reuse=0.3):
    """Random routings with some temporal reuse; gates sorted, renormalised."""
    g = np.random.default_rng(seed)
    idx = np.empty((T, k), dtype=np.int64)
    gate = np.empty((T, k))
    for t in range(T):
        if t and g.random() < reuse:
            idx[t] = g.permutation(idx[t - 1])
        else:
            idx[t] = g.choice(E, size=k, replace=False)
        w = np.sort(g.random(k))[::-1] + 1e-3
        gate[t] = w / w.sum()
    return idx, gate


@pytest.mark.parametrize("seed", range(4))
def test_invariants(seed):
    E, k, C, T = 24, 4, 6, 300
    idx, gate = _routings(seed, T, E, k)
    # fetch-all never substitutes; every miss is a synchronous fetch
    m, sync, bg, _ = mp.replay(idx, gate, E, C, mp.FETCH_ALL, beta=0.5)
    assert not m.any() and not bg.any()
    # the first-choice rule never substitutes slot 0; the 0.15 rule only substitutes
    # non-first slots with gate < 0.15
    for pol in (mp.FIRST_CHOICE, mp.RULE):
        for beta in (0.0, 0.5):
            m, sync, bg, res = mp.replay(idx, gate, E, C, pol, 0.15, beta)
            assert (m >= 0).all() and (m <= 1 - gate[:, 0] + 1e-12).all()
            assert res.sum() <= C
            if beta == 0.0:
                assert not bg.any()
            if pol == mp.RULE:
                # substituted mass is made of slots below the threshold only
                assert (m <= np.where(gate[:, 1:] < 0.15, gate[:, 1:], 0).sum(axis=1) + 1e-12).all()
    # with room for every expert nothing is ever evicted: each expert misses once at most
    m, sync, bg, res = mp.replay(idx, gate, E, E, mp.FETCH_ALL)
    assert sync.sum() == len(np.unique(idx)) and res.sum() == len(np.unique(idx))


def test_fetched_plus_substituted_covers_every_miss():
    """Brute-force count of misses against an independent walk of the cache:
    with the first-choice rule and no admission, a token's misses are its
    synchronous fetches plus its substituted slots."""
    E, k, C, T = 12, 3, 4, 200
    idx, gate = _routings(7, T, E, k, reuse=0.5)
    m, sync, bg, _ = mp.replay(idx, gate, E, C, mp.FIRST_CHOICE)
    # substituted slots recovered from m: gates are distinct, so each subset sum identifies its slots
    n_sub = np.zeros(T, dtype=int)
    for t in range(T):
        best = min(range(1 << (k - 1)), key=lambda b: abs(m[t] - sum(gate[t, 1 + j] for j in range(k - 1) if b >> j & 1)))
        n_sub[t] = bin(best).count("1")
    assert ((sync + n_sub) <= k).all()
    assert (sync <= 1).all()  # only the first choice is ever fetched


def test_rejects_capacity_below_k():
    with pytest.raises(ValueError):
        mp.replay(np.array([[0, 1, 2]]), np.array([[0.5, 0.3, 0.2]]), 8, 2, mp.RULE)
