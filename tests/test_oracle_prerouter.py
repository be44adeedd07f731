"""Pins for the oracle's prerouter head.

"The Other Half of the Memory Wall: Serving 35B MoEs from SSD with Trained Routing
Prediction" (xyznot.com), section 手法 (method), "Prerouterヘッドのアーキテクチャ": the
head's input is the hidden state joined with the top-k one-hot routing vectors of
the current and the previous token (H + 2E values), and the head is
fc2(erf-gelu(fc1(x))) plus a linear residual path warm-started from the next
layer's router. Its top-k is the next layer's routing.

What pins each step (none of them re-types the oracle's own formula):
  - erf-GELU and the fc1/fc2 orientation: printed values of the standard normal
    CDF (z * Phi(z) at z = 1, 2, -1), through an asymmetric fc1 and fc2;
  - the linear residual path and the top-k: at warm start (fc1 = 0, l = [R 0 0])
    the head must give exactly the router's logits, indices and gates;
  - the k-hot layout (current routing at offset H, previous at H + E): hand-worked
    logits and orderings;
  - the biases (fc1's inside the GELU, fc2's outside): hand-worked values.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle

# standard normal CDF, as printed in normal tables
PHI_1 = 0.8413447460685429
PHI_2 = 0.9772498680518208
PHI_M1 = 0.15865525393145707


def _head(H, E, F, seed=0, scale=1.0, bias=True):
    g = np.random.default_rng(seed)
    D = H + 2 * E
    return oracle.PrerouterHead(
        w1=(g.standard_normal((F, D)) * scale / np.sqrt(D)).astype(np.float32),
        b1=(g.standard_normal(F) * 0.1).astype(np.float32) if bias else None,
        w2=(g.standard_normal((E, F)) * scale / np.sqrt(F)).astype(np.float32),
        b2=(g.standard_normal(E) * 0.1).astype(np.float32) if bias else None,
        wl=(g.standard_normal((E, D)) * scale / np.sqrt(D)).astype(np.float32))


def _zero_head(H, E, F):
    D = H + 2 * E
    return oracle.PrerouterHead(w1=np.zeros((F, D), np.float32), b1=None, w2=np.zeros((E, F), np.float32),
                                b2=None, wl=np.zeros((E, D), np.float32))


def _distinct_ids(g, T, E, k):
    return np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def test_erf_gelu_matches_normal_table_through_asymmetric_fc1_fc2():
    H, E, F = 32, 2, 2
    hd = _zero_head(H, E, F)
    hd.w1[0, 3] = 1.0     # a0 = gelu(x3)
    hd.w1[1, 5] = -1.0    # a1 = gelu(-x5)
    hd.w2[:] = [[1.0, 0.5], [0.0, 1.0]]
    x = np.zeros((3, H), np.float32)
    x[0, 3], x[0, 5] = 1.0, -2.0      # gelu(1) = Phi(1), gelu(2) = 2 Phi(2)
    x[1, 3], x[1, 5] = -1.0, 0.0      # gelu(-1) = -Phi(-1), gelu(0) = 0
    x[2, 3], x[2, 5] = 0.0, 1.0       # gelu(0) = 0, gelu(-1) = -Phi(-1)
    _, _, lg = oracle.prerouter(x, hd, None, None, k=1)
    want = np.array([[PHI_1 + 0.5 * 2 * PHI_2, 2 * PHI_2],
                     [-PHI_M1, 0.0],
                     [0.5 * -PHI_M1, -PHI_M1]])
    assert np.allclose(lg, want, rtol=0, atol=1e-14)
    # the tanh approximation of GELU is about 1.5e-4 away at z = 1: the erf form is the one computed
    assert abs(lg[0, 0] - 0.5 * 2 * PHI_2 - 0.8411919906082768) > 1e-4


@pytest.mark.parametrize("T,H,E,k", [(4, 64, 16, 4), (3, 96, 10, 10), (2, 128, 64, 8)])
def test_warm_start_head_is_the_next_router(T, H, E, k):
    g = np.random.default_rng(T * 1000 + E)
    x = g.standard_normal((T, H)).astype(np.float32)
    R = (g.standard_normal((E, H)) * 0.05).astype(np.float32)
    hd = _zero_head(H, E, F=32)
    hd.w2[:] = g.standard_normal(hd.w2.shape)     # irrelevant: gelu(0) = 0 feeds it
    hd.wl[:, :H] = R
    cur, prev = _distinct_ids(g, T, E, k), _distinct_ids(g, T, E, k)
    idx, gate, lg = oracle.prerouter(x, hd, cur, prev, k)
    ridx, rgate = oracle.route(x, R, k)
    assert np.array_equal(lg, oracle.logits(x, R))
    assert np.array_equal(idx, ridx)
    assert np.array_equal(gate, rgate)


def test_khot_layout_current_then_previous():
    H, E, F, k = 32, 12, 32, 3
    hd = _zero_head(H, E, F)
    for e in range(E):
        hd.wl[e, H + e] = 1.0          # current routing
        hd.wl[e, H + E + e] = 2.0      # previous routing
    hd.b2 = (-1e-3 * np.arange(E)).astype(np.float32)
    x = np.zeros((1, H), np.float32)
    cur = np.array([[5, 1, 9]], np.int32)
    prev = np.array([[7, 1, 3]], np.int32)
    idx, _, lg = oracle.prerouter(x, hd, cur, prev, k)
    want = hd.b2.astype(np.float64)
    want[[5, 1, 9]] += 1.0
    want[[7, 1, 3]] += 2.0
    assert np.array_equal(lg[0], want)
    assert idx[0].tolist() == [1, 3, 7]           # 3 + b, then the previous-only ids by id
    idx, _, _ = oracle.prerouter(x, hd, cur, None, k)
    assert idx[0].tolist() == [1, 5, 9]           # no previous token: current ids only
    idx, _, _ = oracle.prerouter(x, hd, None, prev, k)
    assert idx[0].tolist() == [1, 3, 7]


def test_khot_features_reach_fc1():
    H, E, F, k = 32, 6, 2, 2
    hd = _zero_head(H, E, F)
    hd.w1[0, H + 4] = 1.0; hd.w1[0, H + E + 4] = 10.0   # 4 is current, not previous
    hd.w1[1, H + E + 5] = 1.0; hd.w1[1, H + 5] = 10.0   # 5 is previous, not current
    hd.w2[0, 0] = 1.0
    hd.w2[1, 1] = 2.0
    x = np.zeros((1, H), np.float32)
    _, _, lg = oracle.prerouter(x, hd, np.array([[4, 0]]), np.array([[2, 5]]), k)
    assert np.allclose(lg[0], [PHI_1, 2 * PHI_1, 0, 0, 0, 0], rtol=0, atol=1e-14)


def test_biases_enter_inside_and_outside_the_gelu():
    H, E, F = 32, 3, 2
    hd = _zero_head(H, E, F)
    hd.b1 = np.array([1.0, -1.0], np.float32)
    hd.w2[0] = [1.0, 0.0]
    hd.w2[1] = [0.0, 4.0]
    hd.b2 = np.array([0.25, 0.0, -0.5], np.float32)
    _, _, lg = oracle.prerouter(np.zeros((1, H), np.float32), hd, None, None, k=1)
    assert np.allclose(lg[0], [PHI_1 + 0.25, -4 * PHI_M1, -0.5], rtol=0, atol=1e-14)


@pytest.mark.parametrize("renorm", [True, False])
def test_top_k_and_gates_follow_the_router_rules(renorm):
    T, H, E, F, k = 6, 64, 32, 64, 5
    g = np.random.default_rng(11)
    hd = _head(H, E, F, seed=3, scale=3.0)
    x = g.standard_normal((T, H)).astype(np.float32)
    cur, prev = _distinct_ids(g, T, E, k), _distinct_ids(g, T, E, k)
    idx, gate, lg = oracle.prerouter(x, hd, cur, prev, k, flags=oracle.RENORM if renorm else 0)
    p = softmax(lg, axis=1)
    for t in range(T):
        l32 = lg[t].astype(np.float32)
        order = sorted(range(E), key=lambda e: (-l32[e], e))
        assert idx[t].tolist() == order[:k]
        want = p[t, idx[t]] / (p[t, idx[t]].sum() if renorm else 1.0)
        assert np.allclose(gate[t], want, rtol=1e-6, atol=1e-9)
    if renorm:
        assert np.allclose(gate.sum(axis=1), 1.0, atol=1e-6)


def test_low_precision_activations_are_upcast_exactly():
    T, H, E, F, k = 3, 64, 8, 32, 2
    g = np.random.default_rng(5)
    hd = _head(H, E, F, seed=5)
    x16 = g.standard_normal((T, H)).astype(np.float16)
    a = oracle.prerouter(x16, hd, None, None, k)
    b = oracle.prerouter(x16.astype(np.float32), hd, None, None, k)
    assert np.array_equal(a[2], b[2])


def test_out_of_range_ids_are_rejected():
    hd = _head(32, 4, 32)
    x = np.zeros((1, 32), np.float32)
    with pytest.raises(ValueError):
        oracle.prerouter(x, hd, np.array([[4]]), None, 1)
    with pytest.raises(ValueError):
        oracle.prerouter(x, hd, None, np.array([[-1]]), 1)


def test_empty_batch():
    hd = _head(32, 4, 32)
    idx, gate, lg = oracle.prerouter(np.zeros((0, 32), np.float32), hd, None, None, 2)
    assert idx.shape == (0, 2) and gate.shape == (0, 2) and lg.shape == (0, 4)
