"""Pins for the oracle's router and token-by-expert grouping.

Router: gate linear, softmax, top-k ("QwenのMoEルーターを観測してホットエキスパートを先読み
しても速くならなかった", section "ルーターをフックする"). The page's argpartition leaves
the k indices unordered; here they are ordered by descending logit with ties to
the lower expert id, and the k gates are renormalised to sum to one.
"""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _case(T, H, E, seed, std=0.05):
    g = np.random.default_rng(seed)
    return g.standard_normal((T, H)).astype(np.float32), (g.standard_normal((E, H)) * std).astype(np.float32)


def test_logits_one_hot_input_selects_router_column_exactly():
    _, R = _case(1, 64, 12, 0)
    for j in (0, 17, 63):
        x = np.zeros((1, 64), dtype=np.float32)
        x[0, j] = 1.0
        lg = oracle.logits(x, R)
        assert np.array_equal(lg[0], R[:, j].astype(np.float64))


def test_logits_match_numpy_fp64_matmul():
    x, R = _case(5, 256, 16, 1)
    lg = oracle.logits(x, R)
    ref = x.astype(np.float64) @ R.astype(np.float64).T
    assert np.allclose(lg, ref, rtol=1e-12, atol=1e-12)


def test_logits_fp16_and_bf16_inputs_are_upcast_exactly():
    x, R = _case(3, 64, 8, 2)
    x16 = x.astype(np.float16)
    assert np.allclose(oracle.logits(x16, R), x16.astype(np.float64) @ R.astype(np.float64).T, rtol=1e-12)
    import synth
    xb = synth.f32_to_bf16_bits(x)
    xbf = (xb.astype(np.uint32) << 16).view(np.float32)
    assert np.allclose(oracle.logits(xb, R, bf16=True), xbf.astype(np.float64) @ R.astype(np.float64).T, rtol=1e-12)


@pytest.mark.parametrize("E,k", [(6, 1), (6, 3), (8, 4), (8, 8)])
def test_topk_set_maximises_logit_sum_brute_force(E, k):
    x, R = _case(20, 32, E, 3 + E + k, std=0.5)
    idx, _ = oracle.route(x, R, k)
    lg = oracle.logits(x, R).astype(np.float32)
    for t in range(20):
        best = max(itertools.combinations(range(E), k), key=lambda c: (sum(float(lg[t, e]) for e in c), [-e for e in c]))
        assert sorted(idx[t].tolist()) == sorted(best)


def test_topk_order_matches_full_sort_by_logit_then_id():
    x, R = _case(50, 128, 32, 4)
    idx, _ = oracle.route(x, R, 6)
    lg = oracle.logits(x, R).astype(np.float32)
    for t in range(50):
        ref = sorted(range(32), key=lambda e: (-float(lg[t, e]), e))[:6]
        assert idx[t].tolist() == ref


def test_zero_input_ties_break_to_lowest_ids_with_equal_gates():
    _, R = _case(1, 64, 16, 5)
    x = np.zeros((2, 64), dtype=np.float32)
    idx, gate = oracle.route(x, R, 4)
    assert idx.tolist() == [[0, 1, 2, 3]] * 2
    assert np.array_equal(gate, np.full((2, 4), 0.25, dtype=np.float32))


def test_duplicate_router_rows_lower_id_first():
    x, R = _case(1, 64, 10, 6)
    lg = oracle.logits(x, R)[0]
    top = int(np.argmax(lg))
    R2 = R.copy()
    R2[9] = R[top]
    idx, gate = oracle.route(x, R2, 2)
    assert idx[0].tolist() == [min(top, 9), max(top, 9)]
    assert gate[0, 0] == gate[0, 1] == np.float32(0.5)


def test_k1_gate_is_exactly_one():
    x, R = _case(7, 64, 10, 7)
    _, gate = oracle.route(x, R, 1)
    assert (gate == 1.0).all()


def test_k_equals_E_without_renorm_is_the_sorted_softmax():
    x, R = _case(4, 64, 9, 8, std=0.3)
    idx, gate = oracle.route(x, R, 9, flags=0)
    p = softmax(oracle.logits(x, R), axis=1)
    for t in range(4):
        assert np.allclose(gate[t], p[t, idx[t]], rtol=1e-6, atol=1e-9)
        assert sorted(idx[t].tolist()) == list(range(9))


def test_renormalised_gates_sum_to_one_and_do_not_increase():
    x, R = _case(64, 256, 64, 9)
    idx, gate = oracle.route(x, R, 8)
    assert np.allclose(gate.astype(np.float64).sum(axis=1), 1.0, atol=1e-6)
    assert (np.diff(gate, axis=1) <= 0).all()
    idx0, gate0 = oracle.route(x, R, 8, flags=0)
    assert np.array_equal(idx, idx0)
    p = softmax(oracle.logits(x, R), axis=1)
    assert np.allclose(gate0, np.take_along_axis(p, idx.astype(np.int64), axis=1), rtol=1e-6)
    assert np.allclose(gate, gate0 / gate0.astype(np.float64).sum(axis=1, keepdims=True), rtol=1e-6)


def test_group_matches_sorted_by_expert_then_flat_id():
    g = np.random.default_rng(10)
    for T, k, E in [(1, 4, 16), (64, 10, 512), (37, 3, 8), (5, 5, 5)]:
        idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets, perm, uniq = oracle.group(idx, E)
        flat = idx.reshape(-1)
        ref = sorted(range(T * k), key=lambda f: (int(flat[f]), f))
        assert perm.tolist() == ref
        assert counts.tolist() == np.bincount(flat, minlength=E).tolist()
        assert offsets[0] == 0 and offsets[-1] == T * k and (np.diff(offsets) == counts).all()
        assert uniq.tolist() == sorted(set(flat.tolist()))


def test_group_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        oracle.group(np.array([[0, 16]], dtype=np.int32), 16)


def test_topk_on_given_logits_matches_the_router():
    """Top-k on handed-in logits is the router's step after its gate linear."""
    x, R = _case(6, 128, 40, 21)
    lg = oracle.logits(x, R).astype(np.float32)
    for flags in (0, oracle.RENORM):
        idx, gate = oracle.topk_logits(lg, 5, flags)
        ridx, rgate = oracle.route(x, R, 5, flags)
        assert np.array_equal(idx, ridx)
        assert np.allclose(gate, rgate, rtol=1e-6, atol=1e-7)
