"""Pins for the oracle's gathered expert layer.

What is pinned ("鳴かぬなら、カスタムカーネル、ほととぎす", sections 4 and 7): only the
routed experts' weights are used; gate and up share the token; the down
projection of each slot takes that slot's own gated activation; the output is
the gate-weighted sum over the k slots ("QwenのMoEルーターを観測して…", section
"ルーターをフックする", for the routing). The pages print no worked values, so
the pins are closed forms of structured weights, invariants and special cases.
Each planted mistake must fail at least one of them.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
from tests.cases import rel_norm_err

F16 = np.float16


def _silu(z):
    return z * expit(z)  # library logistic function


def _structured(E, H, I, scheme, seed):
    """Experts whose every row has one nonzero code, so each projection reduces
    to a single product. Returns the packed experts and the closed-form pieces."""
    g = np.random.default_rng(seed)
    qmax = 127 if scheme == oracle.SYM8 else 7
    nbh, nbi = H // 32, I // 32
    cb = lambda K: K if scheme == oracle.SYM8 else K // 2
    wgu = np.zeros((E, 2 * I, cb(H)), np.uint8)
    sgu = np.zeros((E, 2 * I, nbh), np.uint16)
    wd = np.zeros((E, H, cb(I)), np.uint8)
    sd = np.zeros((E, H, nbi), np.uint16)
    spec = {"gcol": g.integers(0, H, (E, 2 * I)), "gcode": g.integers(1, qmax + 1, (E, 2 * I)) * g.choice([-1, 1], (E, 2 * I)),
            "gscale": 2.0 ** g.integers(-8, -3, (E, 2 * I, nbh)),
            "dcol": g.integers(0, I, (E, H)), "dcode": g.integers(1, qmax + 1, (E, H)) * g.choice([-1, 1], (E, H)),
            "dscale": 2.0 ** g.integers(-6, -1, (E, H, nbi))}

    def put(codes, row, col, code):
        if scheme == oracle.SYM8:
            codes[row][col] = np.uint8(code & 0xFF)
        else:
            b = codes[row][col // 2]
            nib = code & 0xF
            codes[row][col // 2] = (b & 0xF0) | nib if col % 2 == 0 else (b & 0x0F) | (nib << 4)

    for e in range(E):
        for r in range(2 * I):
            put(wgu[e], r, spec["gcol"][e, r], int(spec["gcode"][e, r]))
        for m in range(H):
            put(wd[e], m, spec["dcol"][e, m], int(spec["dcode"][e, m]))
    sgu[:] = spec["gscale"].astype(F16).view(np.uint16)
    sd[:] = spec["dscale"].astype(F16).view(np.uint16)
    return oracle.Experts(E, H, I, scheme, wgu, sgu, wd, sd), spec


def _closed_form(spec, x, idx, gate, H, I):
    """y by the closed form of structured experts, per token and slot."""
    T, k = idx.shape
    x = x.astype(np.float64)
    ys = np.zeros((T, k, H))
    for t in range(T):
        for s in range(k):
            e = idx[t, s]
            col, code = spec["gcol"][e], spec["gcode"][e]
            sc = spec["gscale"][e][np.arange(2 * I), col // 32]
            u = code * sc * x[t, col]
            h = _silu(u[:I]) * u[I:]
            dcol, dcode = spec["dcol"][e], spec["dcode"][e]
            dsc = spec["dscale"][e][np.arange(H), dcol // 32]
            ys[t, s] = dcode * dsc * h[dcol]
    y = (ys * gate.astype(np.float64)[..., None]).sum(axis=1) if gate is not None else ys
    return y


@pytest.mark.parametrize("scheme", [oracle.SYM8, oracle.INT4])
def test_structured_experts_match_closed_form(scheme):
    E, H, I, T, k = 5, 64, 64, 3, 3
    ex, spec = _structured(E, H, I, scheme, seed=1 + scheme)
    x = np.random.default_rng(2).standard_normal((T, H)).astype(np.float32)
    idx = np.array([[4, 0, 2], [1, 3, 0], [2, 4, 1]], dtype=np.int32)
    gate = np.array([[0.5, 0.3, 0.2], [0.6, 0.25, 0.15], [0.1, 0.2, 0.7]], dtype=np.float32)
    y = oracle.gather_forward(x, ex, idx, gate)
    assert np.allclose(y, _closed_form(spec, x, idx, gate, H, I), rtol=1e-6, atol=1e-7)
    ys = oracle.gather_forward(x, ex, idx, None)
    assert np.allclose(ys, _closed_form(spec, x, idx, None, H, I), rtol=1e-6, atol=1e-7)


def _random_experts(E, H, I, scheme, seed, std=0.02):
    g = np.random.default_rng(seed)
    wgu = (g.standard_normal((E, 2 * I, H)) * std).astype(np.float32)
    wd = (g.standard_normal((E, H, I)) * std).astype(np.float32)
    return oracle.quantize_experts(wgu, wd, scheme)


def test_dense_with_zeroed_gates_equals_gathered():
    E, H, I, T, k = 8, 64, 64, 4, 3
    ex = _random_experts(E, H, I, oracle.SYM8, 3)
    g = np.random.default_rng(4)
    x = g.standard_normal((T, H)).astype(np.float32)
    R = (g.standard_normal((E, H)) * 0.3).astype(np.float32)
    y, idx, gate = oracle.layer_forward(x, R, ex, k)
    full = np.zeros((T, E), np.float32)
    np.put_along_axis(full, idx.astype(np.int64), gate, axis=1)
    yd = oracle.dense_forward(x, ex, full)
    assert rel_norm_err(yd, y) < 1e-6


def test_result_does_not_depend_on_the_thread_count():
    """The oracle's loops split independent outputs only, so one thread and all
    threads give the same bits (the bench times it both ways)."""
    E, H, I, T, k = 8, 128, 64, 16, 3
    ex = _random_experts(E, H, I, oracle.INT4, 5)
    g = np.random.default_rng(6)
    x = g.standard_normal((T, H)).astype(np.float32)
    R = (g.standard_normal((E, H)) * 0.3).astype(np.float32)
    n = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        assert oracle.num_threads() == 1
        y1, i1, g1 = oracle.layer_forward(x, R, ex, k)
    finally:
        oracle.set_num_threads(n)
    assert oracle.num_threads() == n
    yn, i_n, gn = oracle.layer_forward(x, R, ex, k)
    assert np.array_equal(i1, i_n) and np.array_equal(g1, gn) and np.array_equal(y1, yn)


def test_identical_experts_give_the_single_expert_ffn():
    E, H, I, T = 6, 64, 32, 5
    one = _random_experts(1, H, I, oracle.INT4, 5)
    rep = lambda a: np.ascontiguousarray(np.repeat(a, E, axis=0))
    ex = oracle.Experts(E, H, I, oracle.INT4, rep(one.w_gate_up), rep(one.s_gate_up), rep(one.w_down), rep(one.s_down))
    g = np.random.default_rng(6)
    x = g.standard_normal((T, H)).astype(np.float32)
    R = (g.standard_normal((E, H)) * 0.3).astype(np.float32)
    y, _, _ = oracle.layer_forward(x, R, ex, 3)
    ffn = oracle.gather_forward(x, one, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32))
    assert rel_norm_err(y, ffn) < 1e-6


def test_expert_relabeling_permutes_indices_and_keeps_output():
    E, H, I, T, k = 8, 64, 32, 6, 3
    ex = _random_experts(E, H, I, oracle.SYM8, 7)
    g = np.random.default_rng(8)
    x = g.standard_normal((T, H)).astype(np.float32)
    R = (g.standard_normal((E, H)) * 0.3).astype(np.float32)
    y, idx, gate = oracle.layer_forward(x, R, ex, k)
    p = g.permutation(E)   # new id n holds old expert p[n]
    sel = lambda a: np.ascontiguousarray(a[p])
    ex2 = oracle.Experts(E, H, I, oracle.SYM8, sel(ex.w_gate_up), sel(ex.s_gate_up), sel(ex.w_down), sel(ex.s_down))
    y2, idx2, gate2 = oracle.layer_forward(x, np.ascontiguousarray(R[p]), ex2, k)
    assert np.array_equal(p[idx2], idx)
    assert np.allclose(gate2, gate, atol=1e-7)
    assert rel_norm_err(y2, y) < 1e-6


def test_doubling_down_scales_doubles_output_exactly():
    E, H, I, T, k = 4, 64, 64, 2, 2
    ex = _random_experts(E, H, I, oracle.SYM8, 9)
    x = np.random.default_rng(10).standard_normal((T, H)).astype(np.float32)
    idx = np.array([[1, 3], [0, 2]], np.int32)
    gate = np.array([[0.7, 0.3], [0.4, 0.6]], np.float32)
    y = oracle.gather_forward(x, ex, idx, gate)
    sd2 = (ex.s_down.view(F16).astype(np.float32) * 2).astype(F16).view(np.uint16)
    ex2 = oracle.Experts(E, H, I, ex.scheme, ex.w_gate_up, ex.s_gate_up, ex.w_down, np.ascontiguousarray(sd2))
    assert np.array_equal(oracle.gather_forward(x, ex2, idx, gate), y * 2)


def test_k1_layer_is_the_argmax_expert():
    E, H, I, T = 8, 64, 32, 4
    ex = _random_experts(E, H, I, oracle.SYM8, 11)
    g = np.random.default_rng(12)
    x = g.standard_normal((T, H)).astype(np.float32)
    R = (g.standard_normal((E, H)) * 0.3).astype(np.float32)
    y, idx, gate = oracle.layer_forward(x, R, ex, 1)
    am = np.argmax(oracle.logits(x, R), axis=1).astype(np.int32)[:, None]
    assert np.array_equal(idx, am) and (gate == 1).all()
    ffn = oracle.gather_forward(x, ex, am, None)[:, 0, :]
    assert np.array_equal(y, ffn)


def test_zero_gate_rows_give_zero_output():
    # every gate-half code zero -> silu(0) = 0 -> h = 0 -> y = 0
    E, H, I = 3, 64, 32
    ex = _random_experts(E, H, I, oracle.SYM8, 13)
    ex.w_gate_up[:, :I, :] = 0
    x = np.random.default_rng(14).standard_normal((2, H)).astype(np.float32)
    y = oracle.gather_forward(x, ex, np.array([[0, 1], [2, 0]], np.int32), np.full((2, 2), 0.5, np.float32))
    assert not y.any()


# ---------------------------------------------------------------------------
# Planted mistakes: each must fail a pin above and the parity tolerance.

def _pins_pass(scheme):
    E, H, I, T, k = 5, 64, 64, 3, 3
    ex, spec = _structured(E, H, I, scheme, seed=21 + scheme)
    x = np.random.default_rng(22).standard_normal((T, H)).astype(np.float32)
    idx = np.array([[4, 0, 2], [1, 3, 0], [2, 4, 1]], dtype=np.int32)
    gate = np.array([[0.5, 0.3, 0.2], [0.6, 0.25, 0.15], [0.1, 0.2, 0.7]], dtype=np.float32)
    y = oracle.gather_forward(x, ex, idx, gate)
    return rel_norm_err(y, _closed_form(spec, x, idx, gate, H, I)) < 1e-6


@pytest.mark.parametrize("mistake", [oracle.planted.SLOT0_ACTIVATION, oracle.planted.GATE_UP_SWAPPED,
                                     oracle.planted.GATES_IGNORED, oracle.planted.NIBBLE_SWAPPED,
                                     oracle.planted.SCALE_SHIFTED])
def test_planted_mistakes_fail_pins_and_tolerance(mistake):
    scheme = oracle.INT4 if mistake == oracle.planted.NIBBLE_SWAPPED else oracle.SYM8
    assert _pins_pass(scheme)
    E, H, I, T, k = 8, 128, 64, 4, 4
    ex = _random_experts(E, H, I, scheme, 30)
    g = np.random.default_rng(31)
    x = g.standard_normal((T, H)).astype(np.float32)
    R = (g.standard_normal((E, H)) * 0.3).astype(np.float32)
    y, idx, gate = oracle.layer_forward(x, R, ex, k)
    with oracle.planted(mistake):
        assert not _pins_pass(scheme)
        bad = oracle.gather_forward(x, ex, idx, gate)
    assert rel_norm_err(bad, y) > 1e-2
    assert _pins_pass(scheme)
