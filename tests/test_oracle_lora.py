"""Pins for the oracle's quantized linear with an unmerged LoRA delta.

"The Other Half of the Memory Wall: Serving 35B MoEs from SSD with Trained Routing
Prediction" (xyznot.com), section 手法 (method), "非マージアダプターの実行": the layer
keeps its quantized base weights and runs the low-rank delta beside them,
y = W_int4 x + (alpha / r) B A x. Section よくある質問 (FAQ): the delta's RMS (about
1e-3) is below the 4-bit quantisation step, so merging it into the weights and
re-quantising loses most of it, while the unmerged delta keeps all of it.

What pins each part:
  - hand-worked values on 32-column rows in both codecs (sums of small integers,
    exact in fp32), with an asymmetric A and B, for the base, the delta and the
    scale;
  - the merge identity: the unmerged y equals x times the merged fp64 matrix
    dequant(W) + scale B A, computed by numpy in another order;
  - the reduction to the plain quantized linear when B = 0, scale = 0 or r = 0;
  - the page's reason for not merging, as a property of the block quantiser.
"""
import numpy as np
import pytest

import oracle

F16_ONE, F16_HALF = 0x3C00, 0x3800


def _hand_codes(scheme):
    """Row 0: every code 1 at scale 0.5. Row 1: sym8 codes i - 16 at scale 1;
    int4 codes alternating +7, -7 at scale 1."""
    if scheme == oracle.SYM8:
        codes = np.empty((2, 32), np.uint8)
        codes[0] = 1
        codes[1] = (np.arange(32) - 16).astype(np.int8).view(np.uint8)
    else:
        codes = np.empty((2, 16), np.uint8)
        codes[0] = 0x11
        codes[1] = 0x97          # low nibble +7 (even index), high nibble -7 (odd index)
    scales = np.array([[F16_HALF], [F16_ONE]], np.uint16)
    return codes, scales


def test_hand_worked_sym8():
    codes, scales = _hand_codes(oracle.SYM8)
    x = np.stack([np.ones(32), np.arange(32)]).astype(np.float32)
    A = np.zeros((2, 32), np.float32)
    A[0, :] = 1.0 / 32
    A[1, 3] = 1.0
    B = np.array([[2.0, 0.0], [-1.0, 1.0]], np.float32)
    # base: token 0 -> [0.5 * 32, sum(i - 16)] = [16, -16]; token 1 -> [0.5 * 496, sum i(i - 16)] = [248, 2480]
    # u = A x: token 0 -> [1, 1]; token 1 -> [15.5, 3]
    # delta = 0.5 * B u: token 0 -> [1, 0]; token 1 -> [15.5, -6.25]
    y = oracle.qlinear_lora(x, codes, scales, oracle.SYM8, A, B, 0.5)
    assert np.array_equal(y, np.array([[17.0, -16.0], [263.5, 2473.75]], np.float32))
    y0 = oracle.qlinear_lora(x, codes, scales, oracle.SYM8, None, None, 0.5)
    assert np.array_equal(y0, np.array([[16.0, -16.0], [248.0, 2480.0]], np.float32))


def test_hand_worked_int4():
    codes, scales = _hand_codes(oracle.INT4)
    x = np.stack([np.ones(32), np.arange(32)]).astype(np.float32)
    A = np.zeros((1, 32), np.float32)
    A[0, 0] = 1.0
    A[0, 1] = -1.0
    B = np.array([[4.0], [1.0]], np.float32)
    # base: token 0 -> [16, 16*7 - 16*7 = 0]; token 1 -> [248, 7 * sum(even i) - 7 * sum(odd i) = 7 * (240 - 256) = -112]
    # u: token 0 -> 0; token 1 -> 0 - 1 = -1; delta = 0.25 * B u
    y = oracle.qlinear_lora(x, codes, scales, oracle.INT4, A, B, 0.25)
    assert np.array_equal(y, np.array([[16.0, 0.0], [247.0, -112.25]], np.float32))


@pytest.mark.parametrize("scheme", [oracle.SYM8, oracle.INT4])
def test_unmerged_equals_the_merged_matrix(scheme):
    g = np.random.default_rng(7 + scheme)
    T, N, K, r = 5, 48, 96, 8
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, scales = oracle.quantize(W, scheme)
    A = (g.standard_normal((r, K)) * 0.1).astype(np.float32)
    B = (g.standard_normal((N, r)) * 0.1).astype(np.float32)
    x = g.standard_normal((T, K)).astype(np.float32)
    scale = 16.0 / r
    y = oracle.qlinear_lora(x, codes, scales, scheme, A, B, scale)
    Wm = oracle.dequantize(codes, scales, K, scheme).astype(np.float64) + scale * (B.astype(np.float64) @ A)
    ref = x.astype(np.float64) @ Wm.T
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("scheme", [oracle.SYM8, oracle.INT4])
def test_reduces_to_the_quantized_linear(scheme):
    g = np.random.default_rng(11 + scheme)
    T, N, K, r = 3, 20, 64, 4
    codes, scales = oracle.quantize((g.standard_normal((N, K)) * 0.02).astype(np.float32), scheme)
    x = g.standard_normal((T, K)).astype(np.float32)
    A = g.standard_normal((r, K)).astype(np.float32)
    base = oracle.qlinear_lora(x, codes, scales, scheme, None, None, 1.0)
    assert np.array_equal(oracle.qlinear_lora(x, codes, scales, scheme, A, np.zeros((N, r), np.float32), 2.0), base)
    assert np.array_equal(oracle.qlinear_lora(x, codes, scales, scheme, A, g.standard_normal((N, r)).astype(np.float32),
                                              0.0), base)
    ref = x.astype(np.float64) @ oracle.dequantize(codes, scales, K, scheme).astype(np.float64).T
    assert np.allclose(base, ref, rtol=1e-6, atol=1e-7)


def test_merging_a_small_delta_into_int4_loses_most_of_it():
    """The FAQ's reason for keeping the adapter unmerged: a delta of RMS ~1e-3 is
    below the int4 step of weights of std 0.02, so the change that re-quantising
    the merged weights makes is mostly rounding noise (its error exceeds the
    delta itself), while the unmerged path reproduces the delta."""
    g = np.random.default_rng(3)
    N, K, r, T = 256, 512, 16, 4
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = (g.standard_normal((r, K)) / np.sqrt(K)).astype(np.float32)
    B = (g.standard_normal((N, r)) / np.sqrt(r)).astype(np.float32)
    scale = 1e-3 * np.sqrt(K)   # B A has entries of RMS 1/sqrt(K)
    delta = scale * (B.astype(np.float64) @ A)
    assert 0.5e-3 < np.sqrt(np.mean(delta ** 2)) < 2e-3
    q0 = oracle.quantize(W, oracle.INT4)
    q1 = oracle.quantize((W + delta).astype(np.float32), oracle.INT4)
    d0 = oracle.dequantize(*q0, K, oracle.INT4).astype(np.float64)
    d1 = oracle.dequantize(*q1, K, oracle.INT4).astype(np.float64)
    x = g.standard_normal((T, K)).astype(np.float32)
    xd = x.astype(np.float64)
    merged_err = np.linalg.norm(xd @ (d1 - d0).T - xd @ delta.T) / np.linalg.norm(xd @ delta.T)
    assert merged_err > 1.0
    kept = oracle.qlinear_lora(x, *q0, oracle.INT4, A, B, scale) - oracle.qlinear_lora(x, *q0, oracle.INT4, None, None,
                                                                                        scale)
    want = x.astype(np.float64) @ delta.T
    assert np.allclose(kept, want, rtol=1e-3, atol=2e-6)


def test_bad_arguments():
    codes, scales = _hand_codes(oracle.SYM8)
    with pytest.raises(ValueError):
        oracle.qlinear_lora(np.ones((1, 32), np.float32), codes, scales, 5, None, None, 1.0)
