"""Pins for the oracle's block quantiser and dequantiser.

Codec: symmetric linear int8 with one scale per 32 consecutive K elements of a
row ("鳴かぬなら、カスタムカーネル、ほととぎす", section 6), and its 4-bit analogue
(same page, sections 3 and 7). Packed layout: per expert, per output row,
K-contiguous codes (section 4 of the same page: QP is [E, N, K/4] int8 words).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
QMAX = {oracle.SYM8: 127, oracle.INT4: 7}


def _codes(codes, scheme, K):
    """Signed codes [rows][K] from packed bytes, by the layout definition."""
    if scheme == oracle.SYM8:
        return codes.view(np.int8).astype(np.int32).reshape(-1, K)
    c = codes.reshape(-1, K // 2).astype(np.int32)
    lo, hi = c & 0xF, c >> 4
    out = np.empty((c.shape[0], K), dtype=np.int32)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out)


def _draw(rows, K, std=0.02, seed=0):
    return (np.random.default_rng(seed).standard_normal((rows, K)) * std).astype(np.float32)


@pytest.mark.parametrize("scheme", [oracle.SYM8, oracle.INT4])
def test_codes_in_range_and_block_max_hits_qmax(scheme):
    w = _draw(64, 256)
    codes, scales = oracle.quantize(w, scheme)
    q = _codes(codes, scheme, 256)
    qmax = QMAX[scheme]
    assert np.abs(q).max() <= qmax
    blocks = np.abs(w).reshape(64, 8, 32)
    at_max = blocks.argmax(axis=2)
    qb = q.reshape(64, 8, 32)
    hit = np.take_along_axis(np.abs(qb), at_max[..., None], axis=2)[..., 0]
    assert (hit == qmax).all()


@pytest.mark.parametrize("scheme", [oracle.SYM8, oracle.INT4])
def test_scale_is_fp16_of_block_amax_over_qmax(scheme):
    # numpy's fp16 conversion is an independent RNE implementation
    w = _draw(32, 128, seed=3)
    _, scales = oracle.quantize(w, scheme)
    amax = np.abs(w).reshape(32, 4, 32).max(axis=2)
    ref = (amax / np.float32(QMAX[scheme])).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(scales, ref)


@pytest.mark.parametrize("scheme", [oracle.SYM8, oracle.INT4])
def test_reconstruction_error_within_half_step(scheme):
    w = _draw(128, 512, seed=5)
    codes, scales = oracle.quantize(w, scheme)
    deq = oracle.dequantize(codes, scales, 512, scheme)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
    err = np.abs(deq.astype(np.float64) - w.astype(np.float64))
    assert (err <= s / 2 * (1 + 1e-6) + 1e-12).all()
    # dequantisation is exactly code * scale
    assert np.array_equal(deq.astype(np.float64), _codes(codes, scheme, 512) * s)


@pytest.mark.parametrize("scheme", [oracle.SYM8, oracle.INT4])
def test_sign_symmetry_and_power_of_two_scaling(scheme):
    w = _draw(16, 64, seed=7)
    c1, s1 = oracle.quantize(w, scheme)
    c2, s2 = oracle.quantize(-w, scheme)
    assert np.array_equal(_codes(c2, scheme, 64), -_codes(c1, scheme, 64))
    assert np.array_equal(s1, s2)
    c3, s3 = oracle.quantize(w * 4, scheme)
    assert np.array_equal(_codes(c3, scheme, 64), _codes(c1, scheme, 64))
    assert np.array_equal(s3.view(np.float16).astype(np.float32), s1.view(np.float16).astype(np.float32) * 4)


def test_zero_block_gives_zero_scale_and_codes():
    w = np.zeros((2, 64), dtype=np.float32)
    w[1, 32:] = 0.5
    codes, scales = oracle.quantize(w, oracle.SYM8)
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and scales[1, 0] == 0
    assert not codes[0].any() and not codes[1, :32].any()
    assert (codes[1, 32:].view(np.int8) == 127).all()


def test_golden_packed_bytes():
    """Byte layout worked by hand: sym8 bytes are two's-complement codes in K
    order; int4 packs two codes a byte, the even K index in the low nibble."""
    with open(os.path.join(GOLDEN, "quant_packing.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        w = np.array([float.fromhex(v) for v in case["w"]], dtype=np.float32)[None, :]
        scheme = oracle.SYM8 if case["scheme"] == "sym8" else oracle.INT4
        codes, scales = oracle.quantize(w, scheme)
        assert [int(b) for b in codes[0]] == [int(b, 16) for b in case["bytes"]], case["name"]
        assert int(scales[0, 0]) == int(case["scale_bits"], 16), case["name"]


def test_nearest_code_property_against_brute_force():
    """Each code is a nearest point of the grid {-qmax..qmax} * s to w (ties aside)."""
    w = _draw(8, 64, seed=11)
    for scheme in (oracle.SYM8, oracle.INT4):
        codes, scales = oracle.quantize(w, scheme)
        q = _codes(codes, scheme, 64).astype(np.float64)
        s = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
        grid = np.arange(-QMAX[scheme], QMAX[scheme] + 1, dtype=np.float64)
        best = np.abs(w[..., None].astype(np.float64) - grid * s[..., None]).min(axis=-1)
        mine = np.abs(w.astype(np.float64) - q * s)
        assert (mine <= best + s * 1e-6).all()
