"""Pins for the oracle's number formats: binary16 and bfloat16 conversions.

The fp16 scales of the block format (sym8, per-K-block-32 with fp16 scales) are
decoded and rounded by the oracle's own code; these tests hold it to numpy's and
torch's IEEE conversions, which are independent library routines.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_f16_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_bits_to_f32(int(b)) for b in bits], dtype=np.float32)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(ref) & (ref > 0))


def test_f16_round_to_nearest_even_matches_numpy_on_values_and_midpoints():
    # every finite fp16 value, and the exact midpoint to its upper neighbour (a tie)
    bits = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    nxt = np.append(vals[1:], 65536.0)
    mids = ((vals + nxt) / 2).astype(np.float32)   # exact in fp32 (fp16 has 11 significant bits)
    cases = np.concatenate([vals.astype(np.float32), mids, -mids,
                            np.random.default_rng(1).standard_normal(20000).astype(np.float32) * 1e-3,
                            np.array([65504, 65519.99, 65520, 1e6, 5.96e-8, 2.98e-8, 2.99e-8, 0.0, -0.0],
                                     dtype=np.float32)])
    ref = cases.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_bits(float(v)) for v in cases], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_f16_golden_patterns():
    # IEEE 754-2008 binary16 patterns worked by hand from the format definition
    with open(os.path.join(GOLDEN, "fp16_patterns.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert oracle.f32_to_f16_bits(float.fromhex(c["value"])) == int(c["bits"], 16), c
        if c.get("exact", True):
            assert oracle.f16_bits_to_f32(int(c["bits"], 16)) == float.fromhex(c["value"]), c


def test_bf16_decode_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([oracle.bf16_bits_to_f32(int(b)) for b in bits], dtype=np.float32)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
