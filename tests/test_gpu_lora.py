"""Parity of the HIP quantized linear with an unmerged LoRA delta against the
oracle, through the C ABI.

Contract: y within 1e-3 of the output norm per token (the layer's tolerance);
the delta on its own (y with the adapter minus y without) within 1e-3 of the
delta's norm per token, so the adapter's arithmetic is checked even where it is
small next to the base. Each side quantises the same fp32 draws with its own
quantiser (bit-exact with each other, see the quantiser tests).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_expert_quantized_amd as rq
import synth
from tests.cases import Y_REL_NORM, rel_norm_err
from tests.gpu_cases import to_dev_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rq.lib()  # raises if the HIP library is missing


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _draw(T, N, K, r, xtype, seed):
    g = synth.rng(seed, 91, 0, 0, 0)
    W = (g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    A = (g.standard_normal((r, K), dtype=np.float32) / np.float32(np.sqrt(K))).astype(np.float32)
    B = (g.standard_normal((N, r), dtype=np.float32) * np.float32(0.05)).astype(np.float32)
    x = synth.encode_x(synth.draw_x(g, T, K), xtype)
    return W, A, B, x


# T, N, K, r, codec, activations
CASES = [
    (1, 2048, 2048, 16, synth.SYM8, synth.F16),    # a d_model-wide projection at decode
    (1, 1024, 2048, 16, synth.INT4, synth.F16),
    (1, 301, 96, 3, synth.INT4, synth.F32),        # one token: ragged rows per workgroup, K below 256
    (1, 130, 4096, 64, synth.SYM8, synth.BF16),    # one token: largest K and r
    (7, 301, 96, 3, synth.INT4, synth.F32),        # rows not a multiple of 4, K below one 256 chunk
    (5, 130, 4096, 64, synth.SYM8, synth.BF16),    # largest K (two blocks per lane) and r
    (64, 512, 2048, 16, synth.INT4, synth.F16),    # a batch of fp16 tokens: matrix-core tiles
    (20, 77, 96, 5, synth.SYM8, synth.F16),        # matrix cores, ragged token and row tiles
    (16, 130, 4096, 64, synth.INT4, synth.F16),    # matrix cores, largest K and r
    (33, 64, 544, 0, synth.SYM8, synth.F16),       # matrix cores without the delta
    (40, 96, 256, 8, synth.INT4, synth.BF16),      # a bf16 batch: the matvec form
    (3, 77, 32, 1, synth.SYM8, synth.F32),         # one block per row, rank 1
    (2, 64, 544, 0, synth.INT4, synth.F16),        # r = 0: the plain quantized linear
]


@pytest.mark.parametrize("T,N,K,r,scheme,xtype", CASES)
def test_qlinear_lora_parity(T, N, K, r, scheme, xtype):
    say(f"qlinear+lora T={T} N={N} K={K} r={r} scheme={scheme} xtype={xtype}")
    W, A, B, x = _draw(T, N, K, r, xtype, seed=T + N + K + r)
    scale = 2.0
    codes, scales = rq.moe_quantize(torch.from_numpy(W).cuda(), scheme)
    qw = rq.QWeight(N, K, scheme, codes, scales)
    xd = to_dev_x(x, xtype)
    bf16 = xtype == synth.BF16
    if r:
        Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        y = rq.moe_qlinear_lora_forward(xd, qw, Ad, Bd, scale)
    y0 = rq.moe_qlinear_lora_forward(xd, qw, None, None, scale)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize(W, scheme)
    ref0 = oracle.qlinear_lora(x, rc, rs, scheme, None, None, scale, bf16=bf16)
    assert rel_norm_err(y0.cpu().numpy(), ref0) <= Y_REL_NORM
    if r:
        ref = oracle.qlinear_lora(x, rc, rs, scheme, A, B, scale, bf16=bf16)
        assert rel_norm_err(y.cpu().numpy(), ref) <= Y_REL_NORM
        d = y.cpu().numpy().astype(np.float64) - y0.cpu().numpy()
        assert rel_norm_err(d, ref.astype(np.float64) - ref0) <= Y_REL_NORM


def test_qlinear_lora_in_a_graph_replays():
    """Captured in a HIP graph and replayed with new activations in between."""
    T, N, K, r = 1, 1024, 2048, 16
    W, A, B, x = _draw(T, N, K, r, synth.F16, seed=5)
    codes, scales = rq.moe_quantize(torch.from_numpy(W).cuda(), synth.INT4)
    qw = rq.QWeight(N, K, synth.INT4, codes, scales)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    xd = to_dev_x(x, synth.F16)
    ws = rq.Workspace()
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    rq.moe_qlinear_lora_forward(xd, qw, Ad, Bd, 0.5, ws=ws, out=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rq.moe_qlinear_lora_forward(xd, qw, Ad, Bd, 0.5, ws=ws, out=y)
    rc, rs = oracle.quantize(W, synth.INT4)
    for step in range(3):
        say(f"qlinear+lora graph replay {step}")
        x2 = synth.encode_x(synth.draw_x(synth.rng(5, 91, 1, step), T, K), synth.F16)
        xd.copy_(to_dev_x(x2, synth.F16))
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.qlinear_lora(x2, rc, rs, synth.INT4, A, B, 0.5)
        assert rel_norm_err(y.cpu().numpy(), ref) <= Y_REL_NORM
