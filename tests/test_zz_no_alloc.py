"""moe_layer_forward_noalloc (the layer on the library's static device scratch)
against moe_layer_forward (the same kernels on a caller workspace), through the
C ABI: two calls in a row on one GPU, the second with a smaller input, each
bit-identical to the workspace entry point and within the oracle's tolerance."""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_expert_quantized_amd as rq
import synth
from tests.cases import GATE_ATOL, Y_REL_NORM, enforce_gap, rel_norm_err
from tests.gpu_cases import device_pool, oracle_compact, remap, to_dev_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rq.lib()


def _case(name, T, seed):
    w = synth.WORKLOADS[name]
    li = enforce_gap(w, synth.draw_layer(w, seed=seed, T=T, with_experts=False), seed=seed, layer=0)
    ridx, rgate = oracle.route(li.x, li.R, w.k, bf16=w.xtype == synth.BF16)
    used = np.unique(ridx)
    return w, li, ridx, rgate, used


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: 64 tokens of the batched int4 shape (grouped GEMM path, 7.5 MiB
    # of scratch); second call: one token of the decode shape (matvec path)
    for name, T, seed in (("batched_int4", 64, 41), ("decode40", 1, 42)):
        w, li, ridx, rgate, used = _case(name, T, seed)
        print(f"noalloc {name} T={T} E={w.E} k={w.k}", file=sys.stderr, flush=True)
        need = rq.moe_workspace_bytes(T, w.E, w.H, w.I, w.k, w.scheme)
        assert need <= rq.MOE_NOALLOC_SCRATCH_BYTES
        ex = device_pool(w, seed, 0, used)
        x = to_dev_x(li.x, w.xtype)
        R = torch.from_numpy(li.R).cuda()
        y_ws, idx_ws, gate_ws = rq.moe_layer_forward(x, R, ex, w.k)
        y = torch.full((T, w.H), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((T, w.k), -1, dtype=torch.int32, device="cuda")
        gate = torch.full((T, w.k), float("nan"), dtype=torch.float32, device="cuda")
        rq.moe_layer_forward_noalloc(x, R, ex, w.k, out=y, routing_out=(idx, gate))
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), idx_ws.cpu().numpy())
        assert np.array_equal(idx.cpu().numpy(), ridx)
        assert np.array_equal(gate.cpu().numpy(), gate_ws.cpu().numpy())
        assert np.abs(gate.cpu().numpy() - rgate).max() <= GATE_ATOL
        # the same kernels on the same inputs: identical bits
        assert np.array_equal(y.cpu().numpy(), y_ws.cpu().numpy())
        rex, m = oracle_compact(w, seed, 0, used)
        ref = oracle.gather_forward(li.x, rex, remap(ridx, m), rgate, bf16=w.xtype == synth.BF16)
        assert rel_norm_err(y.cpu().numpy(), ref) <= Y_REL_NORM


def test_noalloc_rejects_sizes_beyond_the_scratch():
    w = synth.WORKLOADS["prefill"]
    ex = rq.Experts(w.E, w.H, w.I, w.scheme, *(torch.zeros(16, dtype=torch.uint8, device="cuda") for _ in range(4)))
    x = torch.zeros((2048, w.H), dtype=torch.bfloat16, device="cuda")
    R = torch.zeros((w.E, w.H), dtype=torch.float32, device="cuda")
    with pytest.raises(rq.MoeError) as err:
        rq.moe_layer_forward_noalloc(x, R, ex, w.k)
    assert err.value.status == rq.MOE_ERR_WORKSPACE
