"""Parity of the HIP prerouter head against the oracle, through the C ABI.

Contract: indices bit-exact where the oracle's top k+1 head logits are at least
1e-3 apart (the inputs are redrawn until they are); gates within 1e-5 absolute;
head logits within 1e-4 of the token's largest |logit| (fp32 sums of up to
H + F + 2k terms on the GPU, erff for the GELU; fp64 in the oracle).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_expert_quantized_amd as rq
import synth
from tests.cases import GATE_ATOL, LOGIT_GAP, Y_REL_NORM, rel_inf_err, rel_norm_err
from tests.gpu_cases import to_dev_x

pytestmark = pytest.mark.gpu

HEAD_LOGIT_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rq.lib()  # raises if the HIP library is missing


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _gap_bad(lg: np.ndarray, k: int) -> np.ndarray:
    m = min(k + 1, lg.shape[1])
    top = -np.sort(-lg, axis=1)[:, :m]
    return np.nonzero((top[:, :-1] - top[:, 1:] < LOGIT_GAP).any(axis=1))[0]


def _case(T, H, E, F, k, xtype, seed, hist=True, bias=True):
    """Seeded head, activations and routing history, with every token's decision
    at least LOGIT_GAP clear in the oracle (failing tokens' activations are redrawn)."""
    wts = synth.draw_prerouter(seed, 90, 0, H, E, F, router_std=0.05, bias=bias)
    head = oracle.PrerouterHead(**wts)
    g = synth.rng(seed, 90, 0, 0, 1)
    x32 = synth.draw_x(g, T, H)
    cur = synth.draw_routing(g, T, E, k) if hist else None
    prev = synth.draw_routing(g, T, E, k) if hist else None
    bf16 = xtype == synth.BF16
    for attempt in range(64):
        x = synth.encode_x(x32, xtype)
        ref = oracle.prerouter(x, head, cur, prev, k, bf16=bf16)
        bad = _gap_bad(ref[2], k)
        if len(bad) == 0:
            return head, x, cur, prev, ref
        gg = synth.rng(seed, 90, 1 + attempt, 0, 1)
        x32[bad] = synth.draw_x(gg, len(bad), H)
    raise RuntimeError("logit gap not reached")


def _dev_head(head: oracle.PrerouterHead) -> rq.Prerouter:
    d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return rq.Prerouter(d(head.w1), d(head.b1), d(head.w2), d(head.b2), d(head.wl))


def _dev_ids(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _check(out, ref, k):
    idx, gate, lg = (t.cpu().numpy() for t in out)
    ridx, rgate, rlg = ref
    assert rel_inf_err(lg, rlg) <= HEAD_LOGIT_TOL, rel_inf_err(lg, rlg)
    assert np.array_equal(idx, ridx)
    assert np.abs(gate - rgate).max() <= GATE_ATOL


# name, T, H, E, F, k, xtype, with history, with biases
CASES = [
    ("decode", 1, 2048, 256, synth.PREROUTER_F, 8, synth.F16, True, True),   # the 35B-class shape, one token
    ("batched", 64, 2048, 256, synth.PREROUTER_F, 8, synth.F16, True, True),
    ("ragged", 7, 96, 10, 32, 3, synth.F32, True, True),      # H and F below one 256 chunk, E not a multiple of 64
    ("tail", 9, 800, 130, 288, 5, synth.BF16, True, False),  # ragged chunk tails, no biases
    ("first_token", 5, 256, 16, 64, 4, synth.F16, False, True),  # no routing history yet
    ("max", 3, 4096, 1024, 4096, 16, synth.BF16, True, True),  # largest H, E, F and k
    ("min", 2, 32, 2, 32, 1, synth.F32, True, True),
    ("four_tokens", 4, 512, 64, 96, 6, synth.F16, True, True),
    ("five_tokens", 5, 512, 64, 96, 6, synth.BF16, True, True),
    ("e96", 2, 256, 96, 256, 5, synth.F32, True, True),           # two logits per lane in the top-k
    ("wide_few", 1, 512, 64, 512, 4, synth.F16, True, True),      # one token, F over two 256 chunks
    ("many", 203, 256, 16, 64, 4, synth.BF16, True, True),        # matrix-core stage 1, ragged token tiles
    ("mid", 37, 384, 32, 64, 2, synth.F16, True, True),           # matrix-core stage 1
    ("ragged_batch", 20, 256, 10, 64, 3, synth.F16, True, True),  # matrix-core stage 1, E not a multiple of 16
    ("batched_f32", 16, 512, 64, 128, 4, synth.F32, False, False),  # matrix cores from fp32 input, no history
]


@pytest.mark.parametrize("name,T,H,E,F,k,xtype,hist,bias", CASES)
def test_prerouter_parity(name, T, H, E, F, k, xtype, hist, bias):
    say(f"prerouter {name}: T={T} H={H} E={E} F={F} k={k} xtype={xtype} hist={hist} bias={bias}")
    head, x, cur, prev, ref = _case(T, H, E, F, k, xtype, seed=T + E + F, hist=hist, bias=bias)
    out = rq.moe_prerouter_forward(to_dev_x(x, xtype), _dev_head(head), _dev_ids(cur), _dev_ids(prev), k,
                                   want_logits=True)
    torch.cuda.synchronize()
    _check(out, ref, k)


def test_prerouter_without_renorm_and_history_halves():
    T, H, E, F, k = 6, 512, 64, 128, 6
    head, x, cur, prev, _ = _case(T, H, E, F, k, synth.F16, seed=77)
    dh = _dev_head(head)
    xd = to_dev_x(x, synth.F16)
    for c, p in ((cur, None), (None, prev)):
        ref = oracle.prerouter(x, head, c, p, k, flags=0)
        if len(_gap_bad(ref[2], k)):
            continue  # this history half moves a decision inside the gap; the full-history case covers it
        say(f"prerouter renorm=0 cur={c is not None} prev={p is not None}")
        out = rq.moe_prerouter_forward(xd, dh, _dev_ids(c), _dev_ids(p), k, flags=0, want_logits=True)
        torch.cuda.synchronize()
        _check(out, ref, k)


def test_prerouter_warm_start_equals_router():
    """At warm start (fc1 = 0, residual path = [R 0 0]) the head is the router."""
    T, H, E, F, k = 16, 2048, 256, 256, 8
    w = synth.WORKLOADS["decode40"]
    from tests.cases import enforce_gap
    li = enforce_gap(w, synth.draw_layer(w, seed=4, T=T, with_experts=False), seed=4, layer=0)
    R = li.R
    D = H + 2 * E
    head = oracle.PrerouterHead(w1=np.zeros((F, D), np.float32), b1=None,
                                w2=synth.draw_router(synth.rng(4, 90, 0), E, F, 0.1), b2=None,
                                wl=np.concatenate([R, np.zeros((E, 2 * E), np.float32)], axis=1))
    say("prerouter warm start vs router")
    xd = to_dev_x(li.x, w.xtype)
    g = synth.rng(4, 90, 0, 0, 3)
    cur, prev = synth.draw_routing(g, T, E, k), synth.draw_routing(g, T, E, k)
    idx, gate = rq.moe_prerouter_forward(xd, _dev_head(head), _dev_ids(cur), _dev_ids(prev), k)
    ridx, rgate = rq.moe_route(xd, torch.from_numpy(R).cuda(), k)
    torch.cuda.synchronize()
    oidx, ogate = oracle.route(li.x, R, k)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.array_equal(ridx.cpu().numpy(), oidx)
    assert np.abs(gate.cpu().numpy() - ogate).max() <= GATE_ATOL


def test_predicted_routing_drives_the_expert_layer():
    """Prediction as routing: the head's top-k and gates go straight into the
    gathered expert layer of the next layer (the routed experts only)."""
    T, H, E, F, k, I = 4, 512, 64, 128, 6, 128
    head, x, cur, prev, ref = _case(T, H, E, F, k, synth.F16, seed=21)
    say("prerouter -> gather_qmm")
    g = np.random.default_rng(21)
    wgu = (g.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    wd = (g.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    ex = rq.quantize_experts(torch.from_numpy(wgu).cuda(), torch.from_numpy(wd).cuda(), rq.MOE_Q_SYM8)
    xd = to_dev_x(x, synth.F16)
    idx, gate = rq.moe_prerouter_forward(xd, _dev_head(head), _dev_ids(cur), _dev_ids(prev), k)
    y = rq.moe_gather_qmm_forward(xd, ex, idx, gate)
    torch.cuda.synchronize()
    rex = oracle.quantize_experts(wgu, wd, rq.MOE_Q_SYM8)
    yref = oracle.gather_forward(x, rex, ref[0], ref[1])
    assert np.array_equal(idx.cpu().numpy(), ref[0])
    assert rel_norm_err(y.cpu().numpy(), yref) <= Y_REL_NORM


@pytest.mark.parametrize("T,path", [(1, "auto"), (1, "gemm"), (3, "auto"), (40, "auto"), (40, "gather")])
def test_head_logits_drive_experts_from_logits(T, path):
    """The head stops at its logits and the next layer's expert call takes the
    top-k itself (inside the gate/up kernel for one token)."""
    H, E, F, k, I = 512, 64, 128, 6, 128
    head, x, cur, prev, ref = _case(T, H, E, F, k, synth.F16, seed=31 + T)
    say(f"prerouter logits -> experts_from_logits T={T} path={path}")
    g = np.random.default_rng(31 + T)
    wgu = (g.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    wd = (g.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    ex = rq.quantize_experts(torch.from_numpy(wgu).cuda(), torch.from_numpy(wd).cuda(), rq.MOE_Q_INT4)
    xd = to_dev_x(x, synth.F16)
    lg = rq.moe_prerouter_forward(xd, _dev_head(head), _dev_ids(cur), _dev_ids(prev), k, topk=False)
    fl = rq.MOE_FLAG_RENORM | {"auto": 0, "gemm": rq.MOE_FLAG_PATH_GEMM, "gather": rq.MOE_FLAG_PATH_GATHER}[path]
    y, idx, gate = rq.moe_experts_from_logits(xd, lg, ex, k, flags=fl, return_routing=True)
    torch.cuda.synchronize()
    assert rel_inf_err(lg.cpu().numpy(), ref[2]) <= HEAD_LOGIT_TOL
    assert np.array_equal(idx.cpu().numpy(), ref[0])
    assert np.abs(gate.cpu().numpy() - ref[1]).max() <= GATE_ATOL
    rex = oracle.quantize_experts(wgu, wd, rq.MOE_Q_INT4)
    yref = oracle.gather_forward(x, rex, ref[0], ref[1])
    assert rel_norm_err(y.cpu().numpy(), yref) <= Y_REL_NORM


# T, codec, activations, I, F: the first four run fused (head rows inside the
# expert launches); I = 2048, F = 2048 and T = 3 take the call-after-call path
PREROUTED = [(1, synth.SYM8, synth.F16, 512, 256), (1, synth.INT4, synth.F16, 256, 96),
             (1, synth.SYM8, synth.BF16, 128, 128), (1, synth.INT4, synth.F32, 1024, 1024),
             (1, synth.SYM8, synth.F16, 2048, 128), (1, synth.INT4, synth.F16, 128, 2048),
             (3, synth.SYM8, synth.F16, 128, 128)]


@pytest.mark.parametrize("T,scheme,xtype,I,F", PREROUTED)
def test_prerouted_layer(T, scheme, xtype, I, F):
    """One prerouted decode layer: experts on the predicted logits, and the next
    layer's head on this layer's input and routing."""
    H, E, k = 512, 64, 6
    say(f"prerouted layer T={T} scheme={scheme} xtype={xtype} I={I} F={F}")
    head, x, _, prev, _ = _case(T, H, E, F, k, xtype, seed=50 + I + F + T)
    g = np.random.default_rng(50 + I + F)
    logits = (g.standard_normal((T, E)) * 2.0).astype(np.float32)   # predicted for this layer
    wgu = (g.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    wd = (g.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    ex = rq.quantize_experts(torch.from_numpy(wgu).cuda(), torch.from_numpy(wd).cuda(), scheme)
    xd = to_dev_x(x, xtype)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    nxt = torch.empty((T, E), dtype=torch.float32, device="cuda")
    y = rq.moe_prerouted_layer_forward(xd, torch.from_numpy(logits).cuda(), ex, k, _dev_head(head), _dev_ids(prev), idx,
                                       nxt, gate_out=gate)
    y_last = rq.moe_prerouted_layer_forward(xd, torch.from_numpy(logits).cuda(), ex, k, None, None, idx, None)
    torch.cuda.synchronize()
    bf16 = xtype == synth.BF16
    ridx, rgate = oracle.topk_logits(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(gate.cpu().numpy() - rgate).max() <= GATE_ATOL
    rex = oracle.quantize_experts(wgu, wd, scheme)
    yref = oracle.gather_forward(x, rex, ridx, rgate, bf16=bf16)
    assert rel_norm_err(y.cpu().numpy(), yref) <= Y_REL_NORM
    assert rel_norm_err(y_last.cpu().numpy(), yref) <= Y_REL_NORM
    nref = oracle.prerouter(x, head, ridx, prev, k, bf16=bf16)[2]
    assert rel_inf_err(nxt.cpu().numpy(), nref) <= HEAD_LOGIT_TOL


@pytest.mark.parametrize("T", [3, 16, 64])
def test_prerouter_with_contiguous_fc1_and_residual(T):
    """fc1's and the residual path's rows in one allocation (one matrix-core
    launch for a batch)."""
    H, E, F, k = 512, 64, 96, 6
    say(f"prerouter contiguous weights T={T}")
    head, x, cur, prev, ref = _case(T, H, E, F, k, synth.F16, seed=60 + T)
    D = H + 2 * E
    w1l = torch.from_numpy(np.concatenate([head.w1.ravel(), head.wl.ravel()])).cuda()
    dh = rq.Prerouter(w1l[:F * D].view(F, D), torch.from_numpy(head.b1).cuda(), torch.from_numpy(head.w2).cuda(),
                      torch.from_numpy(head.b2).cuda(), w1l[F * D:].view(E, D))
    out = rq.moe_prerouter_forward(to_dev_x(x, synth.F16), dh, _dev_ids(cur), _dev_ids(prev), k, want_logits=True)
    torch.cuda.synchronize()
    _check(out, ref, k)


def test_prerouted_layer_at_the_large_shape():
    """The fused prerouted layer at H = 4096, E = 512, top-10, I = 1024 (two
    code blocks per lane, eight logits per lane in the top-k, four hidden chunks
    per head wave). Only the routed experts hold weights; the rest have NaN
    scales, so a read of any other expert would show in y."""
    from tests.gpu_cases import device_pool, oracle_compact, remap
    w = synth.Workload("prerouted_large", T=1, H=4096, E=512, k=10, I=1024, scheme=synth.INT4, xtype=synth.F16)
    F = synth.PREROUTER_F
    say("prerouted layer at H=4096 E=512 k=10 I=1024")
    head, x, _, prev, _ = _case(1, w.H, w.E, F, w.k, w.xtype, seed=71)
    g = np.random.default_rng(71)
    logits = (g.standard_normal((1, w.E)) * 2.0).astype(np.float32)
    ridx, rgate = oracle.topk_logits(logits, w.k)
    used = np.unique(ridx)
    ex = device_pool(w, 71, 0, used)
    rex, m = oracle_compact(w, 71, 0, used)
    xd = to_dev_x(x, w.xtype)
    idx = torch.empty((1, w.k), dtype=torch.int32, device="cuda")
    nxt = torch.empty((1, w.E), dtype=torch.float32, device="cuda")
    y = rq.moe_prerouted_layer_forward(xd, torch.from_numpy(logits).cuda(), ex, w.k, _dev_head(head), _dev_ids(prev),
                                       idx, nxt)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ridx)
    yref = oracle.gather_forward(x, rex, remap(ridx, m), rgate)
    assert rel_norm_err(y.cpu().numpy(), yref) <= Y_REL_NORM
    nref = oracle.prerouter(x, head, ridx, prev, w.k)[2]
    assert rel_inf_err(nxt.cpu().numpy(), nref) <= HEAD_LOGIT_TOL
