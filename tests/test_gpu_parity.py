"""Parity of the HIP path against the oracle, element by element, through the C ABI.

Contract: router indices and grouping bit-exact; quantiser codes and scales
bit-exact; gates within 1e-5 absolute; layer outputs within 1e-3 of the
output norm per token (fp32 accumulation on the GPU, fp64 in the oracle).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_expert_quantized_amd as rq
import synth
from tests.cases import GATE_ATOL, Y_REL_NORM, enforce_gap, rel_inf_err, rel_norm_err
from tests.gpu_cases import NAN_F16, device_pool, oracle_compact, remap, to_dev_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rq.lib()  # raises if the HIP library is missing


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- quantiser
@pytest.mark.parametrize("scheme", [rq.MOE_Q_SYM8, rq.MOE_Q_INT4])
def test_quantize_bit_exact(scheme):
    g = np.random.default_rng(100 + scheme)
    w = (g.standard_normal((300, 512)) * 0.02).astype(np.float32)
    w[0] = 0.0                              # zero blocks: scale 0, codes 0
    w[1, :32] = 1e-9                        # scale underflows to a subnormal / zero
    w[2] = g.standard_normal(512).astype(np.float32) * 1e4   # large values
    w[3, :32] = np.arange(32, dtype=np.float32) - 16          # exact grid with ties
    w[4, :32] = 70000.0 * 127               # scale saturates at 65504
    codes, scales = rq.moe_quantize(torch.from_numpy(w).cuda(), scheme)
    rc, rs = oracle.quantize(w, scheme)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), rs)


# ---------------------------------------------------------------- router
# prefill at T >= 128 takes the split-weight bf16 router (T = 128 is the first such batch)
ROUTE_CASES = [("tiny", None), ("decode40", None), ("batched_int4", None), ("large_int4", None),
               ("prefill", None), ("prefill", 130), ("prefill", 128), ("prefill", 127), ("batched_int4", 3)]


@pytest.mark.parametrize("name,T", ROUTE_CASES)
@pytest.mark.parametrize("renorm", [True, False])
def test_route_parity(name, T, renorm):
    w = synth.WORKLOADS[name]
    li = enforce_gap(w, synth.draw_layer(w, seed=0, T=T, with_experts=False), seed=0, layer=0)
    say(f"route {name} T={li.x.shape[0]} renorm={renorm}")
    flags = rq.MOE_FLAG_RENORM if renorm else 0
    idx, gate = rq.moe_route(to_dev_x(li.x, w.xtype), torch.from_numpy(li.R).cuda(), w.k, flags)
    ridx, rgate = oracle.route(li.x, li.R, w.k, flags=oracle.RENORM if renorm else 0, bf16=w.xtype == synth.BF16)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(gate.cpu().numpy() - rgate).max() <= GATE_ATOL


# bf16 batches with at least 256 tiles of 128 tokens x 64 experts take the
# split-weight router's wide tile; ragged T and E included
@pytest.mark.parametrize("T,E,H,k", [(8300, 200, 256, 8), (8192, 256, 512, 6)])
def test_route_split_weight_wide_tiles(T, E, H, k):
    g = np.random.default_rng(T + E)
    x32 = g.standard_normal((T, H)).astype(np.float32)
    R = (g.standard_normal((E, H)) * H ** -0.5).astype(np.float32)
    w = synth.Workload("adhoc", T=T, H=H, E=E, k=k, I=32, scheme=0, xtype=synth.BF16)
    li = enforce_gap(w, synth.LayerInputs(x32, synth.encode_x(x32, synth.BF16), R, None, None), seed=5, layer=E)
    say(f"route wide tiles T={T} E={E} H={H} k={k}")
    idx, gate = rq.moe_route(to_dev_x(li.x, w.xtype), torch.from_numpy(li.R).cuda(), k, rq.MOE_FLAG_RENORM)
    ridx, rgate = oracle.route(li.x, li.R, k, flags=oracle.RENORM, bf16=True)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(gate.cpu().numpy() - rgate).max() <= GATE_ATOL


def test_route_many_experts_and_max_k():
    g = np.random.default_rng(7)
    for T, H, E, k in [(5, 256, 1000, 16), (2, 64, 1024, 3), (4, 32, 16, 16), (1, 4096, 64, 1)]:
        x = g.standard_normal((T, H)).astype(np.float32)
        R = (g.standard_normal((E, H)) * 0.3).astype(np.float32)
        w = synth.Workload("adhoc", T=T, H=H, E=E, k=k, I=32, scheme=0, xtype=synth.F32)
        li = enforce_gap(w, synth.LayerInputs(x, x.copy(), R, None, None), seed=7, layer=T)
        idx, gate = rq.moe_route(torch.from_numpy(li.x).cuda(), torch.from_numpy(R).cuda(), k)
        ridx, rgate = oracle.route(li.x, R, k)
        assert np.array_equal(idx.cpu().numpy(), ridx), (T, H, E, k)
        assert np.abs(gate.cpu().numpy() - rgate).max() <= GATE_ATOL


@pytest.mark.parametrize("E,k", [(16, 4), (256, 8), (64, 16), (512, 10), (1000, 10)])
def test_route_exact_ties_go_to_lower_ids(E, k):
    g = np.random.default_rng(E + k)
    R = (g.standard_normal((E, 64)) * 0.3).astype(np.float32)
    # all-zero activations: every logit is 0, so the first k ids win with equal gates
    idx, gate = rq.moe_route(torch.zeros((3, 64), device="cuda"), torch.from_numpy(R).cuda(), k)
    assert (idx.cpu().numpy() == np.arange(k)).all()
    assert np.allclose(gate.cpu().numpy(), 1.0 / k, atol=GATE_ATOL)
    # duplicated router rows: equal logits, the lower id first
    x = g.standard_normal((4, 64)).astype(np.float32)
    R2 = R.copy()
    R2[E - 1] = R2[E // 2]
    R2[E - 2] = R2[1]
    ridx, rgate = oracle.route(x, R2, k)
    gi, gg = rq.moe_route(torch.from_numpy(x).cuda(), torch.from_numpy(R2).cuda(), k)
    assert np.array_equal(gi.cpu().numpy(), ridx)
    assert np.abs(gg.cpu().numpy() - rgate).max() <= GATE_ATOL


# ---------------------------------------------------------------- grouping
@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (63, 10, 512), (64, 10, 512), (65, 3, 8), (16, 10, 512),
                                   (2048, 8, 256), (300, 16, 1024), (5, 4, 4),
                                   # chunk masks beyond the one-workgroup form's LDS: three kernels,
                                   # the scan splitting each expert's chunks over 1, 4, 3 (unevenly) and 2 threads
                                   (2048, 4, 1024), (520, 2, 1024), (8192, 8, 256), (2000, 3, 300), (1100, 5, 512)])
def test_group_bit_exact(T, k, E):
    g = np.random.default_rng(T * 31 + k)
    idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, uniq, n = rq.moe_group(torch.from_numpy(idx).cuda(), E)
    rc, ro, rp, ru = oracle.group(idx, E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(perm.cpu().numpy(), rp)
    nu = int(n.cpu()[0])
    assert nu == len(ru) and np.array_equal(uniq.cpu().numpy()[:nu], ru)


# ---------------------------------------------------------------- gathered experts, small shapes
# Shapes: rows with an odd number of 32-blocks (H=96, 160; I=32, 96) take the
# register-staged GEMM; the rest the LDS-pipelined one. (200, 4, 192, 128, 2)
# has ~100 assignments per expert (several passes at every tile height) and a
# K tail (H=192); (48, 8, 128, 192, 2) takes four-tile passes with a K tail in
# the down projection (I=192).
SMALL = [(1, 6, 96, 64, 3), (1, 16, 256, 128, 4), (1, 4, 128, 2048, 3), (5, 6, 96, 64, 3), (37, 9, 160, 96, 4), (3, 2, 4096, 4096, 2),
         (2, 16, 64, 32, 16), (200, 4, 192, 128, 2), (48, 8, 128, 192, 2)]


PATHS = {"auto": 0, "gather": rq.MOE_FLAG_PATH_GATHER, "gemm": rq.MOE_FLAG_PATH_GEMM}


@pytest.mark.parametrize("path", ["gather", "gemm"])
@pytest.mark.parametrize("T,E,H,I,k", SMALL)
@pytest.mark.parametrize("scheme", [rq.MOE_Q_SYM8, rq.MOE_Q_INT4])
@pytest.mark.parametrize("xtype", [synth.F32, synth.F16, synth.BF16])
def test_gather_parity_small(T, E, H, I, k, scheme, xtype, path):
    say(f"experts T={T} E={E} H={H} I={I} k={k} scheme={scheme} xtype={xtype} path={path}")
    g = np.random.default_rng(T + E + H + I + k + 10 * scheme + xtype)
    wgu = (g.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    wd = (g.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    x32 = g.standard_normal((T, H)).astype(np.float32)
    x = synth.encode_x(x32, xtype)
    idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    gate = g.random((T, k)).astype(np.float32)
    ex = rq.quantize_experts(torch.from_numpy(wgu).cuda(), torch.from_numpy(wd).cuda(), scheme)
    rex = oracle.quantize_experts(wgu, wd, scheme)
    xd = to_dev_x(x, xtype)
    bf16 = xtype == synth.BF16
    fl = PATHS[path]
    if path == "gemm" and xtype == synth.F32:
        # the grouped GEMM's operands are the activations as given: 16-bit only
        with pytest.raises(rq.MoeError) as err:
            rq.moe_gather_qmm_forward(xd, ex, torch.from_numpy(idx).cuda(), torch.from_numpy(gate).cuda(), flags=fl)
        assert err.value.status == rq.MOE_ERR_UNSUPPORTED
        return
    y = rq.moe_gather_qmm_forward(xd, ex, torch.from_numpy(idx).cuda(), torch.from_numpy(gate).cuda(), flags=fl)
    ref = oracle.gather_forward(x, rex, idx, gate, bf16=bf16)
    assert rel_norm_err(y.cpu().numpy(), ref) <= Y_REL_NORM
    ys = rq.moe_gather_qmm_forward(xd, ex, torch.from_numpy(idx).cuda(), None, flags=fl)
    rys = oracle.gather_forward(x, rex, idx, None, bf16=bf16)
    assert rel_norm_err(ys.cpu().numpy(), rys) <= Y_REL_NORM


# One hot expert: slot 0 of every token routes to expert 0 and the other slots
# spread over the rest, so one expert runs many GEMM passes with a ragged last
# pass while the others run one short pass each. The three cases land in the
# six-tile (sym8; int4 takes four-tile), four-tile and one-tile pass regimes.
HOT = [(1100, 32, 2, 256, 128), (300, 40, 2, 256, 128), (64, 128, 4, 256, 192)]


@pytest.mark.parametrize("T,E,k,H,I", HOT)
@pytest.mark.parametrize("scheme", [rq.MOE_Q_SYM8, rq.MOE_Q_INT4])
@pytest.mark.parametrize("xtype", [synth.F16, synth.BF16])
def test_gemm_hot_expert(T, E, k, H, I, scheme, xtype):
    say(f"hot expert T={T} E={E} k={k} H={H} I={I} scheme={scheme} xtype={xtype}")
    g = np.random.default_rng(T + E + 3 * k + 10 * scheme + xtype)
    wgu = (g.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    wd = (g.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    x = synth.encode_x(g.standard_normal((T, H)).astype(np.float32), xtype)
    idx = np.zeros((T, k), np.int32)
    for t in range(T):
        idx[t, 1:] = 1 + (t * (k - 1) + np.arange(k - 1)) % (E - 1)
    assert np.bincount(idx.ravel(), minlength=E)[0] == T
    gate = g.random((T, k)).astype(np.float32)
    ex = rq.quantize_experts(torch.from_numpy(wgu).cuda(), torch.from_numpy(wd).cuda(), scheme)
    rex = oracle.quantize_experts(wgu, wd, scheme)
    xd = to_dev_x(x, xtype)
    bf16 = xtype == synth.BF16
    fl = rq.MOE_FLAG_PATH_GEMM
    y = rq.moe_gather_qmm_forward(xd, ex, torch.from_numpy(idx).cuda(), torch.from_numpy(gate).cuda(), flags=fl)
    assert rel_norm_err(y.cpu().numpy(), oracle.gather_forward(x, rex, idx, gate, bf16=bf16)) <= Y_REL_NORM
    ys = rq.moe_gather_qmm_forward(xd, ex, torch.from_numpy(idx).cuda(), None, flags=fl)
    assert rel_norm_err(ys.cpu().numpy(), oracle.gather_forward(x, rex, idx, None, bf16=bf16)) <= Y_REL_NORM


# ---------------------------------------------------------------- whole layer at the workloads' sizes
# Every token is compared with the oracle, except at prefill8k (8192 tokens),
# where the tokens are a stratified sample ("passes"): for every routed expert,
# the assignments at the first and last row of each 96-row pass of its grouped
# list (the six-tile passes the GEMM takes at this load) and its last
# assignment, plus a random spread.
LAYER_CASES = [("tiny", None, "all", "auto"), ("decode40", None, "all", "auto"), ("batched_int4", None, "all", "auto"),
               ("large_int4", None, "all", "auto"), ("prefill", None, "all", "auto"), ("batched_int4", 7, "all", "auto"),
               ("batched_int4", None, "all", "gemm"), ("large_int4", None, "all", "gemm"),
               ("prefill", None, "all", "gather"), ("decode40", None, "all", "gemm"), ("prefill", 300, "all", "gemm"),
               # one token at the E=512, top-10 shapes: scan top-k, two blocks per lane (H=4096),
               # the general down kernel (k*I > 4096)
               ("large_int4", 1, "all", "auto"), ("batched_int4", 1, "all", "auto"),
               # ~256 assignments per expert: six-tile GEMM passes
               ("prefill8k", None, "passes", "auto")]


def pass_boundary_tokens(ridx: np.ndarray, E: int, rows: int, extra: int, seed: int) -> np.ndarray:
    """Tokens of every expert's first and last assignment in each `rows`-row pass
    of its grouped list (stable by flat id), its last assignment, and `extra`
    random tokens."""
    k = ridx.shape[1]
    counts, offsets, perm = oracle.group(ridx, E)[:3]
    pos = []
    for e in np.nonzero(counts)[0]:
        n, o = int(counts[e]), int(offsets[e])
        for p0 in range(0, n, rows):
            pos += [o + p0, o + min(p0 + rows, n) - 1]
    toks = set(int(perm[p]) // k for p in pos)
    toks |= set(np.random.default_rng(seed).choice(ridx.shape[0], extra, replace=False).tolist())
    return np.array(sorted(toks))


@pytest.mark.parametrize("name,T,sample,path", LAYER_CASES)
def test_layer_parity(name, T, sample, path):
    w = synth.WORKLOADS[name]
    li = enforce_gap(w, synth.draw_layer(w, seed=0, layer=0, T=T, with_experts=False), seed=0, layer=0)
    bf16 = w.xtype == synth.BF16
    ridx, rgate = oracle.route(li.x, li.R, w.k, bf16=bf16)
    routed = np.unique(ridx)
    say(f"layer {name} T={li.x.shape[0]} unique experts={len(routed)} path={path}")
    ex = device_pool(w, 0, 0, routed)
    y, idx, gate = rq.moe_layer_forward(to_dev_x(li.x, w.xtype), torch.from_numpy(li.R).cuda(), ex, w.k,
                                        rq.MOE_FLAG_RENORM | PATHS[path])
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(gate.cpu().numpy() - rgate).max() <= GATE_ATOL
    yn = y.cpu().numpy()
    assert np.isfinite(yn).all()   # unrouted experts carry NaN scales
    Tn = li.x.shape[0]
    toks = np.arange(Tn) if sample == "all" else pass_boundary_tokens(ridx, w.E, 96, 64, seed=1)
    say(f"  comparing {len(toks)} of {Tn} tokens")
    rex, m = oracle_compact(w, 0, 0, np.unique(ridx[toks]))
    ref = oracle.gather_forward(np.ascontiguousarray(li.x[toks]), rex, remap(ridx[toks], m), rgate[toks], bf16=bf16)
    err, inf = rel_norm_err(yn[toks], ref), rel_inf_err(yn[toks], ref)
    say(f"  rel_norm_err={err:.3e} rel_inf_err={inf:.3e}")
    assert err <= Y_REL_NORM


def test_layer_is_deterministic():
    w = synth.WORKLOADS["batched_int4"]
    li = enforce_gap(w, synth.draw_layer(w, seed=3, with_experts=False), seed=3, layer=0)
    ridx, _ = oracle.route(li.x, li.R, w.k)
    ex = device_pool(w, 3, 0, np.unique(ridx))
    xd, Rd = to_dev_x(li.x, w.xtype), torch.from_numpy(li.R).cuda()
    a = rq.moe_layer_forward(xd, Rd, ex, w.k)[0].clone()
    b = rq.moe_layer_forward(xd, Rd, ex, w.k)[0]
    assert torch.equal(a, b)


# The grouped GEMM multiplies raw codes and applies each block's scale to the
# fp32 partial, and takes bf16 activations as they are: activations beyond the
# fp16 range, scales beyond 65504 / 127 and weights in the fp16 subnormal range
# stay exact. (xtype, activation scale, weight std) per case.
GEMM_RANGE = [(synth.BF16, 1e5, 0.02),      # activations above 65504
              (synth.BF16, 1e-3, 600.0),    # block scales above 516 (code * scale above 65504)
              (synth.F16, 1.0, 1e-5),       # weights below the fp16 normal range
              (synth.BF16, 1.0, 1e-5),
              (synth.F16, 8.0, 40.0)]       # large weights with h and outputs inside the fp16 range


@pytest.mark.parametrize("xtype,xs,wstd", GEMM_RANGE)
@pytest.mark.parametrize("scheme", [rq.MOE_Q_SYM8, rq.MOE_Q_INT4])
def test_gemm_path_range(xtype, xs, wstd, scheme):
    T, E, H, I, k = 48, 8, 256, 128, 3
    say(f"gemm range xtype={xtype} x*{xs} wstd={wstd} scheme={scheme}")
    g = np.random.default_rng(int(xs * 7 + wstd * 11) + scheme + 5 * xtype)
    wgu = (g.standard_normal((E, 2 * I, H)) * wstd).astype(np.float32)
    wd = (g.standard_normal((E, H, I)) * wstd).astype(np.float32)
    x = synth.encode_x((g.standard_normal((T, H)) * xs).astype(np.float32), xtype)
    idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    gate = g.random((T, k)).astype(np.float32)
    ex = rq.quantize_experts(torch.from_numpy(wgu).cuda(), torch.from_numpy(wd).cuda(), scheme)
    rex = oracle.quantize_experts(wgu, wd, scheme)
    y = rq.moe_gather_qmm_forward(to_dev_x(x, xtype), ex, torch.from_numpy(idx).cuda(), torch.from_numpy(gate).cuda(),
                                  flags=rq.MOE_FLAG_PATH_GEMM)
    ref = oracle.gather_forward(x, rex, idx, gate, bf16=xtype == synth.BF16)
    yn = y.cpu().numpy()
    assert np.isfinite(yn).all()
    assert rel_norm_err(yn, ref) <= Y_REL_NORM


@pytest.mark.parametrize("name", ["tiny", "decode40"])
def test_single_token_paths_agree_with_oracle(name):
    """One token: the fused two-kernel path (default) and the three-kernel
    gathered path (forced) both match the oracle, and both route identically."""
    w = synth.WORKLOADS[name]
    outs = []
    for layer in range(3):
        li = enforce_gap(w, synth.draw_layer(w, seed=5, layer=layer, with_experts=False), seed=5, layer=layer)
        ridx, rgate = oracle.route(li.x, li.R, w.k)
        ex = device_pool(w, 5, layer, np.unique(ridx))
        rex, m = oracle_compact(w, 5, layer, np.unique(ridx))
        ref = oracle.gather_forward(li.x, rex, remap(ridx, m), rgate)
        xd, Rd = to_dev_x(li.x, w.xtype), torch.from_numpy(li.R).cuda()
        for flags in (rq.MOE_FLAG_RENORM, rq.MOE_FLAG_RENORM | rq.MOE_FLAG_PATH_GATHER):
            y, idx, gate = rq.moe_layer_forward(xd, Rd, ex, w.k, flags)
            assert np.array_equal(idx.cpu().numpy(), ridx)
            assert np.abs(gate.cpu().numpy() - rgate).max() <= GATE_ATOL
            assert rel_norm_err(y.cpu().numpy(), ref) <= Y_REL_NORM
            outs.append(y.cpu().numpy())


@pytest.mark.parametrize("name", ["decode40", "tiny", "batched_int4"])
def test_single_token_fp32_h_matches_oracle(name):
    """MOE_FLAG_H_FP32: the single-token path keeps h in fp32 (the general down
    kernel); same routing, output within the contract, and no further from the
    oracle than the default fp16 h by more than rounding noise."""
    w = synth.WORKLOADS[name]
    li = enforce_gap(w, synth.draw_layer(w, seed=5, layer=0, T=1, with_experts=False), seed=5, layer=0)
    bf16 = w.xtype == synth.BF16
    ridx, rgate = oracle.route(li.x, li.R, w.k, bf16=bf16)
    ex = device_pool(w, 5, 0, np.unique(ridx))
    xd, Rd = to_dev_x(li.x, w.xtype), torch.from_numpy(li.R).cuda()
    y32, idx, _ = rq.moe_layer_forward(xd, Rd, ex, w.k, rq.MOE_FLAG_RENORM | rq.MOE_FLAG_H_FP32)
    y16 = rq.moe_layer_forward(xd, Rd, ex, w.k, rq.MOE_FLAG_RENORM)[0]
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ridx)
    rex, m = oracle_compact(w, 5, 0, np.unique(ridx))
    ref = oracle.gather_forward(li.x, rex, remap(ridx, m), rgate, bf16=bf16)
    e32, e16 = rel_norm_err(y32.cpu().numpy(), ref), rel_norm_err(y16.cpu().numpy(), ref)
    say(f"{name}: rel_norm_err fp32 h {e32:.2e}, fp16 h {e16:.2e}")
    assert e32 <= Y_REL_NORM
    assert e32 <= e16 + 1e-6


def test_stream_read_runs_on_ragged_sizes():
    """The bandwidth reference reads whole buffers and ragged tails without error."""
    buf = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    for n in (16, 1040, 4096 * 16 + 48, 1 << 20):
        rq.moe_stream_read(buf, n)
    torch.cuda.synchronize()


@pytest.mark.parametrize("E,k", [(256, 8), (512, 10), (1000, 10)])
def test_single_token_layer_exact_ties(E, k):
    """One token through the fused single-token path (top-k inside the gate/up
    kernel): exact logit ties go to the lower expert id, as in the oracle."""
    H, I = 128, 64
    g = np.random.default_rng(E * 7 + k)
    R = (g.standard_normal((E, H)) * 0.3).astype(np.float32)
    wgu = torch.from_numpy((g.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)).cuda()
    wd = torch.from_numpy((g.standard_normal((E, H, I)) * 0.02).astype(np.float32)).cuda()
    ex = rq.quantize_experts(wgu, wd, rq.MOE_Q_SYM8)
    # zero activations: every logit is 0, so ids 0..k-1 win with equal gates and y = 0
    y, idx, gate = rq.moe_layer_forward(torch.zeros((1, H), device="cuda"), torch.from_numpy(R).cuda(), ex, k)
    assert (idx.cpu().numpy() == np.arange(k)).all()
    assert np.allclose(gate.cpu().numpy(), 1.0 / k, atol=GATE_ATOL)
    assert not y.abs().max().item()
    # duplicated router rows: each copy ties with its original, the lower id first
    x = g.standard_normal((1, H)).astype(np.float32)
    R2 = R.copy()
    ridx0, _ = oracle.route(x, R, k)
    for j, e in enumerate(ridx0[0][:3]):
        R2[E - 1 - j] = R2[e]
    ridx, rgate = oracle.route(x, R2, k)
    _, gi, gg = rq.moe_layer_forward(torch.from_numpy(x).cuda(), torch.from_numpy(R2).cuda(), ex, k)
    assert np.array_equal(gi.cpu().numpy(), ridx)
    assert np.abs(gg.cpu().numpy() - rgate).max() <= GATE_ATOL


# one token through moe_layer_forward at edge shapes of the single-token kernels:
# one expert; k = 16 (a 1024-thread down workgroup); H = 4096 (two 16-byte pieces of
# x per thread through LDS); I = 1024 (two blocks per lane in the down kernel);
# I = 2048 (the fp32-activation down kernel); E = 512 (eight logits per lane)
T1_EDGE = [(1, 32, 32, 1), (16, 64, 32, 16), (64, 4096, 64, 8), (32, 256, 1024, 10), (512, 64, 32, 10),
           (8, 256, 2048, 3), (300, 160, 96, 5), (320, 256, 96, 8)]


@pytest.mark.parametrize("E,H,I,k", T1_EDGE)
@pytest.mark.parametrize("scheme", [rq.MOE_Q_SYM8, rq.MOE_Q_INT4])
@pytest.mark.parametrize("xtype", [synth.F32, synth.F16, synth.BF16])
def test_single_token_layer_edge_shapes(E, H, I, k, scheme, xtype):
    from tests.cases import gap_failures
    say(f"one token E={E} H={H} I={I} k={k} scheme={scheme} xtype={xtype}")
    g = np.random.default_rng(E * 31 + H + I + k + 7 * scheme + xtype)
    R = (g.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    bf16 = xtype == synth.BF16
    for _ in range(64):  # a token whose routing has margin (the oracle decides ties in fp64)
        x = synth.encode_x(g.standard_normal((1, H)).astype(np.float32), xtype)
        if k == E or len(gap_failures(x, R, k, bf16)) == 0:
            break
    else:
        pytest.fail("no token with a routing margin")
    wgu = (g.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    wd = (g.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    ex = rq.quantize_experts(torch.from_numpy(wgu).cuda(), torch.from_numpy(wd).cuda(), scheme)
    ridx, rgate = oracle.route(x, R, k, bf16=bf16)
    y, idx, gate = rq.moe_layer_forward(to_dev_x(x, xtype), torch.from_numpy(R).cuda(), ex, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(gate.cpu().numpy() - rgate).max() <= GATE_ATOL
    ref = oracle.gather_forward(x, oracle.quantize_experts(wgu, wd, scheme), ridx, rgate, bf16=bf16)
    assert rel_norm_err(y.cpu().numpy(), ref) <= Y_REL_NORM


# staged layer: (workload, tokens, path); one token runs the slot lookup inside
# the gate/up kernel's top-k, batches inside the grouped kernels
STAGED = [("decode40", 1, "auto"), ("batched_int4", 1, "auto"), ("tiny", 1, "auto"), ("batched_int4", 64, "auto"),
          ("large_int4", 16, "auto"), ("batched_int4", 7, "gather"), ("decode40", 3, "gemm")]


@pytest.mark.parametrize("name,T,path", STAGED)
def test_staged_layer_matches_oracle(name, T, path):
    """The layer on a resident stack behind a slot table (moe_layer_forward_staged):
    routing identical to the oracle's (expert ids), output within the contract
    of the oracle layer on the experts themselves, and equal, bit for bit, to the
    same kernels on the full pool."""
    w = synth.WORKLOADS[name]
    li = enforce_gap(w, synth.draw_layer(w, seed=9, layer=0, T=T, with_experts=False), seed=9, layer=0)
    bf16 = w.xtype == synth.BF16
    ridx, rgate = oracle.route(li.x, li.R, w.k, bf16=bf16)
    routed = np.unique(ridx)
    g = np.random.default_rng(len(routed) + T)
    # resident: the routed experts and as many others, in shuffled slots
    others = g.choice(np.setdiff1d(np.arange(w.E), routed), min(len(routed), w.E - len(routed)), replace=False)
    resident = np.concatenate([routed, others]).astype(np.int32)
    slots = g.permutation(len(resident)).astype(np.int32)
    say(f"staged {name} T={T} path={path}: {len(routed)} routed experts, {len(resident)} slots")
    pool = device_pool(w, 9, 0, resident)
    stack = rq.empty_stack(pool, len(resident))
    rq.moe_stage_experts(pool, stack, torch.from_numpy(resident).cuda(), torch.from_numpy(slots).cuda())
    slot_of = np.full(w.E, -1, dtype=np.int32)
    slot_of[resident] = slots
    xd, Rd = to_dev_x(li.x, w.xtype), torch.from_numpy(li.R).cuda()
    fl = rq.MOE_FLAG_RENORM | PATHS[path]
    y, idx, gate = rq.moe_layer_forward_staged(xd, Rd, stack, torch.from_numpy(slot_of).cuda(), w.k, fl)
    y_pool = rq.moe_layer_forward(xd, Rd, pool, w.k, fl)[0]
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(gate.cpu().numpy() - rgate).max() <= GATE_ATOL
    rex, m = oracle_compact(w, 9, 0, routed)
    ref = oracle.gather_forward(li.x, rex, remap(ridx, m), rgate, bf16=bf16)
    assert rel_norm_err(y.cpu().numpy(), ref) <= Y_REL_NORM
    assert torch.equal(y, y_pool)


@pytest.mark.parametrize("T,path", [(1, "auto"), (5, "auto"), (5, "gather")])
def test_staged_layer_skips_experts_without_a_slot(T, path):
    """A routed expert without a slot contributes nothing: the result equals the
    oracle's with that expert's weights zero, and nothing outside the stack is
    read (the stack holds only the resident experts)."""
    w = synth.WORKLOADS["decode40"]
    li = enforce_gap(w, synth.draw_layer(w, seed=13, layer=0, T=T, with_experts=False), seed=13, layer=0)
    ridx, rgate = oracle.route(li.x, li.R, w.k)
    routed = np.unique(ridx)
    missing = ridx[0, 1]                      # slot 1 of the first token is not resident
    resident = np.array([e for e in routed if e != missing], dtype=np.int32)
    pool = device_pool(w, 13, 0, resident)
    # slot 0 holds no expert: codes 0x5A and NaN scales, which a slot-less expert must not pick up
    stack = rq.empty_stack(pool, len(resident) + 1)
    stack.w_gate_up[0].fill_(0x5A)
    stack.w_down[0].fill_(0x5A)
    stack.s_gate_up[0].fill_(NAN_F16)
    stack.s_down[0].fill_(NAN_F16)
    rq.moe_stage_experts(pool, stack, torch.from_numpy(resident).cuda(),
                         torch.arange(1, len(resident) + 1, dtype=torch.int32, device="cuda"))
    slot_of = np.full(w.E, -1, dtype=np.int32)
    slot_of[resident] = np.arange(1, len(resident) + 1, dtype=np.int32)
    y, idx, gate = rq.moe_layer_forward_staged(to_dev_x(li.x, w.xtype), torch.from_numpy(li.R).cuda(), stack,
                                               torch.from_numpy(slot_of).cuda(), w.k,
                                               rq.MOE_FLAG_RENORM | PATHS[path])
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ridx)
    rex, m = oracle_compact(w, 13, 0, routed)
    j = m[int(missing)]
    rex.s_gate_up[j] = 0
    rex.s_down[j] = 0
    ref = oracle.gather_forward(li.x, rex, remap(ridx, m), rgate)
    yn = y.cpu().numpy()
    assert np.isfinite(yn).all()
    assert rel_norm_err(yn, ref) <= Y_REL_NORM


@pytest.mark.parametrize("scheme", [rq.MOE_Q_SYM8, rq.MOE_Q_INT4])
@pytest.mark.parametrize("T", [1, 5])
def test_staged_stack_matches_pool(scheme, T):
    """Staged decode: experts copied into stack slots (a full fill, then three
    slots rewritten in place) hold the pool's bytes, the slot table maps the
    routing, and the layer on the stack equals the layer on the pool."""
    E, H, I, k, S = 24, 256, 128, 4, 8
    g = np.random.default_rng(40 + scheme + T)
    wgu = torch.from_numpy((g.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)).cuda()
    wd = torch.from_numpy((g.standard_normal((E, H, I)) * 0.02).astype(np.float32)).cuda()
    pool = rq.quantize_experts(wgu, wd, scheme)
    stack = rq.empty_stack(pool, S)
    first = g.choice(E, S, replace=False).astype(np.int32)
    slots1 = g.permutation(S).astype(np.int32)
    rq.moe_stage_experts(pool, stack, torch.from_numpy(first).cuda(), torch.from_numpy(slots1).cuda())
    slot_expert = np.empty(S, dtype=np.int32)
    slot_expert[slots1] = first
    newcomers = g.choice(np.setdiff1d(np.arange(E), first), 3, replace=False).astype(np.int32)
    slots2 = g.choice(S, 3, replace=False).astype(np.int32)
    rq.moe_stage_experts(pool, stack, torch.from_numpy(newcomers).cuda(), torch.from_numpy(slots2).cuda())
    slot_expert[slots2] = newcomers
    torch.cuda.synchronize()
    sel = torch.from_numpy(slot_expert.astype(np.int64)).cuda()
    for name in ("w_gate_up", "s_gate_up", "w_down", "s_down"):
        assert torch.equal(getattr(stack, name), getattr(pool, name)[sel]), name
    slot_of = np.full(E, 0, dtype=np.int32)
    slot_of[slot_expert] = np.arange(S, dtype=np.int32)
    idx = np.stack([g.choice(slot_expert, k, replace=False) for _ in range(T)]).astype(np.int32)
    gate = g.random((T, k)).astype(np.float32)
    sidx = rq.moe_remap_ids(torch.from_numpy(idx).cuda(), torch.from_numpy(slot_of).cuda())
    assert np.array_equal(sidx.cpu().numpy(), slot_of[idx])
    x = torch.from_numpy(g.standard_normal((T, H)).astype(np.float16)).cuda()
    gd = torch.from_numpy(gate).cuda()
    y_stack = rq.moe_gather_qmm_forward(x, stack, sidx, gd)
    y_pool = rq.moe_gather_qmm_forward(x, pool, torch.from_numpy(idx).cuda(), gd)
    torch.cuda.synchronize()
    assert rel_norm_err(y_stack.cpu().numpy(), y_pool.cpu().numpy()) <= 1e-6
    # against the oracle on the experts themselves (expert ids)
    rex = oracle.quantize_experts(wgu.cpu().numpy(), wd.cpu().numpy(), scheme)
    ref = oracle.gather_forward(x.cpu().numpy(), rex, idx, gate)
    assert rel_norm_err(y_stack.cpu().numpy(), ref) <= Y_REL_NORM
    # ids outside [0, E) map to -1
    odd = torch.tensor([-1, E, 0], dtype=torch.int32, device="cuda")
    assert rq.moe_remap_ids(odd, torch.from_numpy(slot_of).cuda()).cpu().tolist() == [-1, -1, int(slot_of[0])]
