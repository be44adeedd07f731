"""The C ABI without a GPU: the library loads, exports every function that
include/moe.h declares, sizes workspaces, and rejects bad arguments on the host
before any launch (no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import routed_expert_quantized_amd as rq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rq.LIB_PATH):
        from routed_expert_quantized_amd import build
        build.build()
    return rq.lib()


def test_exports_every_declared_function(L):
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        header = f.read()
    declared = set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", header))
    assert declared == set(rq.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_stream_read_validation(L):
    assert L.moe_stream_read(None, 1024, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_stream_read(FAKE, 0, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_stream_read(FAKE, 1000, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_stream_read(ctypes.c_void_p(FAKE.value + 8), 1024, None) == rq.MOE_ERR_INVALID_ARG


def test_status_strings(L):
    for s in range(5):
        assert L.moe_status_str(s)
    assert L.moe_status_str(99) == b"unknown status"


def test_workspace_bytes(L):
    n1 = L.moe_workspace_bytes(1, 256, 2048, 512, 8, rq.MOE_Q_SYM8)
    n64 = L.moe_workspace_bytes(64, 512, 2048, 512, 10, rq.MOE_Q_INT4)
    assert n1 > 0 and n64 > n1 and n1 % 256 == 0
    # h for T*k*I fp32 and ys for T*k*H fp32 at least
    assert n64 >= 64 * 10 * (512 + 2048) * 4
    for bad in [(0, 256, 2048, 512, 8, 0), (1, 2048, 2048, 512, 8, 0), (1, 256, 2000, 512, 8, 0),
                (1, 256, 2048, 500, 8, 0), (1, 256, 2048, 512, 17, 0), (1, 4, 256, 128, 5, 0),
                (1, 256, 8192, 512, 8, 0), (1, 256, 2048, 512, 8, 7)]:
        assert L.moe_workspace_bytes(*bad) == 0, bad


def _route(L, **kw):
    a = dict(x=FAKE, xt=rq.MOE_F16, T=1, H=2048, R=FAKE, E=256, k=8, flags=1, idx=FAKE, gate=FAKE, ws=FAKE,
             nws=1 << 30)
    a.update(kw)
    return L.moe_route(a["x"], a["xt"], a["T"], a["H"], a["R"], a["E"], a["k"], a["flags"], a["idx"], a["gate"],
                       a["ws"], a["nws"], None)


def test_route_validation(L):
    assert _route(L, x=None) == rq.MOE_ERR_INVALID_ARG
    assert b"x is NULL" in L.moe_last_error()
    assert _route(L, xt=7) == rq.MOE_ERR_UNSUPPORTED
    assert _route(L, T=0) == rq.MOE_ERR_INVALID_ARG
    assert _route(L, H=2040) == rq.MOE_ERR_INVALID_ARG
    assert _route(L, k=0) == rq.MOE_ERR_INVALID_ARG
    assert _route(L, k=17, E=256) == rq.MOE_ERR_INVALID_ARG
    assert _route(L, k=9, E=8) == rq.MOE_ERR_INVALID_ARG
    assert _route(L, E=1025) == rq.MOE_ERR_INVALID_ARG
    assert _route(L, R=None) == rq.MOE_ERR_INVALID_ARG
    assert _route(L, x=ctypes.c_void_p(0x10008)) == rq.MOE_ERR_INVALID_ARG
    assert _route(L, flags=0x80) == rq.MOE_ERR_UNSUPPORTED
    assert _route(L, nws=1024) == rq.MOE_ERR_WORKSPACE
    assert b"needed" in L.moe_last_error()
    assert _route(L, ws=None) == rq.MOE_ERR_WORKSPACE
    assert _route(L, ws=ctypes.c_void_p(0x10010)) == rq.MOE_ERR_WORKSPACE


def _experts(scheme=rq.MOE_Q_SYM8, E=256, H=2048, I=512, ptr=FAKE):
    return rq._Experts(E, H, I, scheme, ptr.value if ptr is not None else None, FAKE.value, FAKE.value, FAKE.value)


def test_gather_and_layer_validation(L):
    ex = _experts()

    def gather(x=FAKE, xt=rq.MOE_F16, T=1, e=ex, k=8, idx=FAKE, gate=FAKE, y=FAKE, flags=0, ws=FAKE, nws=1 << 30):
        return L.moe_gather_qmm_forward(x, xt, T, ctypes.byref(e) if e is not None else None, k, idx, gate, y,
                                        flags, ws, nws, None)

    assert gather(e=None) == rq.MOE_ERR_INVALID_ARG
    assert gather(e=_experts(scheme=3)) == rq.MOE_ERR_UNSUPPORTED
    assert gather(e=_experts(ptr=None)) == rq.MOE_ERR_INVALID_ARG
    assert gather(e=_experts(ptr=ctypes.c_void_p(0x10004))) == rq.MOE_ERR_INVALID_ARG
    assert gather(e=_experts(I=100)) == rq.MOE_ERR_INVALID_ARG
    assert gather(e=_experts(H=8192)) == rq.MOE_ERR_INVALID_ARG
    assert gather(idx=None) == rq.MOE_ERR_INVALID_ARG
    assert gather(y=None) == rq.MOE_ERR_INVALID_ARG
    assert gather(flags=rq.MOE_FLAG_PATH_GATHER | rq.MOE_FLAG_PATH_GEMM) == rq.MOE_ERR_INVALID_ARG
    assert gather(flags=0x100) == rq.MOE_ERR_UNSUPPORTED
    # fp32 h on the single-token path is a known flag: validation goes on to the workspace
    assert gather(flags=rq.MOE_FLAG_H_FP32, nws=4096) == rq.MOE_ERR_WORKSPACE
    assert gather(flags=rq.MOE_FLAG_H_FP32 | 0x100) == rq.MOE_ERR_UNSUPPORTED
    # the grouped GEMM takes 16-bit activations only; fp32 goes to the gathered path
    assert gather(flags=rq.MOE_FLAG_PATH_GEMM, xt=rq.MOE_F32, T=4) == rq.MOE_ERR_UNSUPPORTED
    assert b"fp16 or bf16" in L.moe_last_error()
    assert gather(nws=4096) == rq.MOE_ERR_WORKSPACE
    need = L.moe_workspace_bytes(64, 256, 2048, 512, 8, 0)
    assert gather(T=64, nws=need - 1) == rq.MOE_ERR_WORKSPACE

    def layer(x=FAKE, R=FAKE, e=ex, k=8, flags=1, y=FAKE, nws=1 << 30):
        return L.moe_layer_forward(x, rq.MOE_F16, 1, R, ctypes.byref(e), k, flags, y, None, None, FAKE, nws, None)

    assert layer(R=None) == rq.MOE_ERR_INVALID_ARG
    assert layer(y=None) == rq.MOE_ERR_INVALID_ARG
    assert layer(k=300) == rq.MOE_ERR_INVALID_ARG
    assert layer(nws=16) == rq.MOE_ERR_WORKSPACE
    assert layer(flags=0x40) == rq.MOE_ERR_UNSUPPORTED


def test_layer_noalloc_validation(L):
    """The static-scratch entry point checks everything on the host, scratch size
    included, before it looks anything up on the device."""
    ex = _experts()

    def layer(x=FAKE, xt=rq.MOE_F16, T=1, R=FAKE, e=ex, k=8, flags=1, y=FAKE):
        return L.moe_layer_forward_noalloc(x, xt, T, R, ctypes.byref(e) if e is not None else None, k, flags, y,
                                           None, None, None)

    assert layer(x=None) == rq.MOE_ERR_INVALID_ARG
    assert layer(R=None) == rq.MOE_ERR_INVALID_ARG
    assert layer(y=None) == rq.MOE_ERR_INVALID_ARG
    assert layer(e=None) == rq.MOE_ERR_INVALID_ARG
    assert layer(k=300) == rq.MOE_ERR_INVALID_ARG
    assert layer(flags=0x40) == rq.MOE_ERR_UNSUPPORTED
    assert layer(xt=9) == rq.MOE_ERR_UNSUPPORTED
    # prefill: 2048 tokens need about 175 MiB of scratch, beyond the static 16 MiB
    big = _experts(E=256, H=2048, I=512)
    assert layer(T=2048, e=big, xt=rq.MOE_BF16) == rq.MOE_ERR_WORKSPACE
    assert b"static scratch" in L.moe_last_error()
    assert L.moe_workspace_bytes(2048, 256, 2048, 512, 8, 0) > rq.MOE_NOALLOC_SCRATCH_BYTES
    # the shapes the scratch is sized for
    for T, E, H, I, k, s in [(1, 1024, 4096, 4096, 16, 0), (64, 512, 2048, 512, 10, 1), (16, 512, 4096, 1024, 10, 1)]:
        assert 0 < L.moe_workspace_bytes(T, E, H, I, k, s) <= rq.MOE_NOALLOC_SCRATCH_BYTES


def test_group_and_quantize_validation(L):
    assert L.moe_group(None, 4, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_group(FAKE, 4, 9, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_group(FAKE, 4, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None) == rq.MOE_ERR_WORKSPACE
    assert L.moe_quantize(FAKE, 4, 48, 0, FAKE, FAKE, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_quantize(FAKE, 4, 64, 2, FAKE, FAKE, None) == rq.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize(None, 4, 64, 0, FAKE, FAKE, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_quantize(FAKE, -1, 64, 0, FAKE, FAKE, None) == rq.MOE_ERR_INVALID_ARG


def test_stage_and_remap_validation(L):
    pool = rq._Experts(8, 64, 32, rq.MOE_Q_SYM8, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    wrong = rq._Experts(4, 64, 64, rq.MOE_Q_SYM8, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    big = rq._Experts(9, 64, 32, rq.MOE_Q_SYM8, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    odd = rq._Experts(4, 64, 32, rq.MOE_Q_SYM8, FAKE.value, FAKE.value + 2, FAKE.value, FAKE.value)
    assert L.moe_stage_experts(ctypes.byref(pool), ctypes.byref(wrong), FAKE, FAKE, 1, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_stage_experts(ctypes.byref(pool), ctypes.byref(big), FAKE, FAKE, 1, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_stage_experts(ctypes.byref(pool), ctypes.byref(odd), FAKE, FAKE, 1, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_stage_experts(ctypes.byref(pool), ctypes.byref(pool), None, FAKE, 1, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_stage_experts(ctypes.byref(pool), ctypes.byref(pool), FAKE, FAKE, -1, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_remap_ids(None, 4, FAKE, 8, FAKE, None) == rq.MOE_ERR_INVALID_ARG
    assert L.moe_remap_ids(FAKE, -1, FAKE, 8, FAKE, None) == rq.MOE_ERR_INVALID_ARG


def test_prerouter_workspace_and_validation(L):
    n1 = L.moe_prerouter_workspace_bytes(1, 256, 256)
    n64 = L.moe_prerouter_workspace_bytes(64, 256, 512)
    assert n1 >= 256 * 4 * 2 and n64 >= 64 * (256 + 512) * 4 and n1 % 256 == 0
    for bad in [(0, 256, 256), (1, 255, 256), (1, 2048, 256), (1, 256, 100), (1, 256, 8192), (1, 0, 256)]:
        assert L.moe_prerouter_workspace_bytes(*bad) == 0, bad

    def head(H=2048, E=256, F=256, w1=FAKE, w2=FAKE, wl=FAKE, b1=None, b2=None):
        v = lambda p: None if p is None else p.value
        return rq._Prerouter(H, E, F, v(w1), v(b1), v(w2), v(b2), v(wl))

    def call(x=FAKE, xt=rq.MOE_BF16, T=1, hd="default", cur=FAKE, prev=FAKE, k=8, flags=1, idx=FAKE, gate=FAKE,
             lg=None, ws=FAKE, nws=1 << 30):
        hd = head() if hd == "default" else hd
        return L.moe_prerouter_forward(x, xt, T, ctypes.byref(hd) if hd is not None else None, cur, prev, k, flags,
                                       idx, gate, lg, ws, nws, None)

    assert call(x=None) == rq.MOE_ERR_INVALID_ARG
    assert call(xt=5) == rq.MOE_ERR_UNSUPPORTED
    assert call(hd=None) == rq.MOE_ERR_INVALID_ARG
    assert call(T=0) == rq.MOE_ERR_INVALID_ARG
    assert call(hd=head(E=255), k=8) == rq.MOE_ERR_INVALID_ARG
    assert b"even" in L.moe_last_error()
    assert call(hd=head(E=2048)) == rq.MOE_ERR_INVALID_ARG
    assert call(hd=head(H=2050)) == rq.MOE_ERR_INVALID_ARG
    assert call(hd=head(F=100)) == rq.MOE_ERR_INVALID_ARG
    assert call(hd=head(F=8192)) == rq.MOE_ERR_INVALID_ARG
    assert call(k=17) == rq.MOE_ERR_INVALID_ARG
    assert call(hd=head(w1=None)) == rq.MOE_ERR_INVALID_ARG
    assert call(hd=head(wl=ctypes.c_void_p(0x10008))) == rq.MOE_ERR_INVALID_ARG
    assert call(hd=head(b1=ctypes.c_void_p(0x10002))) == rq.MOE_ERR_INVALID_ARG
    assert call(cur=ctypes.c_void_p(0x10002)) == rq.MOE_ERR_INVALID_ARG
    assert call(idx=None) == rq.MOE_ERR_INVALID_ARG
    assert call(flags=2) == rq.MOE_ERR_UNSUPPORTED
    assert call(ws=None) == rq.MOE_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x10010)) == rq.MOE_ERR_WORKSPACE
    assert call(nws=1024) == rq.MOE_ERR_WORKSPACE
    assert b"needed" in L.moe_last_error()
    assert call(idx=None, gate=None) == rq.MOE_ERR_INVALID_ARG     # nothing to write
    assert call(lg=ctypes.c_void_p(0x10008)) == rq.MOE_ERR_INVALID_ARG


def test_experts_from_logits_validation(L):
    ex = _experts()

    def call(x=FAKE, xt=rq.MOE_F16, T=1, lg=FAKE, e=ex, k=8, flags=1, y=FAKE, ws=FAKE, nws=1 << 30):
        return L.moe_experts_from_logits(x, xt, T, lg, ctypes.byref(e) if e is not None else None, k, flags, y,
                                         None, None, ws, nws, None)

    assert call(lg=None) == rq.MOE_ERR_INVALID_ARG
    assert b"logits" in L.moe_last_error()
    assert call(lg=ctypes.c_void_p(0x10004)) == rq.MOE_ERR_INVALID_ARG
    assert call(x=None) == rq.MOE_ERR_INVALID_ARG
    assert call(e=None) == rq.MOE_ERR_INVALID_ARG
    assert call(y=None) == rq.MOE_ERR_INVALID_ARG
    assert call(k=0) == rq.MOE_ERR_INVALID_ARG
    assert call(flags=rq.MOE_FLAG_PATH_GATHER | rq.MOE_FLAG_PATH_GEMM) == rq.MOE_ERR_INVALID_ARG
    assert call(flags=0x40) == rq.MOE_ERR_UNSUPPORTED
    assert call(nws=16) == rq.MOE_ERR_WORKSPACE


def test_qlinear_lora_validation(L):
    assert L.moe_qlinear_lora_workspace_bytes(1, 16) == 256
    assert L.moe_qlinear_lora_workspace_bytes(100, 64) == 25600
    assert L.moe_qlinear_lora_workspace_bytes(3, 5) == 256
    assert L.moe_qlinear_lora_workspace_bytes(1, 0) == 256
    for bad in [(0, 8), (1, 65), (1, -1), (70000, 8)]:
        assert L.moe_qlinear_lora_workspace_bytes(*bad) == 0, bad

    def qw(N=2048, K=2048, scheme=rq.MOE_Q_INT4, codes=FAKE, scales=FAKE):
        v = lambda p: None if p is None else p.value
        return rq._QWeight(N, K, scheme, v(codes), v(scales))

    def call(x=FAKE, xt=rq.MOE_F16, T=1, w="default", a=FAKE, b=FAKE, r=16, y=FAKE, ws=FAKE, nws=1 << 20):
        w = qw() if w == "default" else w
        return L.moe_qlinear_lora_forward(x, xt, T, ctypes.byref(w) if w is not None else None, a, b, r, 0.5, y, ws,
                                          nws, None)

    assert call(x=None) == rq.MOE_ERR_INVALID_ARG
    assert call(xt=9) == rq.MOE_ERR_UNSUPPORTED
    assert call(w=None) == rq.MOE_ERR_INVALID_ARG
    assert call(w=qw(scheme=4)) == rq.MOE_ERR_UNSUPPORTED
    assert call(w=qw(K=100)) == rq.MOE_ERR_INVALID_ARG
    assert call(w=qw(K=8192)) == rq.MOE_ERR_INVALID_ARG
    assert call(w=qw(N=0)) == rq.MOE_ERR_INVALID_ARG
    assert call(w=qw(codes=None)) == rq.MOE_ERR_INVALID_ARG
    assert call(w=qw(codes=ctypes.c_void_p(0x10004))) == rq.MOE_ERR_INVALID_ARG
    assert call(w=qw(scales=ctypes.c_void_p(0x10001))) == rq.MOE_ERR_INVALID_ARG
    assert call(T=0) == rq.MOE_ERR_INVALID_ARG
    assert call(r=65) == rq.MOE_ERR_INVALID_ARG
    assert call(a=None) == rq.MOE_ERR_INVALID_ARG
    assert call(a=ctypes.c_void_p(0x10008)) == rq.MOE_ERR_INVALID_ARG
    assert call(y=None) == rq.MOE_ERR_INVALID_ARG
    assert call(ws=None) == rq.MOE_ERR_WORKSPACE
    assert call(T=4096, nws=1024) == rq.MOE_ERR_WORKSPACE


def test_prerouted_layer_validation(L):
    ex = _experts(E=256, H=2048, I=512)
    hd = rq._Prerouter(2048, 256, 256, FAKE.value, None, FAKE.value, None, FAKE.value)
    other = ctypes.c_void_p(0x20000)

    def call(lg=FAKE, e=ex, h=hd, idx=FAKE, prev=None, nxt=other, y=FAKE, ws=FAKE, nws=1 << 30):
        return L.moe_prerouted_layer_forward(FAKE, rq.MOE_F16, 1, lg, ctypes.byref(e), 8, 1, y, idx, None,
                                             ctypes.byref(h) if h is not None else None, prev, nxt, ws, nws, None)

    assert call(lg=None) == rq.MOE_ERR_INVALID_ARG
    assert call(idx=None) == rq.MOE_ERR_INVALID_ARG
    assert b"topk_idx_out" in L.moe_last_error()
    assert call(nxt=None) == rq.MOE_ERR_INVALID_ARG
    assert call(nxt=FAKE) == rq.MOE_ERR_INVALID_ARG        # the same array as logits
    assert b"aliases" in L.moe_last_error()
    assert call(prev=FAKE) == rq.MOE_ERR_INVALID_ARG       # the same array as topk_idx_out
    assert call(h=rq._Prerouter(2048, 128, 256, FAKE.value, None, FAKE.value, None, FAKE.value)) == \
        rq.MOE_ERR_INVALID_ARG                              # head E differs from the experts'
    assert call(h=rq._Prerouter(2048, 256, 100, FAKE.value, None, FAKE.value, None, FAKE.value)) == \
        rq.MOE_ERR_INVALID_ARG
    assert call(nws=1 << 16) == rq.MOE_ERR_WORKSPACE


def test_binding_rejects_half_an_adapter():
    import torch
    qw = rq.QWeight(32, 32, rq.MOE_Q_SYM8, torch.zeros((32, 32), dtype=torch.uint8),
                    torch.zeros((32, 1), dtype=torch.int16))
    with pytest.raises(ValueError):
        rq.moe_qlinear_lora_forward(torch.zeros((1, 32)), qw, torch.zeros((4, 32)), None, 1.0)
