"""Python binding of libmoe.so, the MI355X (gfx950) routed block-quantized MoE layer.

This module only marshals arguments: it turns torch device tensors into
pointers, allocates outputs and workspace through torch, and calls the C ABI
declared in include/moe.h. Every step of the layer runs in the library's HIP
kernels. There is no fallback: if libmoe.so is missing or the GPU is absent,
the calls raise.

Entry points mirror the C names: moe_route, moe_group, moe_gather_qmm_forward,
moe_layer_forward, moe_quantize, moe_workspace_bytes, moe_prerouter_forward.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_F16, MOE_BF16 = 0, 1, 2
MOE_Q_SYM8, MOE_Q_INT4 = 0, 1
MOE_FLAG_RENORM, MOE_FLAG_PATH_GATHER, MOE_FLAG_PATH_GEMM, MOE_FLAG_H_FP32 = 1, 2, 4, 8

# Every function the header declares; the library must export all of them.
EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_group", "moe_gather_qmm_forward", "moe_layer_forward",
           "moe_layer_forward_noalloc", "moe_layer_forward_staged", "moe_quantize", "moe_timer_start", "moe_timer_read", "moe_stream_read", "moe_miss_replay",
           "moe_stage_experts", "moe_remap_ids", "moe_prerouter_workspace_bytes", "moe_prerouter_forward",
           "moe_experts_from_logits", "moe_prerouted_layer_forward", "moe_qlinear_lora_workspace_bytes",
           "moe_qlinear_lora_forward",
           "moe_status_str", "moe_last_error")

(MOE_KERNEL_ROUTE_LOGITS, MOE_KERNEL_TOPK, MOE_KERNEL_GROUP, MOE_KERNEL_GATE_UP, MOE_KERNEL_DOWN, MOE_KERNEL_COMBINE,
 MOE_KERNEL_GEMM_GATE_UP, MOE_KERNEL_GEMM_DOWN, MOE_KERNEL_QUANTIZE, MOE_KERNEL_HEAD, MOE_KERNEL_LORA) = range(11)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: status {status} ({detail})")
        self.status = status


class _Experts(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("scheme", ctypes.c_int32),
                ("w_gate_up", ctypes.c_void_p), ("s_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


class _QWeight(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("K", ctypes.c_int32), ("scheme", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class _Prerouter(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("E", ctypes.c_int32), ("F", ctypes.c_int32),
                ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("wl", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by routed_expert_quantized_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m routed_expert_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
        E = ctypes.POINTER(_Experts)
        sigs = {
            "moe_workspace_bytes": ([I32, I32, I32, I32, I32, I32], SZ),
            "moe_route": ([P, I32, I32, I32, P, I32, I32, U32, P, P, P, SZ, P], ctypes.c_int),
            "moe_group": ([P, I32, I32, I32, P, P, P, P, P, P, SZ, P], ctypes.c_int),
            "moe_gather_qmm_forward": ([P, I32, I32, E, I32, P, P, P, U32, P, SZ, P], ctypes.c_int),
            "moe_layer_forward": ([P, I32, I32, P, E, I32, U32, P, P, P, P, SZ, P], ctypes.c_int),
            "moe_layer_forward_noalloc": ([P, I32, I32, P, E, I32, U32, P, P, P, P], ctypes.c_int),
            "moe_layer_forward_staged": ([P, I32, I32, P, I32, E, P, I32, U32, P, P, P, P, SZ, P], ctypes.c_int),
            "moe_quantize": ([P, I64, I32, I32, P, P, P], ctypes.c_int),
            "moe_timer_start": ([I32, I32], ctypes.c_int),
            "moe_timer_read": ([P, I32, P], ctypes.c_int),
            "moe_stream_read": ([P, I64, P], ctypes.c_int),
            "moe_stage_experts": ([E, E, P, P, I32, P], ctypes.c_int),
            "moe_remap_ids": ([P, I64, P, I32, P, P], ctypes.c_int),
            "moe_miss_replay": ([P, P, I32, I32, I32, I32, I32, ctypes.c_float, ctypes.c_float, P, P, P, P],
                                ctypes.c_int),
            "moe_prerouter_workspace_bytes": ([I32, I32, I32], SZ),
            "moe_prerouter_forward": ([P, I32, I32, ctypes.POINTER(_Prerouter), P, P, I32, U32, P, P, P, P, SZ, P],
                                      ctypes.c_int),
            "moe_experts_from_logits": ([P, I32, I32, P, E, I32, U32, P, P, P, P, SZ, P], ctypes.c_int),
            "moe_prerouted_layer_forward": ([P, I32, I32, P, E, I32, U32, P, P, P, ctypes.POINTER(_Prerouter), P, P, P,
                                             SZ, P], ctypes.c_int),
            "moe_qlinear_lora_workspace_bytes": ([I32, I32], SZ),
            "moe_qlinear_lora_forward": ([P, I32, I32, ctypes.POINTER(_QWeight), P, P, I32, ctypes.c_float, P, P, SZ,
                                          P], ctypes.c_int),
            "moe_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "moe_last_error": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status, lib().moe_last_error().decode())


def _xtype(x: torch.Tensor) -> int:
    return {torch.float32: MOE_F32, torch.float16: MOE_F16, torch.bfloat16: MOE_BF16}[x.dtype]


def _p(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _device_tensor(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class Experts:
    """Packed experts on the device (layout in include/moe.h).

    w_gate_up uint8 [E][2I][H] (int4: [E][2I][H/2]); s_gate_up int16/uint16 bits [E][2I][H/32];
    w_down uint8 [E][H][I] (int4: [E][H][I/2]); s_down [E][H][I/32]."""
    E: int
    H: int
    I: int
    scheme: int
    w_gate_up: torch.Tensor
    s_gate_up: torch.Tensor
    w_down: torch.Tensor
    s_down: torch.Tensor

    def c(self) -> _Experts:
        for n in ("w_gate_up", "s_gate_up", "w_down", "s_down"):
            _device_tensor(getattr(self, n), n)
        return _Experts(self.E, self.H, self.I, self.scheme, self.w_gate_up.data_ptr(), self.s_gate_up.data_ptr(),
                        self.w_down.data_ptr(), self.s_down.data_ptr())

    @property
    def expert_bytes(self) -> int:
        """Bytes of one expert's codes and scales."""
        cpb = 32 if self.scheme == MOE_Q_SYM8 else 16
        return 3 * self.H * self.I // 32 * (cpb + 2)


class Workspace:
    """A growable 256-byte-aligned device scratch buffer (torch caching allocator)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes + 256:
            self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        off = (-self.buf.data_ptr()) % 256
        return self.buf[off:off + max(nbytes, 1)]


_default_ws: dict = {}


def _ws(ws: Workspace | None, nbytes: int, device) -> torch.Tensor:
    if ws is None:
        key = str(device)
        ws = _default_ws.setdefault(key, Workspace(device))
    return ws.get(nbytes)


def moe_workspace_bytes(T: int, E: int, H: int, I: int, k: int, scheme: int) -> int:
    return int(lib().moe_workspace_bytes(T, E, H, I, k, scheme))


def moe_quantize(w: torch.Tensor, scheme: int, stream=None):
    """Quantise fp32 w[..., K] per block of 32 along K. Returns (codes uint8, scales int16 bits)."""
    _device_tensor(w, "w")
    assert w.dtype == torch.float32
    K = w.shape[-1]
    rows = w.numel() // K
    cb = K if scheme == MOE_Q_SYM8 else K // 2
    codes = torch.empty(w.shape[:-1] + (cb,), dtype=torch.uint8, device=w.device)
    scales = torch.empty(w.shape[:-1] + (K // 32,), dtype=torch.int16, device=w.device)
    _check("moe_quantize", lib().moe_quantize(_p(w), rows, K, scheme, _p(codes), _p(scales), _stream(stream)))
    return codes, scales


def empty_stack(pool: "Experts", slots: int) -> "Experts":
    """A resident stack of `slots` expert slots shaped like `pool` (uninitialised)."""
    def like(t):
        return torch.empty((slots,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    return Experts(slots, pool.H, pool.I, pool.scheme, like(pool.w_gate_up), like(pool.s_gate_up), like(pool.w_down),
                   like(pool.s_down))


def moe_stage_experts(pool: "Experts", stack: "Experts", experts: torch.Tensor, slots: torch.Tensor,
                      stream=None) -> None:
    """Copy pool experts `experts` (device int32 [n]) into stack slots `slots` (device int32 [n])."""
    _device_tensor(experts, "experts")
    _device_tensor(slots, "slots")
    assert experts.dtype == torch.int32 and slots.dtype == torch.int32 and experts.shape == slots.shape
    cp, cs = pool.c(), stack.c()
    _check("moe_stage_experts", lib().moe_stage_experts(ctypes.byref(cp), ctypes.byref(cs), _p(experts), _p(slots),
                                                        experts.numel(), _stream(stream)))


def moe_remap_ids(idx: torch.Tensor, slot_of: torch.Tensor, stream=None) -> torch.Tensor:
    """out[...] = slot_of[idx[...]] on the device (int32)."""
    _device_tensor(idx, "idx")
    _device_tensor(slot_of, "slot_of")
    assert idx.dtype == torch.int32 and slot_of.dtype == torch.int32
    out = torch.empty_like(idx)
    _check("moe_remap_ids", lib().moe_remap_ids(_p(idx), idx.numel(), _p(slot_of), slot_of.numel(), _p(out),
                                                _stream(stream)))
    return out


def moe_layer_forward_staged(x: torch.Tensor, router_w: torch.Tensor, stack: "Experts", slot_of: torch.Tensor, k: int,
                             flags: int = MOE_FLAG_RENORM, ws: "Workspace | None" = None, stream=None,
                             out: torch.Tensor | None = None, return_routing: bool = True, routing_out=None):
    """Router over E = router_w.shape[0] experts, then the routed experts read from
    their slots slot_of[e] (device int32 [E]) of the resident stack. Returns y
    [T][H] (and topk_idx, topk_gate: expert ids, with return_routing)."""
    _device_tensor(x, "x")
    _device_tensor(router_w, "router_w")
    _device_tensor(slot_of, "slot_of")
    if slot_of.dtype != torch.int32:
        raise ValueError("slot_of must be int32")
    T = x.shape[0]
    E = router_w.shape[0]
    y = out if out is not None else torch.empty((T, stack.H), dtype=torch.float32, device=x.device)
    idx = gate = None
    if routing_out is not None:
        idx, gate = routing_out
    elif return_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        gate = torch.empty((T, k), dtype=torch.float32, device=x.device)
    nb = moe_workspace_bytes(T, E, stack.H, stack.I, k, stack.scheme)
    w = _ws(ws, nb, x.device)
    c = stack.c()
    _check("moe_layer_forward_staged",
           lib().moe_layer_forward_staged(_p(x), _xtype(x), T, _p(router_w), E, ctypes.byref(c), _p(slot_of), k,
                                          flags, _p(y), _p(idx), _p(gate), _p(w), w.numel(), _stream(stream)))
    return (y, idx, gate) if return_routing else y


MOE_MISS_FETCH_ALL, MOE_MISS_RULE, MOE_MISS_FIRST_CHOICE = 0, 1, 2


def moe_miss_replay(topk_idx, topk_gate, E: int, capacity: int, policy: int, threshold: float = 0.15,
                    admit_beta: float = 0.0):
    """Replay the expert-cache miss policy over a sequence of routings (host arrays
    [T][k] in slot order). Returns (m float32 [T], sync_fetches int32 [T],
    bg_fetches int32 [T], resident bool [E])."""
    import numpy as np
    idx = np.ascontiguousarray(np.asarray(topk_idx), dtype=np.int32)
    gate = np.ascontiguousarray(np.asarray(topk_gate), dtype=np.float32)
    if idx.ndim != 2 or gate.shape != idx.shape:
        raise ValueError("topk_idx and topk_gate must be [T][k] arrays of one shape")
    T, k = idx.shape
    m = np.empty(T, dtype=np.float32)
    sync = np.empty(T, dtype=np.int32)
    bg = np.empty(T, dtype=np.int32)
    res = np.empty(E, dtype=np.uint8)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check("moe_miss_replay", lib().moe_miss_replay(ptr(idx), ptr(gate), T, k, E, capacity, policy, threshold,
                                                    admit_beta, ptr(m), ptr(sync), ptr(bg), ptr(res)))
    return m, sync, bg, res.astype(bool)


def moe_stream_read(buf: torch.Tensor, nbytes: int | None = None, stream=None) -> None:
    """Plain streaming read of the first nbytes bytes of buf (the bandwidth reference)."""
    _device_tensor(buf, "buf")
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check("moe_stream_read", lib().moe_stream_read(_p(buf), n, _stream(stream)))


@dataclass
class Prerouter:
    """Prerouter head weights on the device, fp32 (layout in include/moe.h):
    w1 [F][H+2E], b1 [F] or None, w2 [E][F], b2 [E] or None, wl [E][H+2E]."""
    w1: torch.Tensor
    b1: torch.Tensor | None
    w2: torch.Tensor
    b2: torch.Tensor | None
    wl: torch.Tensor

    @property
    def E(self) -> int:
        return self.w2.shape[0]

    @property
    def F(self) -> int:
        return self.w1.shape[0]

    @property
    def H(self) -> int:
        return self.w1.shape[1] - 2 * self.E

    def c(self) -> _Prerouter:
        for n in ("w1", "b1", "w2", "b2", "wl"):
            t = getattr(self, n)
            if t is not None:
                _device_tensor(t, n)
                if t.dtype != torch.float32:
                    raise ValueError(f"{n} must be float32")
        ptr = lambda t: None if t is None else t.data_ptr()
        return _Prerouter(self.H, self.E, self.F, ptr(self.w1), ptr(self.b1), ptr(self.w2), ptr(self.b2),
                          ptr(self.wl))


def moe_prerouter_workspace_bytes(T: int, E: int, F: int) -> int:
    return int(lib().moe_prerouter_workspace_bytes(T, E, F))


def moe_prerouter_forward(x: torch.Tensor, head: Prerouter, cur: torch.Tensor | None, prev: torch.Tensor | None,
                          k: int, flags: int = MOE_FLAG_RENORM, want_logits: bool = False,
                          ws: Workspace | None = None, stream=None, out=None, logits_out: torch.Tensor | None = None,
                          topk: bool = True):
    """Prerouter head: the next layer's routing for the next token.
    Returns (topk_idx int32 [T][k], topk_gate fp32 [T][k]) and, with want_logits,
    also the head logits fp32 [T][E]. `out` may pass (idx, gate) tensors to fill,
    `logits_out` a [T][E] fp32 tensor. With topk=False only the logits are made
    (returned alone; for moe_experts_from_logits)."""
    _device_tensor(x, "x")
    T = x.shape[0]
    for n, t in (("cur", cur), ("prev", prev)):
        if t is not None:
            _device_tensor(t, n)
            if t.dtype != torch.int32 or t.shape != (T, k):
                raise ValueError(f"{n} must be int32 [T][k]")
    if not topk:
        idx = gate = None
        want_logits = True
    elif out is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        gate = torch.empty((T, k), dtype=torch.float32, device=x.device)
    else:
        idx, gate = out
    lg = logits_out
    if lg is None and want_logits:
        lg = torch.empty((T, head.E), dtype=torch.float32, device=x.device)
    hc = head.c()
    nb = moe_prerouter_workspace_bytes(T, head.E, head.F)
    w = _ws(ws, nb, x.device)
    _check("moe_prerouter_forward",
           lib().moe_prerouter_forward(_p(x), _xtype(x), T, ctypes.byref(hc), _p(cur), _p(prev), k, flags, _p(idx),
                                       _p(gate), _p(lg), _p(w), w.numel(), _stream(stream)))
    if not topk:
        return lg
    return (idx, gate, lg) if want_logits else (idx, gate)


def moe_experts_from_logits(x: torch.Tensor, logits: torch.Tensor, ex: "Experts", k: int,
                            flags: int = MOE_FLAG_RENORM, ws: Workspace | None = None, stream=None,
                            out: torch.Tensor | None = None, return_routing: bool = False, routing_out=None):
    """Expert layer on given router logits [T][E] fp32 (top-k, then the routed experts).
    Returns y [T][H] (and topk_idx, topk_gate with return_routing). routing_out
    may pass (idx, gate) tensors that receive the routing."""
    _device_tensor(x, "x")
    _device_tensor(logits, "logits")
    T = x.shape[0]
    y = out if out is not None else torch.empty((T, ex.H), dtype=torch.float32, device=x.device)
    if routing_out is not None:
        idx, gate = routing_out
    else:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device) if return_routing else None
        gate = torch.empty((T, k), dtype=torch.float32, device=x.device) if return_routing else None
    nb = moe_workspace_bytes(T, ex.E, ex.H, ex.I, k, ex.scheme)
    w = _ws(ws, nb, x.device)
    c = ex.c()
    _check("moe_experts_from_logits",
           lib().moe_experts_from_logits(_p(x), _xtype(x), T, _p(logits), ctypes.byref(c), k, flags, _p(y), _p(idx),
                                         _p(gate), _p(w), w.numel(), _stream(stream)))
    return (y, idx, gate) if return_routing else y


@dataclass
class QWeight:
    """One block-quantized matrix [N][K] on the device (codes uint8 [N][K] or [N][K/2],
    scales int16 bits [N][K/32])."""
    N: int
    K: int
    scheme: int
    codes: torch.Tensor
    scales: torch.Tensor

    def c(self) -> _QWeight:
        _device_tensor(self.codes, "codes")
        _device_tensor(self.scales, "scales")
        return _QWeight(self.N, self.K, self.scheme, self.codes.data_ptr(), self.scales.data_ptr())


def moe_qlinear_lora_forward(x: torch.Tensor, w: QWeight, lora_a: torch.Tensor | None, lora_b: torch.Tensor | None,
                             scale: float, ws: Workspace | None = None, stream=None,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """y [T][N] = W_q x + scale * B (A x); lora_a [r][K], lora_b [N][r] fp32 (None: no delta)."""
    _device_tensor(x, "x")
    T = x.shape[0]
    r = 0
    if (lora_a is None) != (lora_b is None):
        raise ValueError("lora_a and lora_b must be given together")
    if lora_a is not None:
        _device_tensor(lora_a, "lora_a")
        _device_tensor(lora_b, "lora_b")
        r = lora_a.shape[0]
        if lora_a.shape != (r, w.K) or lora_b.shape != (w.N, r):
            raise ValueError("lora_a must be [r][K] and lora_b [N][r]")
    y = out if out is not None else torch.empty((T, w.N), dtype=torch.float32, device=x.device)
    nb = int(lib().moe_qlinear_lora_workspace_bytes(T, r))
    buf = _ws(ws, nb, x.device)
    c = w.c()
    _check("moe_qlinear_lora_forward",
           lib().moe_qlinear_lora_forward(_p(x), _xtype(x), T, ctypes.byref(c), _p(lora_a), _p(lora_b), r, scale,
                                          _p(y), _p(buf), buf.numel(), _stream(stream)))
    return y


def moe_prerouted_layer_forward(x: torch.Tensor, logits: torch.Tensor, ex: "Experts", k: int,
                                head: Prerouter | None, prev_idx: torch.Tensor | None, idx_out: torch.Tensor,
                                logits_next: torch.Tensor | None, flags: int = MOE_FLAG_RENORM,
                                gate_out: torch.Tensor | None = None, ws: Workspace | None = None, stream=None,
                                out: torch.Tensor | None = None) -> torch.Tensor:
    """One prerouted decode layer: experts on the predicted `logits` (routing into
    idx_out), then the next layer's head writing logits_next. Returns y [T][H]."""
    _device_tensor(x, "x")
    _device_tensor(logits, "logits")
    T = x.shape[0]
    y = out if out is not None else torch.empty((T, ex.H), dtype=torch.float32, device=x.device)
    nb = -(-moe_workspace_bytes(T, ex.E, ex.H, ex.I, k, ex.scheme) // 256) * 256
    hc = None
    if head is not None:
        nb += moe_prerouter_workspace_bytes(T, head.E, head.F)
        hc = head.c()
    w = _ws(ws, nb, x.device)
    c = ex.c()
    _check("moe_prerouted_layer_forward",
           lib().moe_prerouted_layer_forward(_p(x), _xtype(x), T, _p(logits), ctypes.byref(c), k, flags, _p(y),
                                             _p(idx_out), _p(gate_out), ctypes.byref(hc) if hc is not None else None,
                                             _p(prev_idx), _p(logits_next), _p(w), w.numel(), _stream(stream)))
    return y


def moe_route(x: torch.Tensor, router_w: torch.Tensor, k: int, flags: int = MOE_FLAG_RENORM,
              ws: Workspace | None = None, stream=None):
    """Router: returns (topk_idx int32 [T][k], topk_gate fp32 [T][k])."""
    _device_tensor(x, "x")
    _device_tensor(router_w, "router_w")
    T, H = x.shape
    E = router_w.shape[0]
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    gate = torch.empty((T, k), dtype=torch.float32, device=x.device)
    nb = moe_workspace_bytes(T, E, H, 32, k, MOE_Q_SYM8)
    w = _ws(ws, nb, x.device)
    _check("moe_route", lib().moe_route(_p(x), _xtype(x), T, H, _p(router_w), E, k, flags, _p(idx), _p(gate),
                                        _p(w), w.numel(), _stream(stream)))
    return idx, gate


def moe_group(topk_idx: torch.Tensor, E: int, ws: Workspace | None = None, stream=None):
    """Token-by-expert grouping: returns (counts [E], offsets [E+1], perm [T*k], uniq [E], n_uniq [1])."""
    _device_tensor(topk_idx, "topk_idx")
    T, k = topk_idx.shape
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    uniq = torch.empty(E, dtype=torch.int32, device=dev)
    n_uniq = torch.empty(1, dtype=torch.int32, device=dev)
    nb = moe_workspace_bytes(T, E, 32, 32, k, MOE_Q_SYM8)
    w = _ws(ws, nb, dev)
    _check("moe_group", lib().moe_group(_p(topk_idx), T, k, E, _p(counts), _p(offsets), _p(perm), _p(uniq),
                                        _p(n_uniq), _p(w), w.numel(), _stream(stream)))
    return counts, offsets, perm, uniq, n_uniq


def moe_gather_qmm_forward(x: torch.Tensor, ex: Experts, topk_idx: torch.Tensor, topk_gate: torch.Tensor | None,
                           flags: int = 0, ws: Workspace | None = None, stream=None, out: torch.Tensor | None = None):
    """Routed-only expert layer on given routing. y [T][H], or [T][k][H] when topk_gate is None."""
    _device_tensor(x, "x")
    _device_tensor(topk_idx, "topk_idx")
    T, k = topk_idx.shape
    shape = (T, ex.H) if topk_gate is not None else (T, k, ex.H)
    y = out if out is not None else torch.empty(shape, dtype=torch.float32, device=x.device)
    nb = moe_workspace_bytes(T, ex.E, ex.H, ex.I, k, ex.scheme)
    w = _ws(ws, nb, x.device)
    c = ex.c()
    _check("moe_gather_qmm_forward",
           lib().moe_gather_qmm_forward(_p(x), _xtype(x), T, ctypes.byref(c), k, _p(topk_idx), _p(topk_gate), _p(y),
                                        flags, _p(w), w.numel(), _stream(stream)))
    return y


def moe_layer_forward(x: torch.Tensor, router_w: torch.Tensor, ex: Experts, k: int, flags: int = MOE_FLAG_RENORM,
                      ws: Workspace | None = None, stream=None, out: torch.Tensor | None = None,
                      return_routing: bool = True, routing_out=None):
    """Router + routed-only experts. Returns y [T][H] (and topk_idx, topk_gate).
    routing_out may pass (idx, gate) tensors that receive the routing."""
    _device_tensor(x, "x")
    _device_tensor(router_w, "router_w")
    T = x.shape[0]
    y = out if out is not None else torch.empty((T, ex.H), dtype=torch.float32, device=x.device)
    idx = gate = None
    if routing_out is not None:
        idx, gate = routing_out
    elif return_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
        gate = torch.empty((T, k), dtype=torch.float32, device=x.device)
    nb = moe_workspace_bytes(T, ex.E, ex.H, ex.I, k, ex.scheme)
    w = _ws(ws, nb, x.device)
    c = ex.c()
    _check("moe_layer_forward",
           lib().moe_layer_forward(_p(x), _xtype(x), T, _p(router_w), ctypes.byref(c), k, flags, _p(y), _p(idx),
                                   _p(gate), _p(w), w.numel(), _stream(stream)))
    return (y, idx, gate) if return_routing else y


MOE_NOALLOC_SCRATCH_BYTES = 16 << 20


def moe_layer_forward_noalloc(x: torch.Tensor, router_w: torch.Tensor, ex: Experts, k: int,
                              flags: int = MOE_FLAG_RENORM, stream=None, out: torch.Tensor | None = None,
                              routing_out=None):
    """moe_layer_forward with the library's static device scratch instead of a
    workspace (for callers that cannot allocate). `out` and `routing_out`
    ((idx, gate) tensors) let the caller pass every output, so the call itself
    allocates nothing; without them y (and no routing) is allocated here.
    Returns y [T][H]."""
    _device_tensor(x, "x")
    _device_tensor(router_w, "router_w")
    T = x.shape[0]
    y = out if out is not None else torch.empty((T, ex.H), dtype=torch.float32, device=x.device)
    idx, gate = routing_out if routing_out is not None else (None, None)
    c = ex.c()
    _check("moe_layer_forward_noalloc",
           lib().moe_layer_forward_noalloc(_p(x), _xtype(x), T, _p(router_w), ctypes.byref(c), k, flags, _p(y),
                                           _p(idx), _p(gate), _stream(stream)))
    return y


class KernelTimer:
    """Durations of the next `capacity` launches of one kernel family (HIP events).

    Use around eager (not graph-captured) calls: `with KernelTimer(MOE_KERNEL_GATE_UP, n) as t: ...`,
    then t.ms holds the per-launch durations in milliseconds."""

    def __init__(self, kernel: int, capacity: int):
        self.kernel, self.capacity, self.ms = kernel, capacity, []

    def __enter__(self):
        _check("moe_timer_start", lib().moe_timer_start(self.kernel, self.capacity))
        return self

    def __exit__(self, *exc):
        buf = (ctypes.c_float * self.capacity)()
        n = ctypes.c_int32(0)
        _check("moe_timer_read", lib().moe_timer_read(buf, self.capacity, ctypes.byref(n)))
        self.ms = list(buf[: n.value])
        return False


def quantize_experts(w_gate_up: torch.Tensor, w_down: torch.Tensor, scheme: int, stream=None) -> Experts:
    """Quantise fp32 device weights w_gate_up [E][2I][H], w_down [E][H][I] with the library's kernel."""
    E, I2, H = w_gate_up.shape
    cgu, sgu = moe_quantize(w_gate_up, scheme, stream)
    cd, sd = moe_quantize(w_down, scheme, stream)
    return Experts(E, H, I2 // 2, scheme, cgu, sgu, cd, sd)
