"""Plain CPU oracle for the routed, block-quantized MoE expert layer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import this package. It shares nothing
with the GPU library (``routed_expert_quantized_amd``) and never imports it.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64 sums, each function
citing the page passage it follows); this module only marshals numpy arrays
through ctypes. Page keys:

  [LR] "QwenのMoEルーターを観測してホットエキスパートを先読みしても速くならなかった" (lilting.ch)
  [QK] "鳴かぬなら、カスタムカーネル、ほととぎす" (qiita.com, john-rocky)
  [MW] "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with
       Trained Routing Prediction" (xyznot.com)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

F32, F16, BF16 = 0, 1, 2
SYM8, INT4 = 0, 1
RENORM = 1

_XTYPE = {np.dtype(np.float32): F32, np.dtype(np.float16): F16}


def build(verbose: bool = False) -> str:
    """Compile moe_oracle.c with gcc into libmoe_oracle.so next to it.

    No fast-math and no FMA contraction, so the C arithmetic is exactly what
    the source says; no -march=native, so the library runs on any x86-64 host.
    """
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


class _Experts(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("scheme", ctypes.c_int32),
                ("w_gate_up", ctypes.c_void_p), ("s_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


def _declare(L: ctypes.CDLL) -> None:
    P, I32, I64, U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    sigs = {
        "oref_f32_to_f16": ([ctypes.c_float], ctypes.c_uint16),
        "oref_f16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
        "oref_bf16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
        "oref_quantize": ([P, I64, I32, I32, P, P], ctypes.c_int),
        "oref_dequantize": ([P, P, I64, I32, I32, P], ctypes.c_int),
        "oref_logits": ([P, I32, I32, I32, P, I32, P], ctypes.c_int),
        "oref_route": ([P, I32, I32, I32, P, I32, I32, U32, P, P], ctypes.c_int),
        "oref_group": ([P, I32, I32, I32, P, P, P, P, P], ctypes.c_int),
        "oref_topk_logits": ([P, I32, I32, I32, U32, P, P], ctypes.c_int),
        "oref_qlinear_lora": ([P, I32, I32, I32, I32, I32, P, P, P, P, I32, ctypes.c_double, P], ctypes.c_int),
        "oref_prerouter": ([P, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, I32, U32, P, P, P], ctypes.c_int),
        "oref_gather_forward": ([P, I32, I32, ctypes.POINTER(_Experts), I32, P, P, P], ctypes.c_int),
        "oref_layer_forward": ([P, I32, I32, P, ctypes.POINTER(_Experts), I32, U32, P, P, P], ctypes.c_int),
        "oref_dense_forward": ([P, I32, I32, ctypes.POINTER(_Experts), P, P], ctypes.c_int),
        "oref_set_plant": ([I32], None),
        "oref_num_threads": ([], I32),
        "oref_set_num_threads": ([I32], None),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"{what} failed with code {rc}")


@dataclass
class Experts:
    """Packed experts in the oracle's layout (see moe_oracle.h).

    w_gate_up [E][2I][H] (int4: [E][2I][H/2]) uint8, s_gate_up [E][2I][H/32] uint16 (fp16 bits),
    w_down    [E][H][I]  (int4: [E][H][I/2])  uint8, s_down    [E][H][I/32]  uint16.
    """
    E: int
    H: int
    I: int
    scheme: int
    w_gate_up: np.ndarray
    s_gate_up: np.ndarray
    w_down: np.ndarray
    s_down: np.ndarray

    def _c(self) -> _Experts:
        for a in (self.w_gate_up, self.s_gate_up, self.w_down, self.s_down):
            assert a.flags.c_contiguous
        return _Experts(self.E, self.H, self.I, self.scheme, self.w_gate_up.ctypes.data,
                        self.s_gate_up.ctypes.data, self.w_down.ctypes.data, self.s_down.ctypes.data)


def _xtype(x: np.ndarray, bf16: bool) -> int:
    if bf16:
        assert x.dtype == np.uint16
        return BF16
    return _XTYPE[x.dtype]


def f32_to_f16_bits(v: float) -> int:
    return int(lib().oref_f32_to_f16(float(v)))


def f16_bits_to_f32(b: int) -> float:
    return float(lib().oref_f16_to_f32(int(b)))


def bf16_bits_to_f32(b: int) -> float:
    return float(lib().oref_bf16_to_f32(int(b)))


def quantize(w: np.ndarray, scheme: int) -> tuple[np.ndarray, np.ndarray]:
    """Quantise fp32 w[..., K] per block of 32 along K [QK §6]. Returns (codes, scales)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K = w.shape[-1]
    rows = int(np.prod(w.shape[:-1])) if w.ndim > 1 else 1
    cb = K if scheme == SYM8 else K // 2
    codes = np.zeros(w.shape[:-1] + (cb,), dtype=np.uint8)
    scales = np.zeros(w.shape[:-1] + (K // 32,), dtype=np.uint16)
    _check(lib().oref_quantize(_ptr(w), rows, K, scheme, _ptr(codes), _ptr(scales)), "oref_quantize")
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, K: int, scheme: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    rows = scales.size // (K // 32)
    w = np.empty(scales.shape[:-1] + (K,), dtype=np.float32)
    _check(lib().oref_dequantize(_ptr(codes), _ptr(scales), rows, K, scheme, _ptr(w)), "oref_dequantize")
    return w


def quantize_experts(w_gate_up: np.ndarray, w_down: np.ndarray, scheme: int) -> Experts:
    """Quantise fp32 expert weights w_gate_up [E][2I][H], w_down [E][H][I]."""
    E, I2, H = w_gate_up.shape
    cgu, sgu = quantize(w_gate_up, scheme)
    cd, sd = quantize(w_down, scheme)
    return Experts(E, H, I2 // 2, scheme, cgu, sgu, cd, sd)


def logits(x: np.ndarray, R: np.ndarray, bf16: bool = False) -> np.ndarray:
    x = np.ascontiguousarray(x)
    R = np.ascontiguousarray(R, dtype=np.float32)
    T, H = x.shape
    E = R.shape[0]
    out = np.empty((T, E), dtype=np.float64)
    _check(lib().oref_logits(_ptr(x), _xtype(x, bf16), T, H, _ptr(R), E, _ptr(out)), "oref_logits")
    return out


def route(x: np.ndarray, R: np.ndarray, k: int, flags: int = RENORM, bf16: bool = False):
    x = np.ascontiguousarray(x)
    R = np.ascontiguousarray(R, dtype=np.float32)
    T, H = x.shape
    E = R.shape[0]
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float32)
    _check(lib().oref_route(_ptr(x), _xtype(x, bf16), T, H, _ptr(R), E, k, flags, _ptr(idx), _ptr(gate)),
           "oref_route")
    return idx, gate


@dataclass
class PrerouterHead:
    """Prerouter head weights, fp32, in the page's layout: the input feature is
    [hidden (H) ; k-hot current routing (E) ; k-hot previous routing (E)].

    w1 [F][H+2E] and b1 [F] (fc1), w2 [E][F] and b2 [E] (fc2), wl [E][H+2E] (the
    linear residual path). b1 and b2 may be None (no bias)."""
    w1: np.ndarray
    b1: np.ndarray | None
    w2: np.ndarray
    b2: np.ndarray | None
    wl: np.ndarray

    @property
    def E(self) -> int:
        return self.w2.shape[0]

    @property
    def F(self) -> int:
        return self.w1.shape[0]

    @property
    def H(self) -> int:
        return self.w1.shape[1] - 2 * self.E


def prerouter(x: np.ndarray, head: PrerouterHead, cur: np.ndarray | None, prev: np.ndarray | None, k: int,
              flags: int = RENORM, bf16: bool = False):
    """Head logits (fp64), then the router's softmax/top-k on them [MW "prerouter head
    architecture"]. Returns (idx [T][k] int32, gate [T][k] fp32, logits [T][E] fp64)."""
    x = np.ascontiguousarray(x)
    T, H = x.shape
    E, F = head.E, head.F
    assert head.H == H and head.wl.shape == (E, H + 2 * E) and head.w2.shape == (E, F)
    f32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    i32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.int32).reshape(T, k)
    w1, b1, w2, b2, wl = f32(head.w1), f32(head.b1), f32(head.w2), f32(head.b2), f32(head.wl)
    cur, prev = i32(cur), i32(prev)
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float32)
    lg = np.empty((T, E), dtype=np.float64)
    _check(lib().oref_prerouter(_ptr(x), _xtype(x, bf16), T, H, E, F, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                                _ptr(wl), _ptr(cur), _ptr(prev), k, flags, _ptr(idx), _ptr(gate), _ptr(lg)),
           "oref_prerouter")
    return idx, gate, lg


def qlinear_lora(x: np.ndarray, codes: np.ndarray, scales: np.ndarray, scheme: int, A: np.ndarray | None,
                 B: np.ndarray | None, scale: float, bf16: bool = False) -> np.ndarray:
    """y = W_q x + scale * B (A x) [MW "非マージアダプターの実行"]: codes/scales of W_q
    [N][K] in the block format, A [r][K], B [N][r] fp32 (None for r = 0). Returns y [T][N] fp32."""
    x = np.ascontiguousarray(x)
    T, K = x.shape
    N = scales.shape[0]
    assert scales.shape == (N, K // 32)
    r = 0 if A is None else A.shape[0]
    if r:
        A = np.ascontiguousarray(A, dtype=np.float32)
        B = np.ascontiguousarray(B, dtype=np.float32)
        assert A.shape == (r, K) and B.shape == (N, r)
    y = np.empty((T, N), dtype=np.float32)
    _check(lib().oref_qlinear_lora(_ptr(x), _xtype(x, bf16), T, N, K, scheme, _ptr(np.ascontiguousarray(codes)),
                                   _ptr(np.ascontiguousarray(scales)), _ptr(A if r else None),
                                   _ptr(B if r else None), r, float(scale), _ptr(y)), "oref_qlinear_lora")
    return y


def topk_logits(logits: np.ndarray, k: int, flags: int = RENORM):
    """The router's softmax/top-k on given fp32 logits [T][E]: (idx [T][k], gate [T][k])."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float32)
    _check(lib().oref_topk_logits(_ptr(lg), T, E, k, flags, _ptr(idx), _ptr(gate)), "oref_topk_logits")
    return idx, gate


def group(idx: np.ndarray, E: int):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    uniq = np.empty(E, dtype=np.int32)
    n = np.zeros(1, dtype=np.int32)
    _check(lib().oref_group(_ptr(idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(uniq), _ptr(n)),
           "oref_group")
    return counts, offsets, perm, uniq[: int(n[0])].copy()


def gather_forward(x: np.ndarray, ex: Experts, idx: np.ndarray, gate: np.ndarray | None, bf16: bool = False):
    """y[T][H] (gate given) or per-slot y[T][k][H] (gate None) [QK §4, §7]."""
    x = np.ascontiguousarray(x)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    y = np.empty((T, ex.H) if gate is not None else (T, k, ex.H), dtype=np.float32)
    g = None if gate is None else np.ascontiguousarray(gate, dtype=np.float32)
    c = ex._c()
    _check(lib().oref_gather_forward(_ptr(x), _xtype(x, bf16), T, ctypes.byref(c), k, _ptr(idx), _ptr(g), _ptr(y)),
           "oref_gather_forward")
    return y


def layer_forward(x: np.ndarray, R: np.ndarray, ex: Experts, k: int, flags: int = RENORM, bf16: bool = False):
    """Router then gathered experts. Returns (y [T][H], idx [T][k], gate [T][k])."""
    x = np.ascontiguousarray(x)
    R = np.ascontiguousarray(R, dtype=np.float32)
    T = x.shape[0]
    y = np.empty((T, ex.H), dtype=np.float32)
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float32)
    c = ex._c()
    _check(lib().oref_layer_forward(_ptr(x), _xtype(x, bf16), T, _ptr(R), ctypes.byref(c), k, flags,
                                    _ptr(y), _ptr(idx), _ptr(gate)), "oref_layer_forward")
    return y, idx, gate


def dense_forward(x: np.ndarray, ex: Experts, gate_full: np.ndarray, bf16: bool = False):
    """Every expert evaluated, weighted by gate_full[T][E] (zeros for non-routed)."""
    x = np.ascontiguousarray(x)
    gate_full = np.ascontiguousarray(gate_full, dtype=np.float32)
    T = x.shape[0]
    y = np.empty((T, ex.H), dtype=np.float32)
    c = ex._c()
    _check(lib().oref_dense_forward(_ptr(x), _xtype(x, bf16), T, ctypes.byref(c), _ptr(gate_full), _ptr(y)),
           "oref_dense_forward")
    return y


class planted:
    """Context manager that plants a known mistake in the oracle (tests only)."""

    NONE, SLOT0_ACTIVATION, GATE_UP_SWAPPED, GATES_IGNORED, NIBBLE_SWAPPED, SCALE_SHIFTED = range(6)

    def __init__(self, mistake: int):
        self.mistake = mistake

    def __enter__(self):
        lib().oref_set_plant(self.mistake)
        return self

    def __exit__(self, *exc):
        lib().oref_set_plant(0)
        return False


def num_threads() -> int:
    return int(lib().oref_num_threads())


def set_num_threads(n: int) -> None:
    lib().oref_set_num_threads(int(n))
