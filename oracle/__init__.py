"""ctypes wrapper of the CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import this package.  It takes
numpy arrays (bf16 values as their uint16 bit patterns, codes as uint8) and
never imports the HIP library or its binding.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from . import build as _build

FMT_FP8_B128 = 0
FMT_NVFP4 = 1
FMT_INT8_ROW = 2
FMT_INT4_ROW = 3
FMT_INT4_G64 = 4
INT_FORMATS = (FMT_INT8_ROW, FMT_INT4_ROW, FMT_INT4_G64)
FMT_FP8_B128_BF16S = 5

_lib = None


class _Expert(C.Structure):
    _fields_ = [("gu_q", C.c_void_p), ("gu_s", C.c_void_p), ("gu_g", C.c_float),
                ("dn_q", C.c_void_p), ("dn_s", C.c_void_p), ("dn_g", C.c_float)]


class _Layer(C.Structure):
    _fields_ = [("hidden", C.c_int), ("n_experts", C.c_int), ("top_k", C.c_int),
                ("inter", C.c_int), ("shared_inter", C.c_int), ("fmt", C.c_int),
                ("router_w", C.c_void_p), ("router_bias", C.c_void_p),
                ("shared_gate_w", C.c_void_p), ("experts", C.POINTER(_Expert)),
                ("shared", C.POINTER(_Expert))]


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(_build.ensure_built())
        L = _lib
        L.orc_bf16_to_f32.argtypes = [C.c_uint16]
        L.orc_bf16_to_f32.restype = C.c_float
        L.orc_f32_to_bf16_rne.argtypes = [C.c_float]
        L.orc_f32_to_bf16_rne.restype = C.c_uint16
        L.orc_e4m3_to_f32.argtypes = [C.c_uint8]
        L.orc_e4m3_to_f32.restype = C.c_float
        L.orc_e2m1_to_f32.argtypes = [C.c_uint8]
        L.orc_e2m1_to_f32.restype = C.c_float
        L.orc_int8_to_f32.argtypes = [C.c_uint8]
        L.orc_int8_to_f32.restype = C.c_float
        L.orc_int4_to_f32.argtypes = [C.c_uint8]
        L.orc_int4_to_f32.restype = C.c_float
        L.orc_dequant_int.argtypes = [C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p]
        L.orc_dequant_fp8_bf16s.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p]
        L.orc_set_threads.argtypes = [C.c_int]
        L.orc_get_threads.restype = C.c_int
        L.orc_dequant_fp8.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p]
        L.orc_dequant_nvfp4.argtypes = [C.c_void_p, C.c_void_p, C.c_float, C.c_int, C.c_int,
                                        C.c_void_p]
        L.orc_router_logits.argtypes = [C.POINTER(_Layer), C.c_void_p, C.c_int, C.c_void_p]
        L.orc_shared_gate.argtypes = [C.POINTER(_Layer), C.c_void_p, C.c_int, C.c_void_p]
        L.orc_topk_softmax.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                       C.c_void_p]
        L.orc_group.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                                C.c_void_p]
        L.orc_expert_apply.argtypes = [C.POINTER(_Layer), C.POINTER(_Expert), C.c_int,
                                       C.c_void_p, C.c_void_p]
        L.orc_layer_forward.argtypes = [C.POINTER(_Layer), C.c_void_p, C.c_int, C.c_void_p,
                                        C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_void_p, C.c_void_p]
        L.orc_rms_norm.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_double, C.c_void_p]
        L.orc_dense_fp8.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_void_p]
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


# ------------------------------------------------------------------ formats

def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).ravel()
    f = lib().orc_bf16_to_f32
    return np.array([f(int(v)) for v in b], dtype=np.float32).reshape(np.shape(bits))


def f32_to_bf16(vals) -> np.ndarray:
    v = np.asarray(vals, dtype=np.float32).ravel()
    f = lib().orc_f32_to_bf16_rne
    return np.array([f(float(x)) for x in v], dtype=np.uint16).reshape(np.shape(vals))


def e4m3_to_f32(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).ravel()
    f = lib().orc_e4m3_to_f32
    return np.array([f(int(v)) for v in c], dtype=np.float32).reshape(np.shape(codes))


def e2m1_to_f32(nibbles) -> np.ndarray:
    c = np.asarray(nibbles, dtype=np.uint8).ravel()
    f = lib().orc_e2m1_to_f32
    return np.array([f(int(v)) for v in c], dtype=np.float32).reshape(np.shape(nibbles))


def int8_to_f32(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).ravel()
    f = lib().orc_int8_to_f32
    return np.array([f(int(v)) for v in c], dtype=np.float32).reshape(np.shape(codes))


def int4_to_f32(nibbles) -> np.ndarray:
    c = np.asarray(nibbles, dtype=np.uint8).ravel()
    f = lib().orc_int4_to_f32
    return np.array([f(int(v)) for v in c], dtype=np.float32).reshape(np.shape(nibbles))


def dequant_int(fmt: int, q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Integer-format codes (int8 [O][I] bytes, int4 [O][I/2] bytes) with f32
    scales [O][I/G] to the f32 matrix [O][I]."""
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    O, nb = q.shape
    I = nb if fmt == FMT_INT8_ROW else 2 * nb
    W = np.empty((O, I), np.float32)
    if lib().orc_dequant_int(int(fmt), _ptr(q), _ptr(scale), O, I, _ptr(W)) != 0:
        raise ValueError("orc_dequant_int rejected its arguments")
    return W


def dequant_fp8(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    O, I = q.shape
    W = np.empty((O, I), np.float32)
    if lib().orc_dequant_fp8(_ptr(q), _ptr(scale), O, I, _ptr(W)) != 0:
        raise ValueError("orc_dequant_fp8 rejected its arguments")
    return W


def dequant_fp8_bf16s(q: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """fp8 codes [O][I] with bf16 block scales (uint16 bit patterns) [O/128][I/128]."""
    q = _c(q, np.uint8)
    scale_bits = _c(scale_bits, np.uint16)
    O, I = q.shape
    W = np.empty((O, I), np.float32)
    if lib().orc_dequant_fp8_bf16s(_ptr(q), _ptr(scale_bits), O, I, _ptr(W)) != 0:
        raise ValueError("orc_dequant_fp8_bf16s rejected its arguments")
    return W


def dequant_nvfp4(q: np.ndarray, scale: np.ndarray, g: float) -> np.ndarray:
    q = _c(q, np.uint8)
    scale = _c(scale, np.uint8)
    O, half = q.shape
    W = np.empty((O, 2 * half), np.float32)
    if lib().orc_dequant_nvfp4(_ptr(q), _ptr(scale), float(g), O, 2 * half, _ptr(W)) != 0:
        raise ValueError("orc_dequant_nvfp4 rejected its arguments")
    return W


# ------------------------------------------------------------------ layers

def _scale_dtype(fmt):
    """Stored scale element type: e4m3 bytes (nvfp4), bf16 bits, else f32."""
    return {FMT_NVFP4: np.uint8, FMT_FP8_B128_BF16S: np.uint16}.get(fmt, np.float32)


@dataclass
class Expert:
    """One expert's stored weights (numpy).  fp8: gu_s/dn_s are f32 block
    scales; nvfp4: e4m3 scale bytes plus the f32 globals gu_g/dn_g; integer
    formats: f32 row or group scales."""
    gu_q: np.ndarray
    gu_s: np.ndarray
    dn_q: np.ndarray
    dn_s: np.ndarray
    gu_g: float = 1.0
    dn_g: float = 1.0


class Layer:
    """Holds numpy weights of one layer and the C view of them.

    experts: mapping expert index -> Expert; experts never routed to may be
    left out (their table entries stay NULL and the oracle rejects a call that
    would read them)."""

    def __init__(self, hidden, n_experts, top_k, inter, shared_inter, fmt,
                 router_w=None, router_bias=None, shared_gate_w=None,
                 experts: Optional[Dict[int, Expert]] = None, shared: Optional[Expert] = None):
        self.hidden, self.n_experts, self.top_k = int(hidden), int(n_experts), int(top_k)
        self.inter, self.shared_inter, self.fmt = int(inter), int(shared_inter), int(fmt)
        sdt = _scale_dtype(fmt)
        self._keep = []
        self.router_w = _c(router_w, np.uint16)
        self.router_bias = _c(router_bias, np.float32)
        self.shared_gate_w = _c(shared_gate_w, np.uint16)
        self._experts = (_Expert * self.n_experts)()
        for e, X in (experts or {}).items():
            self._experts[e] = self._mk(X, sdt)
        self._shared = None
        if shared is not None:
            self._shared = self._mk(shared, sdt)
        self._c = _Layer(self.hidden, self.n_experts, self.top_k, self.inter, self.shared_inter,
                         self.fmt, _ptr(self.router_w), _ptr(self.router_bias),
                         _ptr(self.shared_gate_w),
                         C.cast(self._experts, C.POINTER(_Expert)),
                         C.pointer(self._shared) if self._shared is not None else None)

    def _mk(self, X: Expert, sdt):
        arrs = [_c(X.gu_q, np.uint8), _c(X.gu_s, sdt), _c(X.dn_q, np.uint8), _c(X.dn_s, sdt)]
        self._keep.extend(arrs)
        return _Expert(_ptr(arrs[0]), _ptr(arrs[1]), float(X.gu_g),
                       _ptr(arrs[2]), _ptr(arrs[3]), float(X.dn_g))

    @property
    def cptr(self):
        return C.byref(self._c)


def router_logits(layer: Layer, x: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    R = x.shape[0]
    out = np.empty((R, layer.n_experts), np.float32)
    if lib().orc_router_logits(layer.cptr, _ptr(x), R, _ptr(out)) != 0:
        raise ValueError("orc_router_logits rejected its arguments")
    return out


def shared_gate(layer: Layer, x: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    R = x.shape[0]
    out = np.empty((R,), np.float32)
    if lib().orc_shared_gate(layer.cptr, _ptr(x), R, _ptr(out)) != 0:
        raise ValueError("orc_shared_gate rejected its arguments")
    return out


def topk_softmax(logits: np.ndarray, k: int):
    logits = _c(logits, np.float32)
    R, E = logits.shape
    ids = np.empty((R, k), np.int32)
    w = np.empty((R, k), np.float32)
    if lib().orc_topk_softmax(_ptr(logits), R, E, int(k), _ptr(ids), _ptr(w)) != 0:
        raise ValueError("orc_topk_softmax rejected its arguments")
    return ids, w


def group(ids: np.ndarray, n_experts: int):
    ids = _c(ids, np.int32)
    R, k = ids.shape
    counts = np.empty((n_experts,), np.int32)
    offsets = np.empty((n_experts + 1,), np.int32)
    perm = np.empty((R * k,), np.int32)
    if lib().orc_group(_ptr(ids), R, k, int(n_experts), _ptr(counts), _ptr(offsets),
                       _ptr(perm)) != 0:
        raise ValueError("orc_group rejected its arguments")
    return counts, offsets, perm


def expert_apply(layer: Layer, expert: Expert, inter: int, x_row: np.ndarray) -> np.ndarray:
    sdt = _scale_dtype(layer.fmt)
    keep = []
    cx = layer._mk(expert, sdt)
    keep.append(cx)
    x_row = _c(x_row, np.uint16)
    d = np.empty((layer.hidden,), np.float64)
    if lib().orc_expert_apply(layer.cptr, C.byref(cx), int(inter), _ptr(x_row), _ptr(d)) != 0:
        raise ValueError("orc_expert_apply rejected its arguments")
    return d


def layer_forward(layer: Layer, x: np.ndarray, logits_in: Optional[np.ndarray] = None,
                  residual: Optional[np.ndarray] = None) -> dict:
    x = _c(x, np.uint16)
    R = x.shape[0]
    H, k = layer.hidden, layer.top_k
    logits_in = _c(logits_in, np.float32)
    residual = _c(residual, np.uint16)
    ids = np.empty((R, k), np.int32)
    w = np.empty((R, k), np.float32)
    s = np.empty((R,), np.float32)
    y = np.empty((R, H), np.float32)
    out = np.empty((R, H), np.uint16)
    rc = lib().orc_layer_forward(layer.cptr, _ptr(x), R, _ptr(logits_in), _ptr(residual),
                                 _ptr(ids), _ptr(w), _ptr(s), _ptr(y), _ptr(out))
    if rc != 0:
        raise ValueError(f"orc_layer_forward failed ({rc})")
    return {"ids": ids, "w": w, "s": s, "y": y, "out": out}


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of bf16 rows (uint16 bit patterns [R][H]) with bf16 weights
    gamma [H]: x / sqrt(mean(x^2) + eps) * gamma, one bf16 rounding."""
    x = _c(np.atleast_2d(x), np.uint16)
    gamma = _c(gamma, np.uint16)
    R, H = x.shape
    if gamma.shape != (H,):
        raise ValueError("gamma must have one value per column")
    out = np.empty((R, H), np.uint16)
    if lib().orc_rms_norm(_ptr(x), R, H, _ptr(gamma), float(eps), _ptr(out)) != 0:
        raise ValueError("orc_rms_norm rejected its arguments")
    return out


def dense_fp8(q: np.ndarray, scale: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = x . dequant(W)^T in double: q e4m3 codes [N][K], scale f32
    [N/128][K/128], x bf16 bit patterns [R][K]."""
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    x = _c(np.atleast_2d(x), np.uint16)
    N, K = q.shape
    R = x.shape[0]
    if x.shape[1] != K or scale.shape != (N // 128, K // 128):
        raise ValueError("shape mismatch")
    y = np.empty((R, N), np.float64)
    if lib().orc_dense_fp8(_ptr(q), _ptr(scale), N, K, _ptr(x), R, _ptr(y)) != 0:
        raise ValueError("orc_dense_fp8 rejected its arguments")
    return y
