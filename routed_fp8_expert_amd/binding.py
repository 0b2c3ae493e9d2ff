"""ctypes binding of the C ABI in include/moe.h (and include/moe_debug.h).

Argument marshalling only: every function takes torch device tensors (or
None for NULL), passes their addresses and the current HIP stream to the
library of the same name, and raises MoeError on a non-zero status.  No step
of the layer runs here; the library must be built (build.py), and loading
fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

# The in-tree build; MOE_LIBRARY names another build of the same sources.
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_ffn.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED_SHAPE = -2
MOE_ERR_MISALIGNED = -3
MOE_ERR_WORKSPACE_TOO_SMALL = -4
MOE_ERR_HIP = -5
MOE_ERR_DEVICE_LOST = -6
MOE_ERR_TOO_MANY_CTX = -7

MOE_WFMT_FP8_E4M3_B128 = 0
MOE_WFMT_NVFP4 = 1
MOE_WFMT_INT8_ROW = 2
MOE_WFMT_INT4_ROW = 3
MOE_WFMT_INT4_G64 = 4
MOE_WFMT_FP8_E4M3_B128_BF16S = 5

KERNELS = ["router", "topk", "group", "gate_up", "down", "blend", "mfma_gate_up", "mfma_down", "layer", "norm", "dense"]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} ({status})")
        self.status = status


class ExpertWeights(C.Structure):
    _fields_ = [("gate_up", C.c_void_p), ("gate_up_scale", C.c_void_p),
                ("gate_up_global", C.c_void_p), ("down", C.c_void_p),
                ("down_scale", C.c_void_p), ("down_global", C.c_void_p),
                ("gate_up_stride", C.c_int64), ("gate_up_scale_stride", C.c_int64),
                ("down_stride", C.c_int64), ("down_scale_stride", C.c_int64)]


class LayerWeightsC(C.Structure):
    _fields_ = [("struct_size", C.c_size_t), ("hidden", C.c_int), ("n_experts", C.c_int),
                ("top_k", C.c_int), ("inter", C.c_int), ("shared_inter", C.c_int),
                ("weight_format", C.c_int), ("router_w", C.c_void_p),
                ("router_bias", C.c_void_p), ("shared_gate_w", C.c_void_p),
                ("routed", ExpertWeights), ("shared", ExpertWeights)]


class RoutingC(C.Structure):
    _fields_ = [("struct_size", C.c_size_t), ("topk_ids", C.c_void_p), ("topk_w", C.c_void_p),
                ("shared_gate", C.c_void_p), ("expert_count", C.c_void_p),
                ("expert_offset", C.c_void_p), ("perm", C.c_void_p), ("logits", C.c_void_p)]


class NormC(C.Structure):
    """moe_norm: the RMSNorm epilogue of moe_layer_forward_norm."""
    _fields_ = [("struct_size", C.c_size_t), ("weight", C.c_void_p), ("eps", C.c_float),
                ("out", C.c_void_p), ("ldo", C.c_int64)]


class DenseWeightsC(C.Structure):
    """moe_dense_weights: e4m3 codes [n][ldw] with f32 scales [n/128][k/128]."""
    _fields_ = [("struct_size", C.c_size_t), ("codes", C.c_void_p), ("ldw", C.c_int64),
                ("scales", C.c_void_p), ("n", C.c_int32), ("k", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"the HIP library is not built ({LIB_PATH} missing); "
                               "run routed_fp8_expert_amd/build.py or __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
        sig = {
            "moe_abi_version": ([], i32),
            "moe_strerror": ([i32], C.c_char_p),
            "moe_ctx_create": ([i32, C.POINTER(vp)], i32),
            "moe_ctx_destroy": ([vp], i32),
            "moe_ctx_status": ([vp], i32),
            "moe_ctx_set_fault_at": ([vp, i64], i32),
            "moe_ctx_set_mfma_min_rows": ([vp, i32], i32),
            "moe_ctx_set_force_arm": ([vp, i32], i32),
            "moe_ctx_set_one_row_path": ([vp, i32], i32),
            "moe_ctx_set_few_rows": ([vp, i32], i32),
            "moe_ctx_device_errors": ([vp, C.POINTER(C.c_uint32), i32], i32),
            "moe_ctx_set_wait_limit": ([vp, i64], i32),
            "moe_ctx_set_timing": ([vp, i32], i32),
            "moe_ctx_kernel_stats": ([vp, i32, C.POINTER(C.c_double), C.POINTER(i64)], i32),
            "moe_workspace_bytes": ([C.POINTER(LayerWeightsC), i32], sz),
            "moe_route": ([vp, C.POINTER(LayerWeightsC), vp, i32, i64, vp, C.POINTER(RoutingC),
                           vp, sz, vp], i32),
            "moe_expert_ffn": ([vp, C.POINTER(LayerWeightsC), vp, i32, i64, C.POINTER(RoutingC),
                                vp, vp, i64, vp, sz, vp], i32),
            "moe_layer_forward": ([vp, C.POINTER(LayerWeightsC), vp, i32, i64, vp,
                                   C.POINTER(RoutingC), vp, vp, i64, vp, sz, vp], i32),
            "moe_layer_forward_static": ([vp, C.POINTER(LayerWeightsC), vp, i32, i64, vp,
                                          C.POINTER(RoutingC), vp, vp, i64, vp], i32),
            "moe_layer_forward_norm": ([vp, C.POINTER(LayerWeightsC), vp, i32, i64, vp,
                                        C.POINTER(RoutingC), vp, vp, i64, C.POINTER(NormC), vp, sz, vp], i32),
            "moe_dense_fp8": ([vp, C.POINTER(DenseWeightsC), vp, i32, i64, vp, i64, vp], i32),
            "moe_debug_decode": ([vp, i32, vp, vp, i32, vp], i32),
            "moe_debug_set_phase_stamps": ([vp, vp, i64, C.POINTER(i64)], i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().moe_strerror(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------ ctx

class Ctx:
    """Owns a moe_ctx handle (moe_ctx_create / moe_ctx_destroy)."""

    def __init__(self, device: int = 0):
        h = C.c_void_p()
        _check(lib().moe_ctx_create(int(device), C.byref(h)), "moe_ctx_create")
        self.handle = h
        self.device = int(device)

    def close(self):
        if self.handle is not None and self.handle.value:
            lib().moe_ctx_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def moe_abi_version() -> int:
    return int(lib().moe_abi_version())


def moe_ctx_create(device: int = 0) -> Ctx:
    return Ctx(device)


def moe_ctx_destroy(ctx: Ctx) -> None:
    ctx.close()


def moe_ctx_status(ctx: Ctx) -> int:
    return int(lib().moe_ctx_status(ctx.handle))


def moe_ctx_set_fault_at(ctx: Ctx, n: int) -> None:
    _check(lib().moe_ctx_set_fault_at(ctx.handle, int(n)), "moe_ctx_set_fault_at")


def moe_ctx_set_mfma_min_rows(ctx: Ctx, rows: int) -> None:
    _check(lib().moe_ctx_set_mfma_min_rows(ctx.handle, int(rows)), "moe_ctx_set_mfma_min_rows")


def moe_ctx_set_force_arm(ctx: Ctx, arm: int) -> None:
    _check(lib().moe_ctx_set_force_arm(ctx.handle, int(arm)), "moe_ctx_set_force_arm")


def moe_ctx_set_one_row_path(ctx: Ctx, path: int) -> None:
    _check(lib().moe_ctx_set_one_row_path(ctx.handle, int(path)), "moe_ctx_set_one_row_path")


def moe_ctx_set_few_rows(ctx: Ctx, rows: int) -> None:
    _check(lib().moe_ctx_set_few_rows(ctx.handle, int(rows)), "moe_ctx_set_few_rows")


def moe_ctx_device_errors(ctx: Ctx, clear: bool = True) -> int:
    v = C.c_uint32(0)
    _check(lib().moe_ctx_device_errors(ctx.handle, C.byref(v), int(clear)), "moe_ctx_device_errors")
    return int(v.value)


def moe_ctx_set_wait_limit(ctx: Ctx, us: int) -> None:
    _check(lib().moe_ctx_set_wait_limit(ctx.handle, int(us)), "moe_ctx_set_wait_limit")


def moe_ctx_set_timing(ctx: Ctx, enable: bool) -> None:
    _check(lib().moe_ctx_set_timing(ctx.handle, int(enable)), "moe_ctx_set_timing")


def moe_ctx_kernel_stats(ctx: Ctx, kernel: int):
    ms, n = C.c_double(0.0), C.c_int64(0)
    _check(lib().moe_ctx_kernel_stats(ctx.handle, int(kernel), C.byref(ms), C.byref(n)),
           "moe_ctx_kernel_stats")
    return float(ms.value), int(n.value)


# ------------------------------------------------------------------ weights

class LayerWeights:
    """moe_layer_weights over torch device tensors (kept alive here).

    Routed tensors are stacked per expert along dim 0 (byte strides are taken
    from the tensors); shared tensors hold one expert ([1, ...] or unstacked).
    Key names: router_w, router_bias, shared_gate_w, gu_q, gu_s, gu_g, dn_q,
    dn_s, dn_g and sh_-prefixed copies for the shared expert."""

    def __init__(self, hidden, n_experts, top_k, inter, shared_inter, weight_format, tensors: dict):
        self.tensors = {k: v for k, v in tensors.items() if v is not None}
        t = self.tensors
        c = LayerWeightsC()
        c.struct_size = C.sizeof(LayerWeightsC)
        c.hidden, c.n_experts, c.top_k = int(hidden), int(n_experts), int(top_k)
        c.inter, c.shared_inter, c.weight_format = int(inter), int(shared_inter), int(weight_format)
        c.router_w = _p(t.get("router_w"))
        c.router_bias = _p(t.get("router_bias"))
        c.shared_gate_w = _p(t.get("shared_gate_w"))
        c.routed = self._family("")
        if shared_inter > 0:
            c.shared = self._family("sh_")
        self.c = c
        self.hidden, self.n_experts, self.top_k = c.hidden, c.n_experts, c.top_k
        self.inter, self.shared_inter, self.weight_format = c.inter, c.shared_inter, c.weight_format

    def _family(self, pre):
        t = self.tensors
        f = ExpertWeights()

        def stride(x):
            return x.stride(0) * x.element_size() if x.dim() >= 3 else 0

        f.gate_up, f.gate_up_scale = _p(t.get(pre + "gu_q")), _p(t.get(pre + "gu_s"))
        f.down, f.down_scale = _p(t.get(pre + "dn_q")), _p(t.get(pre + "dn_s"))
        f.gate_up_global, f.down_global = _p(t.get(pre + "gu_g")), _p(t.get(pre + "dn_g"))
        if pre + "gu_q" in t:
            f.gate_up_stride = stride(t[pre + "gu_q"])
            f.gate_up_scale_stride = stride(t[pre + "gu_s"])
            f.down_stride = stride(t[pre + "dn_q"])
            f.down_scale_stride = stride(t[pre + "dn_s"])
        return f

    @property
    def ref(self):
        return C.byref(self.c)


class Routing:
    """Caller-owned routing arrays (moe_routing) as torch device tensors."""

    def __init__(self, rows, n_experts, top_k, device, logits=False, grouping=True):
        dev = torch.device(device)
        self.topk_ids = torch.empty((rows, top_k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((rows, top_k), dtype=torch.float32, device=dev)
        self.shared_gate = torch.empty((rows,), dtype=torch.float32, device=dev)
        # grouping arrays: optional for moe_layer_forward (NULL when not asked for)
        self.expert_count = torch.empty((n_experts,), dtype=torch.int32, device=dev) if grouping else None
        self.expert_offset = torch.empty((n_experts + 1,), dtype=torch.int32, device=dev) if grouping else None
        self.perm = torch.empty((rows * top_k,), dtype=torch.int32, device=dev) if grouping else None
        self.logits = (torch.empty((rows, n_experts), dtype=torch.float32, device=dev)
                       if logits else None)
        self.c = RoutingC(C.sizeof(RoutingC), _p(self.topk_ids), _p(self.topk_w),
                          _p(self.shared_gate), _p(self.expert_count), _p(self.expert_offset),
                          _p(self.perm), _p(self.logits))

    @property
    def ref(self):
        return C.byref(self.c)


def moe_workspace_bytes(w: LayerWeights, rows: int) -> int:
    return int(lib().moe_workspace_bytes(w.ref, int(rows)))


def workspace(w: LayerWeights, rows: int, device) -> torch.Tensor:
    n = moe_workspace_bytes(w, rows)
    if n == 0 and rows > 0:
        raise MoeError(MOE_ERR_INVALID_ARG, "moe_workspace_bytes")
    return torch.empty((max(n, 256),), dtype=torch.uint8, device=device)


def _ld(t: Optional[torch.Tensor], hidden: int) -> int:
    if t is None:
        return hidden
    return t.stride(0) if t.dim() == 2 else hidden


def moe_route(ctx: Ctx, w: LayerWeights, x: torch.Tensor, routing: Routing, ws: torch.Tensor,
              logits_in: Optional[torch.Tensor] = None, stream=None) -> None:
    rows = x.shape[0]
    _check(lib().moe_route(ctx.handle, w.ref, _p(x), rows, _ld(x, w.hidden), _p(logits_in),
                           routing.ref, _p(ws), ws.numel(), _stream(stream)), "moe_route")


def moe_expert_ffn(ctx: Ctx, w: LayerWeights, x: torch.Tensor, routing: Routing,
                   y: Optional[torch.Tensor], residual: Optional[torch.Tensor], ws: torch.Tensor,
                   stream=None) -> None:
    rows = x.shape[0]
    ldy = _ld(y if y is not None else residual, w.hidden)
    _check(lib().moe_expert_ffn(ctx.handle, w.ref, _p(x), rows, _ld(x, w.hidden), routing.ref,
                                _p(y), _p(residual), ldy, _p(ws), ws.numel(), _stream(stream)),
           "moe_expert_ffn")


def moe_layer_forward(ctx: Ctx, w: LayerWeights, x: torch.Tensor, y: Optional[torch.Tensor],
                      residual: Optional[torch.Tensor], ws: torch.Tensor,
                      logits_in: Optional[torch.Tensor] = None, routing: Optional[Routing] = None,
                      stream=None) -> None:
    rows = x.shape[0]
    ldy = _ld(y if y is not None else residual, w.hidden)
    _check(lib().moe_layer_forward(ctx.handle, w.ref, _p(x), rows, _ld(x, w.hidden),
                                   _p(logits_in), routing.ref if routing is not None else None,
                                   _p(y), _p(residual), ldy, _p(ws), ws.numel(), _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_static(ctx: Ctx, w: LayerWeights, x: torch.Tensor, y: Optional[torch.Tensor],
                             residual: Optional[torch.Tensor], logits_in: Optional[torch.Tensor] = None,
                             routing: Optional[Routing] = None, stream=None) -> None:
    """moe_layer_forward on the library's static device scratch (no workspace argument)."""
    rows = x.shape[0]
    ldy = _ld(y if y is not None else residual, w.hidden)
    _check(lib().moe_layer_forward_static(ctx.handle, w.ref, _p(x), rows, _ld(x, w.hidden), _p(logits_in),
                                          routing.ref if routing is not None else None, _p(y), _p(residual),
                                          ldy, _stream(stream)),
           "moe_layer_forward_static")


def moe_layer_forward_norm(ctx: Ctx, w: LayerWeights, x: torch.Tensor, y: Optional[torch.Tensor],
                           residual: Optional[torch.Tensor], ws: torch.Tensor, norm_weight: torch.Tensor,
                           eps: float, norm_out: torch.Tensor, logits_in: Optional[torch.Tensor] = None,
                           routing: Optional[Routing] = None, stream=None) -> None:
    """moe_layer_forward plus the RMSNorm of every output row into norm_out."""
    rows = x.shape[0]
    ldy = _ld(y if y is not None else residual, w.hidden)
    n = NormC(C.sizeof(NormC), _p(norm_weight), float(eps), _p(norm_out), _ld(norm_out, w.hidden))
    _check(lib().moe_layer_forward_norm(ctx.handle, w.ref, _p(x), rows, _ld(x, w.hidden),
                                        _p(logits_in), routing.ref if routing is not None else None,
                                        _p(y), _p(residual), ldy, C.byref(n), _p(ws), ws.numel(),
                                        _stream(stream)),
           "moe_layer_forward_norm")


class DenseWeights:
    """A dense fp8 block-128 matrix for moe_dense_fp8: codes u8 [n][k] (row
    stride codes.stride(0) bytes) and scales f32 [n/128][k/128], device
    tensors the caller keeps alive."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor):
        n, k = codes.shape
        self.codes, self.scales = codes, scales
        self.n, self.k = n, k
        self.ref = DenseWeightsC(C.sizeof(DenseWeightsC), _p(codes), codes.stride(0), _p(scales), n, k)


def moe_dense_fp8(ctx: Ctx, w: DenseWeights, x: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """y[r] = x[r] . dequant(W)^T in bf16 (one launch)."""
    _check(lib().moe_dense_fp8(ctx.handle, C.byref(w.ref), _p(x), x.shape[0], _ld(x, w.k), _p(y),
                               _ld(y, w.n), _stream(stream)), "moe_dense_fp8")


def moe_debug_decode(ctx: Ctx, fmt: int, codes: torch.Tensor, out: torch.Tensor,
                     stream=None) -> None:
    _check(lib().moe_debug_decode(ctx.handle, int(fmt), _p(codes), _p(out), codes.numel(),
                                  _stream(stream)), "moe_debug_decode")


def moe_debug_set_phase_stamps(ctx: Ctx, stamps: Optional[torch.Tensor]) -> int:
    """Phase stamps of the one-launch layer into an int64 device tensor (None:
    off); returns the constant clock's rate in kHz."""
    n = 0 if stamps is None else stamps.numel()
    khz = C.c_int64(0)
    _check(lib().moe_debug_set_phase_stamps(ctx.handle, _p(stamps), n, C.byref(khz)), "moe_debug_set_phase_stamps")
    return int(khz.value)
