"""Seeded synthetic inputs for the decode-step MoE FFN.

This module serves both the HIP path and the CPU oracle.  It holds none of the
layer's arithmetic: it draws random numbers, encodes weights into their stored
formats (the inverse of the decoders the two sides implement on their own),
and shapes them like the pages' models.  Every tensor comes from a torch
Generator seeded by a stable hash of (base seed, workload, layer, tensor,
chunk, attempt), so a run can be rebuilt exactly on the same device type.

Workloads (shapes from the GB10 blueprint for Qwen3.6-35B-A3B-FP8, header:
256-expert top-8 with a shared expert, 40 layers; "Inspecting
Qwen3.5-397B-A17B-NVFP4", "The Architectural Revelations": hidden 4096, 60
layers, 512 experts, 10 per token, NVFP4):

  tiny      H 256,  E 16,  k 2,  I 128,  fp8-b128, 1 layer, router bias 1e-3*e
  a3b       H 2048, E 256, k 8,  I 512,  fp8-b128, 40 layers, router GEMV
  a3b_multi as a3b, rows 2..64, router logits iid U(0,1)
  a17b      H 4096, E 512, k 10, I 1024, nvfp4, 12 layers, router GEMV
  a3b_zipf  as a3b, rows 64 and 512, Gumbel-top-k logits with Zipf(1.2)
  a3b_i8, a3b_i4, a3b_i4g64   as a3b with int8 per-row, int4 per-row and
            int4-g64 experts (colibri PR: per-row int4 and int4-g64 experts)
  tiny_i4g64  as tiny with int4-g64 experts
  a3b_f8bs, tiny_f8bs   as a3b / tiny with bf16 block scales (colibri PR: fp8
            experts with BF16 128x128 block scales)
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

BASE_SEED = 20261203
FP8_MAX = 448.0
E2M1_MAX = 6.0

FMT_FP8_B128 = 0
FMT_NVFP4 = 1
FMT_INT8_ROW = 2
FMT_INT4_ROW = 3
FMT_INT4_G64 = 4
INT_FORMATS = (FMT_INT8_ROW, FMT_INT4_ROW, FMT_INT4_G64)
FMT_FP8_B128_BF16S = 5


@dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    fmt: int
    layers: int
    rows: List[int] = field(default_factory=lambda: [1])
    router: str = "gemv"           # "gemv" | "uniform" | "zipf"
    router_bias: bool = False
    rms_norm_x: bool = True
    weight_std: float = 0.02


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 256, 16, 2, 128, 128, FMT_FP8_B128, 1, [1], "gemv", True, False),
    "a3b": Workload("a3b", 2048, 256, 8, 512, 512, FMT_FP8_B128, 40, [1]),
    "a3b_multi": Workload("a3b_multi", 2048, 256, 8, 512, 512, FMT_FP8_B128, 40,
                          [2, 4, 8, 16, 32, 64], "uniform"),
    "a17b": Workload("a17b", 4096, 512, 10, 1024, 1024, FMT_NVFP4, 12, [1, 8]),
    "a3b_zipf": Workload("a3b_zipf", 2048, 256, 8, 512, 512, FMT_FP8_B128, 40, [64, 512],
                         "zipf"),
    "a3b_i8": Workload("a3b_i8", 2048, 256, 8, 512, 512, FMT_INT8_ROW, 40, [1, 8]),
    "a3b_i4": Workload("a3b_i4", 2048, 256, 8, 512, 512, FMT_INT4_ROW, 40, [1, 8]),
    "a3b_i4g64": Workload("a3b_i4g64", 2048, 256, 8, 512, 512, FMT_INT4_G64, 40, [1, 8]),
    "a3b_f8bs": Workload("a3b_f8bs", 2048, 256, 8, 512, 512, FMT_FP8_B128_BF16S, 40, [1, 8]),
    "tiny_f8bs": Workload("tiny_f8bs", 256, 16, 2, 128, 128, FMT_FP8_B128_BF16S, 1, [1], "gemv", True, False),
    "tiny_i4g64": Workload("tiny_i4g64", 256, 16, 2, 128, 128, FMT_INT4_G64, 1, [1], "gemv", True, False),
}


def subseed(*parts) -> int:
    """Stable 63-bit seed from any tuple of ints and strings."""
    h = hashlib.blake2b(repr((BASE_SEED,) + tuple(parts)).encode(), digest_size=8)
    return int.from_bytes(h.digest(), "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(subseed(*parts))
    return g


# ----------------------------------------------------------------- encoders

def quant_fp8_b128(w: torch.Tensor):
    """Encode f32 weights [..., O, I] as OCP e4m3 codes with one f32 scale per
    128x128 block: scale = amax/448 (1 for an all-zero block), codes = the
    torch e4m3 cast of w/scale clamped to +-448.  Returns (codes u8, scales
    f32 [..., O/128, I/128])."""
    *lead, O, I = w.shape
    assert O % 128 == 0 and I % 128 == 0
    b = w.reshape(*lead, O // 128, 128, I // 128, 128)
    amax = b.abs().amax(dim=(-3, -1))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    v = (b / scale[..., :, None, :, None]).clamp(-FP8_MAX, FP8_MAX)
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, O, I)
    return codes.contiguous(), scale.to(torch.float32).contiguous()


_E2M1_MID = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def quant_nvfp4(w: torch.Tensor):
    """Encode f32 weights [..., O, I] in the NVFP4 layout: a global f32 scale
    g = amax/(448*6) per matrix, one e4m3 scale per 16 columns
    (amax_block/(6g), torch e4m3 cast), e2m1 codes by nearest magnitude, two
    per byte with the even column in the low nibble.  Returns
    (packed u8 [..., O, I/2], scales u8 [..., O, I/16], g f32 [...])."""
    *lead, O, I = w.shape
    assert I % 16 == 0
    amax = w.abs().amax(dim=(-2, -1))
    g = torch.where(amax > 0, amax / (FP8_MAX * E2M1_MAX), torch.ones_like(amax))
    blk = w.reshape(*lead, O, I // 16, 16)
    bamax = blk.abs().amax(dim=-1)
    sc = (bamax / (E2M1_MAX * g[..., None, None])).clamp(max=FP8_MAX).to(torch.float8_e4m3fn)
    scf = sc.to(torch.float32) * g[..., None, None]
    v = torch.where(scf[..., None] > 0, blk / scf[..., None], torch.zeros_like(blk))
    mag = v.abs().clamp(max=E2M1_MAX)
    idx = torch.bucketize(mag, _E2M1_MID.to(w.device))
    code = (idx | ((v < 0) & (idx > 0)).to(idx.dtype) << 3).to(torch.uint8)
    code = code.reshape(*lead, O, I)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).contiguous()
    return packed, sc.view(torch.uint8).contiguous(), g.to(torch.float32).contiguous()


def quant_fp8_b128_bf16s(w: torch.Tensor):
    """As quant_fp8_b128 with the block scale rounded to bf16 first (the codes
    are taken against the rounded scale).  Returns (codes u8, scales bf16
    [..., O/128, I/128])."""
    *lead, O, I = w.shape
    b = w.reshape(*lead, O // 128, 128, I // 128, 128)
    amax = b.abs().amax(dim=(-3, -1))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.bfloat16)
    v = (b / scale.to(torch.float32)[..., :, None, :, None]).clamp(-FP8_MAX, FP8_MAX)
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, O, I)
    return codes.contiguous(), scale.contiguous()


def quant_int(w: torch.Tensor, fmt: int):
    """Encode f32 weights [..., O, I] in an integer format: symmetric codes
    round(w / scale) clamped to +-qmax (127 for int8, 7 for int4), one f32
    scale amax/qmax per group of G consecutive input columns of a row (G = I
    per row, 64 for g64; 1 for an all-zero group).  int8 codes are bytes
    [..., O, I]; int4 codes two per byte, the even column in the low nibble,
    [..., O, I/2].  Returns (codes u8, scales f32 [..., O, I/G])."""
    *lead, O, I = w.shape
    G = 64 if fmt == FMT_INT4_G64 else I
    qmax = 127.0 if fmt == FMT_INT8_ROW else 7.0
    assert I % G == 0
    b = w.reshape(*lead, O, I // G, G)
    amax = b.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / qmax, torch.ones_like(amax))
    code = torch.round(b / scale[..., None]).clamp(-qmax, qmax).to(torch.int32).reshape(*lead, O, I)
    if fmt == FMT_INT8_ROW:
        packed = (code & 0xFF).to(torch.uint8)
    else:
        nib = code & 0xF
        packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).to(torch.uint8)
    return packed.contiguous(), scale.to(torch.float32).contiguous()


# ----------------------------------------------------------------- weights

EXPERT_CHUNK = 32


def _normal(shape, std, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def _encode(w: torch.Tensor, fmt: int):
    if fmt == FMT_FP8_B128:
        q, s = quant_fp8_b128(w)
        return q, s, None
    if fmt in INT_FORMATS:
        q, s = quant_int(w, fmt)
        return q, s, None
    if fmt == FMT_FP8_B128_BF16S:
        q, s = quant_fp8_b128_bf16s(w)
        return q, s, None
    return quant_nvfp4(w)


def make_layer_weights(wl: Workload, layer: int, device="cpu", n_experts: Optional[int] = None):
    """All weights of one layer as device tensors.

    Keys: router_w (bf16 [E,H]), router_bias (f32 [E] or None), shared_gate_w
    (bf16 [H]), gu_q/gu_s[/gu_g] for the routed experts stacked [E, ...],
    dn_q/dn_s[/dn_g], and sh_gu_q/... for the shared expert ([1, ...]).
    Weights are N(0, std) before encoding.  Experts are drawn in chunks of
    EXPERT_CHUNK, each chunk with its own seed."""
    E = wl.n_experts if n_experts is None else n_experts
    H, I, Is, std = wl.hidden, wl.inter, wl.shared_inter, wl.weight_std
    out = {}
    g = _gen(device, wl.name, layer, "router")
    out["router_w"] = _normal((E, H), std, g, device).to(torch.bfloat16)
    out["router_bias"] = (1e-3 * torch.arange(E, dtype=torch.float32, device=device)
                          if wl.router_bias else None)
    g = _gen(device, wl.name, layer, "shared_gate")
    out["shared_gate_w"] = _normal((H,), std, g, device).to(torch.bfloat16)

    def stack(kind, rows, cols, count, tag):
        qs, ss, gs = [], [], []
        for c0 in range(0, count, EXPERT_CHUNK):
            n = min(EXPERT_CHUNK, count - c0)
            gen = _gen(device, wl.name, layer, tag, kind, c0)
            q, s, gg = _encode(_normal((n, rows, cols), std, gen, device), wl.fmt)
            qs.append(q)
            ss.append(s)
            if gg is not None:
                gs.append(gg)
        return (torch.cat(qs), torch.cat(ss), torch.cat(gs) if gs else None)

    for kind, rows, cols in (("gu", 2 * I, H), ("dn", H, I)):
        q, s, gg = stack(kind, rows, cols, E, "routed")
        out[kind + "_q"], out[kind + "_s"] = q, s
        if gg is not None:
            out[kind + "_g"] = gg
    if Is > 0:
        for kind, rows, cols in (("gu", 2 * Is, H), ("dn", H, Is)):
            q, s, gg = stack(kind, rows, cols, 1, "shared")
            out["sh_" + kind + "_q"], out["sh_" + kind + "_s"] = q, s
            if gg is not None:
                out["sh_" + kind + "_g"] = gg
    return out


# ----------------------------------------------------------------- dense projections

# Dense fp8 block-128 projections next to the experts (GB10 blueprint,
# "Kernels": w8a16_gemm_pipelined_m32): the pages give no shapes, so two
# stand-ins into and out of the 35B-A3B hidden size, and a small ragged one.
DENSE_SHAPES: Dict[str, tuple] = {
    "up_4096x2048": (4096, 2048),      # (n, k): hidden 2048 -> 4096
    "down_2048x4096": (2048, 4096),    # 4096 -> hidden 2048
    "small_384x640": (384, 640),
    "wide_256x8192": (256, 8192),
}


def make_dense_weights(name: str, n: int, k: int, device="cpu", std: float = 0.02):
    """A dense matrix N(0, std) [n, k] encoded fp8 block-128: (codes u8 [n, k],
    scales f32 [n/128, k/128])."""
    g = _gen(device, "dense", name, n, k)
    return quant_fp8_b128(_normal((n, k), std, g, device))


def make_dense_x(name: str, rows: int, k: int, device="cpu") -> torch.Tensor:
    """Activation rows for a dense projection, bf16 [rows, k], N(0, 1)."""
    g = _gen(device, "dense-x", name, rows, k)
    return torch.randn((rows, k), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


# ----------------------------------------------------------------- activations

def make_x(wl: Workload, layer: int, rows: int, attempt: int = 0, device="cpu") -> torch.Tensor:
    """Activation rows, bf16 [rows, H]: N(0,1), RMS-normalised per row
    (x / sqrt(mean(x^2) + 1e-6), unit weight) for every workload but tiny."""
    g = _gen(device, wl.name, layer, "x", rows, attempt)
    x = torch.randn((rows, wl.hidden), generator=g, device=device, dtype=torch.float32)
    if wl.rms_norm_x:
        x = x / torch.sqrt(x.pow(2).mean(dim=-1, keepdim=True) + 1e-6)
    return x.to(torch.bfloat16)


def make_residual(wl: Workload, layer: int, rows: int, device="cpu") -> torch.Tensor:
    g = _gen(device, wl.name, layer, "residual", rows)
    return torch.randn((rows, wl.hidden), generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def make_logits_in(wl: Workload, layer: int, rows: int, device="cpu") -> Optional[torch.Tensor]:
    """Router logits given directly (the router GEMV is then skipped):
    uniform -> iid U(0,1); zipf -> log p_rank(e) + Gumbel(0,1) with
    p_rank proportional to rank^-1.2 over a seeded permutation of the experts,
    so a row's top-k is a draw of k experts without replacement weighted by
    p.  None for workloads that run the router GEMV."""
    E = wl.n_experts
    if wl.router == "gemv":
        return None
    g = _gen(device, wl.name, layer, "logits", rows)
    if wl.router == "uniform":
        return torch.rand((rows, E), generator=g, device=device, dtype=torch.float32)
    gp = _gen("cpu", wl.name, layer, "zipf_perm")
    rank = torch.randperm(E, generator=gp).to(device)          # rank of each expert, 0-based
    logp = -1.2 * torch.log((rank + 1).to(torch.float64))
    logp = logp - torch.logsumexp(logp, 0)
    u = torch.rand((rows, E), generator=g, device=device, dtype=torch.float64)
    u = u.clamp(min=1e-300)
    gumbel = -torch.log(-torch.log(u))
    return (logp[None, :] + gumbel).to(torch.float32)


def effective_weight_bytes(wl: Workload, distinct_routed: int, router_gemv: bool) -> int:
    """Bytes the layer must move once per step: each distinct touched routed
    expert's codes and scales, the shared expert, the shared-gate vector and
    the router matrix when the router GEMV runs."""
    H, I, Is, E = wl.hidden, wl.inter, wl.shared_inter, wl.n_experts

    def expert_bytes(inter):
        n = 2 * inter * H + H * inter          # weights of gate|up and down
        if wl.fmt in (FMT_FP8_B128, FMT_FP8_B128_BF16S):
            sb = 4 if wl.fmt == FMT_FP8_B128 else 2
            return n + sb * ((2 * inter // 128) * (H // 128) + (H // 128) * (inter // 128))
        if wl.fmt == FMT_INT8_ROW:
            return n + 4 * (2 * inter + H)
        if wl.fmt == FMT_INT4_ROW:
            return n // 2 + 4 * (2 * inter + H)
        if wl.fmt == FMT_INT4_G64:
            return n // 2 + 4 * (n // 64)
        return n // 2 + n // 16 + 8

    b = distinct_routed * expert_bytes(I)
    if Is > 0:
        b += expert_bytes(Is) + 2 * H
    if router_gemv:
        b += 2 * E * H
    return b


def expected_distinct(wl: Workload, rows: int) -> float:
    """Expected distinct experts under uniform independent routing."""
    E, k = wl.n_experts, wl.top_k
    return E * (1.0 - (1.0 - k / E) ** rows)


def describe() -> str:
    return "\n".join(f"{w.name}: {w}" for w in WORKLOADS.values())


if __name__ == "__main__":
    print(describe())
    print(effective_weight_bytes(WORKLOADS["a3b"], 8, True))
    print(math.ceil(expected_distinct(WORKLOADS["a3b_multi"], 64)))
