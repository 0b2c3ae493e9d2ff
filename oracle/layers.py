"""Oracle layers from generated weights (test infrastructure, like the rest of
this package): turns the torch tensors that moe_synth makes into the numpy
arrays of an oracle Layer.  Plumbing only -- the arithmetic is the C
oracle's."""
from __future__ import annotations

import numpy as np


def bits(t) -> np.ndarray:
    """bf16 tensor -> its uint16 bit patterns (numpy, host)."""
    import torch
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t):
    """Tensor -> numpy on the host (bf16 as its uint16 bit patterns)."""
    import torch
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return bits(t)
    return t.detach().cpu().contiguous().numpy()


def oracle_layer(orc, wl, W: dict, experts=None):
    """An oracle Layer from make_layer_weights() output for workload `wl`.
    `experts` limits the routed experts copied to the host (None = all)."""
    E = W["gu_q"].shape[0] if experts is None else wl.n_experts
    sel = range(E) if experts is None else sorted(set(int(e) for e in experts))
    nv = wl.fmt == orc.FMT_NVFP4

    def ex(prefix, e, gu_q, gu_s, dn_q, dn_s):
        kw = {}
        if nv:
            kw = {"gu_g": float(W[prefix + "gu_g"][e]), "dn_g": float(W[prefix + "dn_g"][e])}
        return orc.Expert(host(gu_q[e]), host(gu_s[e]), host(dn_q[e]), host(dn_s[e]), **kw)

    experts_np = {e: ex("", e, W["gu_q"], W["gu_s"], W["dn_q"], W["dn_s"]) for e in sel}
    shared = None
    if wl.shared_inter > 0:
        shared = ex("sh_", 0, W["sh_gu_q"], W["sh_gu_s"], W["sh_dn_q"], W["sh_dn_s"])
    return orc.Layer(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, wl.fmt,
                     router_w=bits(W["router_w"]), router_bias=host(W["router_bias"]),
                     shared_gate_w=bits(W["shared_gate_w"]) if W.get("shared_gate_w") is not None
                     else None,
                     experts=experts_np, shared=shared)


def router_only_layer(orc, wl, W: dict):
    """A Layer holding only the router (for router logits)."""
    return orc.Layer(wl.hidden, wl.n_experts, wl.top_k, wl.inter, 0, wl.fmt,
                     router_w=bits(W["router_w"]), router_bias=host(W["router_bias"]))


def min_top_gap(logits: np.ndarray, k: int) -> float:
    """Smallest gap between adjacent values among the k+1 largest logits of
    each row (the margin that keeps a GPU top-k equal to the oracle's)."""
    s = -np.sort(-logits.astype(np.float64), axis=1)[:, : k + 1]
    return float(np.min(s[:, :-1] - s[:, 1:])) if s.shape[1] > 1 else np.inf
