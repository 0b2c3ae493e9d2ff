"""Shared test plumbing: turning generated torch tensors into the oracle's
numpy layer, and the tie-margin redraw of activation rows.  Holds none of the
layer's arithmetic beyond calling the oracle."""
from __future__ import annotations

import numpy as np
import torch

import moe_synth as syn


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> its uint16 bit patterns (numpy, host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t):
    """Tensor -> numpy on the host (bf16 as its uint16 bit patterns)."""
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return bits(t)
    return t.detach().cpu().contiguous().numpy()


def oracle_layer(orc, wl: syn.Workload, W: dict, experts=None):
    """Build an oracle Layer from make_layer_weights() output.  `experts`
    limits the routed experts copied to the host (None = all)."""
    E = W["gu_q"].shape[0] if experts is None else wl.n_experts
    sel = range(E) if experts is None else sorted(set(int(e) for e in experts))
    nv = wl.fmt == syn.FMT_NVFP4

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


def router_only_layer(orc, wl: syn.Workload, W: dict):
    return orc.Layer(wl.hidden, wl.n_experts, wl.top_k, wl.inter, 0, wl.fmt,
                     router_w=bits(W["router_w"]), router_bias=host(W["router_bias"]))


def min_top_gap(logits: np.ndarray, k: int) -> float:
    """Smallest gap between adjacent values among the k+1 largest logits of
    each row (the margin that keeps a GPU top-k equal to the oracle's)."""
    s = -np.sort(-logits.astype(np.float64), axis=1)[:, : k + 1]
    return float(np.min(s[:, :-1] - s[:, 1:])) if s.shape[1] > 1 else np.inf


def tie_free_x(orc, wl: syn.Workload, W: dict, layer: int, rows: int, device="cpu",
               margin: float = 1e-3, max_attempts: int = 64):
    """Draw activation rows whose oracle router logits keep every adjacent gap
    among the top k+1 at least `margin`; redraw with the next attempt number
    otherwise.  Returns (x, attempt)."""
    rl = router_only_layer(orc, wl, W)
    for attempt in range(max_attempts):
        x = syn.make_x(wl, layer, rows, attempt, device)
        if min_top_gap(orc.router_logits(rl, bits(x)), wl.top_k) >= margin:
            return x, attempt
    raise RuntimeError("no tie-free activation draw found")


def tie_rows(E: int, k: int, R: int, seed: int) -> np.ndarray:
    """R rows of E logits, row r following pattern r % 6:
      0  every logit equal
      1  distinct values, then the values ranked k-2 .. k+2 made equal (a
         tie group straddling the k-th place)
      2  all negative but 2k experts at +0 or -0 (alternating signs), spread
         over lanes, 16-lane rows and registers
      3  the top value shared by experts b, b+16, b+32, b+48 (four 16-lane
         rows) and b+64, b+128, ... (one lane's registers), k+2 in all
      4  the three largest equal, the rest distinct
      5  distinct (control)
    Distinct values are at least 1e-3 apart, in [-2, 2)."""
    rng = np.random.default_rng(seed)
    out = np.empty((R, E), np.float32)
    for r in range(R):
        base = (rng.permutation(E).astype(np.float64) * (3.0 / E) - 1.5).astype(np.float32)
        p = r % 6
        if p == 0:
            row = np.full(E, 0.25, np.float32)
        elif p == 1:
            row = base.copy()
            order = np.argsort(-row, kind="stable")
            grp = order[max(0, k - 2): min(E, k + 3)]
            row[grp] = row[order[min(E - 1, k + 2)]]
        elif p == 2:
            row = (base - 3.5) / 2.0
            row = np.minimum(row, -1.0).astype(np.float32)
            n = min(E, 2 * k)
            zs = rng.choice(E, size=n, replace=False)
            for i, e in enumerate(zs):
                row[e] = np.float32(-0.0) if i % 2 else np.float32(0.0)
        elif p == 3:
            row = base.copy() - 2.0
            b = int(rng.integers(0, min(16, E)))
            cand = [b + 16 * j for j in range(4)] + [b + 64 * j for j in range(1, E // 64 + 1)]
            cand += [b + 1 + 16 * j for j in range(4)]
            cand = [e for e in dict.fromkeys(cand) if e < E][: k + 2]
            row[cand] = 1.75
        elif p == 4:
            row = base.copy()
            order = np.argsort(-row, kind="stable")
            row[order[:3]] = row[order[0]]
        else:
            row = base.copy()
        out[r] = row
    return out
