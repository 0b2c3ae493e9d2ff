"""Shared test plumbing: the tie-margin redraw of activation rows and the
tie inputs (the oracle-layer construction lives in oracle/layers.py).  Holds none of the
layer's arithmetic beyond calling the oracle."""
from __future__ import annotations

import numpy as np
import torch

import moe_synth as syn
from oracle.layers import bits, host, min_top_gap, oracle_layer, router_only_layer  # noqa: F401


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
