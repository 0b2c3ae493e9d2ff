"""Device-resident synthetic workloads: L independent layers of weights,
activations, residuals, outputs and one shared workspace, all in HBM, run back
to back through moe_layer_forward.  Plumbing for the benchmark and the GPU
tests; the inputs come from moe_synth, the arithmetic from the HIP library."""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

import moe_synth as syn

from . import binding as B


def layer_weights(wl: syn.Workload, W: dict) -> B.LayerWeights:
    return B.LayerWeights(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, wl.fmt, W)


class Resident:
    """`layers` layers of workload `wl` at `rows` rows, resident on `device`.

    x_attempts: per-layer attempt numbers for the activation draw (the tests'
    tie-margin redraw); default 0 everywhere."""

    def __init__(self, wl: syn.Workload, rows: int, layers: Optional[int] = None, device="cuda",
                 x_attempts: Optional[Sequence[int]] = None, layer_ids: Optional[Sequence[int]] = None,
                 keep_y: bool = True, with_routing: bool = True, norm: bool = False, progress=None):
        self.wl, self.rows, self.device = wl, rows, torch.device(device)
        ids = list(layer_ids) if layer_ids is not None else list(range(layers or wl.layers))
        self.layer_ids = ids
        self.W: List[dict] = []
        self.lw: List[B.LayerWeights] = []
        self.x, self.logits_in, self.residual0, self.y, self.routing = [], [], [], [], []
        for n, l in enumerate(ids):
            if progress is not None and n % 8 == 0:
                progress(f"building layer {n + 1} of {len(ids)}")
            W = syn.make_layer_weights(wl, l, self.device)
            self.W.append(W)
            self.lw.append(layer_weights(wl, W))
            att = 0 if x_attempts is None else int(x_attempts[n])
            self.x.append(syn.make_x(wl, l, rows, att, self.device))
            self.logits_in.append(syn.make_logits_in(wl, l, rows, self.device))
            self.residual0.append(syn.make_residual(wl, l, rows, self.device))
            self.y.append(torch.empty((rows, wl.hidden), dtype=torch.bfloat16, device=self.device)
                          if keep_y else None)
            self.routing.append(B.Routing(rows, wl.n_experts, wl.top_k, self.device, logits=True, grouping=False)
                                if with_routing else None)
        self.residual = [r.clone() for r in self.residual0]
        self.ws = B.workspace(self.lw[0], rows, self.device)
        # optional RMSNorm epilogue: a weight near 1 per layer and the output rows
        self.norm = norm
        self.norm_w, self.norm_out = [], []
        if norm:
            for l in ids:
                g = torch.Generator(device=self.device)
                g.manual_seed(syn.subseed("norm-weight", wl.name, l))
                w = 1.0 + 0.1 * torch.randn(wl.hidden, generator=g, device=self.device)
                self.norm_w.append(w.to(torch.bfloat16))
                self.norm_out.append(torch.empty((rows, wl.hidden), dtype=torch.bfloat16, device=self.device))

    def reset_residual(self):
        for r, r0 in zip(self.residual, self.residual0):
            r.copy_(r0)

    def run(self, ctx: B.Ctx, stream=None, write_y: bool = True):
        for n in range(len(self.lw)):
            if self.norm:
                B.moe_layer_forward_norm(ctx, self.lw[n], self.x[n], self.y[n] if write_y else None,
                                         self.residual[n], self.ws, self.norm_w[n], 1e-6, self.norm_out[n],
                                         logits_in=self.logits_in[n], routing=self.routing[n], stream=stream)
            else:
                B.moe_layer_forward(ctx, self.lw[n], self.x[n], self.y[n] if write_y else None,
                                    self.residual[n], self.ws, logits_in=self.logits_in[n],
                                    routing=self.routing[n], stream=stream)

    def weight_bytes_resident(self) -> int:
        total = 0
        for W in self.W:
            for v in W.values():
                if v is not None:
                    total += v.numel() * v.element_size()
        return total
