"""GPU-test plumbing: run layers through the C ABI and compare with the
oracle on the same seeded inputs.

Acceptance (the layer's stated bar): expert ids, their order and the grouping
arrays bit-exact; routing weights and the shared gate within 1e-5; the bf16
MoE output y within max|err| <= 2e-2 * rms(y_oracle) and
sum|err| / sum|y_oracle| <= 5e-3 against the oracle's unrounded f32 y; the
residual-blended output within the same absolute bound plus one bf16 ulp of
the blended value (the residual's magnitude dominates its rounding).
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import moe_synth as syn
from helpers import bits, host, oracle_layer, router_only_layer, tie_free_x

Y_MAX_REL_RMS = 2e-2
Y_MEAN_REL = 5e-3
W_TOL = 1e-5


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def oracle_threads():
    n = min(16, len(os.sched_getaffinity(0)))
    return max(1, n)


def make_tie_free(orc, res, rows_from=None):
    """Redraw activation rows of a Resident workload whose oracle router
    logits have a top-(k+1) gap below the margin (router-GEMV workloads)."""
    wl = res.wl
    if wl.router != "gemv":
        return
    for n, l in enumerate(res.layer_ids):
        x, att = tie_free_x(orc, wl, res.W[n], l, res.rows, device=res.device)
        res.x[n] = x


def logits_for(orc, wl, W, x, logits_in):
    if logits_in is not None:
        return host(logits_in).astype(np.float32)
    return orc.router_logits(router_only_layer(orc, wl, W), bits(x))


def compare_y(y_gpu: torch.Tensor, y_ref: np.ndarray, what=""):
    g = y_gpu.float().cpu().numpy().astype(np.float64)
    o = y_ref.astype(np.float64)
    rms = float(np.sqrt(np.mean(o * o)))
    err = np.abs(g - o)
    maxerr = float(err.max()) if err.size else 0.0
    mre = float(err.sum() / max(np.abs(o).sum(), 1e-300))
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    assert maxerr <= Y_MAX_REL_RMS * rms, f"{what}: max|err| {maxerr:.3e} > {Y_MAX_REL_RMS} * rms {rms:.3e}"
    assert mre <= Y_MEAN_REL, f"{what}: mean rel err {mre:.3e} > {Y_MEAN_REL}"
    return maxerr / max(rms, 1e-300), mre


def compare_out(out_gpu: torch.Tensor, out_ref_bits: np.ndarray, y_ref: np.ndarray, what=""):
    g = out_gpu.float().cpu().numpy().astype(np.float64)
    o = torch.from_numpy(out_ref_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    rms = float(np.sqrt(np.mean(y_ref.astype(np.float64) ** 2)))
    ulp = np.abs(o) * 2.0 ** -7 + 1e-30
    bad = np.abs(g - o) > Y_MAX_REL_RMS * rms + ulp
    assert not bad.any(), f"{what}: {int(bad.sum())} blended outputs off"


def check_layer(orc, wl, W, x, logits_in, residual0, y, residual, routing, rows=None,
                check_grouping=True, what=""):
    """Full check of one layer's GPU results against the oracle.  `rows`
    restricts the FFN comparison to a subset of rows (routing and grouping are
    always checked on every row)."""
    R = x.shape[0]
    k = wl.top_k
    logits = logits_for(orc, wl, W, x, logits_in)
    ids_o, w_o = orc.topk_softmax(logits, k)
    ids_g = routing.topk_ids.cpu().numpy()
    assert np.array_equal(ids_g, ids_o), f"{what}: ids differ in rows {np.where((ids_g != ids_o).any(1))[0][:8]}"
    w_g = routing.topk_w.cpu().numpy()
    assert np.max(np.abs(w_g - w_o)) <= W_TOL, f"{what}: routing weights off by {np.max(np.abs(w_g - w_o)):.2e}"
    if routing.logits is not None and logits_in is None:
        lg = routing.logits.cpu().numpy()
        scale = np.abs(logits).max() + 1
        assert np.max(np.abs(lg - logits)) <= 1e-5 * scale, f"{what}: logits off"
    if R >= 2 and check_grouping and routing.expert_count is not None:
        c_o, off_o, perm_o = orc.group(ids_o, wl.n_experts)
        assert np.array_equal(routing.expert_count.cpu().numpy(), c_o), f"{what}: counts"
        assert np.array_equal(routing.expert_offset.cpu().numpy(), off_o), f"{what}: offsets"
        assert np.array_equal(routing.perm.cpu().numpy(), perm_o), f"{what}: perm"
    sel = np.arange(R) if rows is None else np.asarray(rows)
    touched = np.unique(ids_o[sel])
    L = oracle_layer(orc, wl, W, experts=touched)
    xs = bits(x)[sel]
    ref = orc.layer_forward(L, xs, logits_in=logits[sel], residual=bits(residual0)[sel])
    s_g = routing.shared_gate.cpu().numpy()[sel]
    assert np.max(np.abs(s_g - ref["s"])) <= W_TOL, f"{what}: shared gate off"
    stats = compare_y(y[sel], ref["y"], what)
    compare_out(residual[sel], ref["out"], ref["y"], what)
    return stats
