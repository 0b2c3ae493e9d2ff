"""GPU tests of the few-rows path (steps of 2 to E / 2k rows at the default arm
choice: no grouping, one GEMV per row and slot with the one-row kernels, down
fused with the blend per row).  Its rows have one-row bits, so it must give
exactly the grouped path's bits (which also equal one-row calls); parity
against the oracle comes from the multi-row parity tests, which run on it.
The grouping arrays are written when given and left alone when not."""
import numpy as np
import pytest
import torch

import moe_synth as syn
from gpu_helpers import check_layer, need_gpu, oracle_threads
from helpers import bits, tie_free_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    need_gpu()
    import routed_fp8_expert_amd as m
    return m


def _forward(moe, few, wl, W, x, li, res0, grouping=True, norm=None):
    from routed_fp8_expert_amd.workload import layer_weights
    R = x.shape[0]
    c = moe.Ctx(0)
    moe.moe_ctx_set_few_rows(c, few)
    lw = layer_weights(wl, W)
    rt = moe.Routing(R, wl.n_experts, wl.top_k, "cuda", logits=True, grouping=grouping)
    if grouping:
        rt.expert_count.fill_(-7)
        rt.perm.fill_(-7)
    ws = moe.workspace(lw, R, "cuda")
    y = torch.full((R, wl.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    res = res0.clone()
    moe.moe_layer_forward(c, lw, x, y, res, ws, logits_in=li, routing=rt)
    torch.cuda.synchronize()
    assert moe.moe_ctx_status(c) == 0 and moe.moe_ctx_device_errors(c) == 0
    c.close()
    return y, res, rt


CASES = [("a3b_multi", r) for r in (2, 3, 4, 8)] + [("tiny", r) for r in (2, 5)] + \
        [("a17b", 8), ("a3b_i4g64", 4), ("a3b_f8bs", 3)]


@pytest.mark.parametrize("name,rows", CASES)
def test_few_rows_path_equals_grouped_path(moe, orc, name, rows):
    wl = syn.WORKLOADS[name]
    W = syn.make_layer_weights(wl, 0, "cuda")
    if wl.router == "gemv":
        x, _ = tie_free_x(orc, wl, W, 0, rows, device="cuda")
    else:
        x = syn.make_x(wl, 0, rows, 0, "cuda")
    li = syn.make_logits_in(wl, 0, rows, "cuda")
    res0 = syn.make_residual(wl, 0, rows, "cuda")
    print(f"few rows: {name} rows {rows}", flush=True)
    yf, rf, tf = _forward(moe, 8, wl, W, x, li, res0)
    yg, rg, tg = _forward(moe, 0, wl, W, x, li, res0)
    assert np.array_equal(bits(yf), bits(yg)), f"{name}: y differs between the paths"
    assert np.array_equal(bits(rf), bits(rg)), f"{name}: residual differs between the paths"
    for f in ("topk_ids", "topk_w", "shared_gate", "expert_count", "expert_offset", "perm"):
        assert torch.equal(getattr(tf, f), getattr(tg, f)), f
    orc.set_threads(oracle_threads())
    check_layer(orc, wl, W, x, li, res0, yf, rf, tf, what=f"{name} R{rows} few")


@pytest.mark.parametrize("logits", [True, False])
def test_few_rows_ungated_shared_expert(moe, orc, logits):
    """No shared-gate vector: s = 1 on both paths (given logits or the router)."""
    wl = syn.WORKLOADS["tiny"]
    W = dict(syn.make_layer_weights(wl, 0, "cuda"))
    W["shared_gate_w"] = None
    x, _ = tie_free_x(orc, wl, W, 0, 4, device="cuda")
    li = syn.make_logits_in(syn.WORKLOADS["a3b_multi"], 0, 4, "cuda")[:, :wl.n_experts].contiguous() if logits else None
    res0 = syn.make_residual(wl, 0, 4, "cuda")
    yf, rf, tf = _forward(moe, 8, wl, W, x, li, res0)
    yg, rg, tg = _forward(moe, 0, wl, W, x, li, res0)
    assert np.array_equal(bits(yf), bits(yg))
    assert bool(torch.all(tf.shared_gate == 1.0)) and torch.equal(tf.topk_ids, tg.topk_ids)
    orc.set_threads(oracle_threads())
    check_layer(orc, wl, W, x, li, res0, yf, rf, tf, what=f"tiny ungated few logits={logits}")


def test_grouping_arrays_optional(moe, orc):
    wl = syn.WORKLOADS["a3b_multi"]
    W = syn.make_layer_weights(wl, 1, "cuda")
    x = syn.make_x(wl, 1, 4, 0, "cuda")
    li = syn.make_logits_in(wl, 1, 4, "cuda")
    res0 = syn.make_residual(wl, 1, 4, "cuda")
    y0, _, t0 = _forward(moe, 8, wl, W, x, li, res0, grouping=True)
    y1, _, t1 = _forward(moe, 8, wl, W, x, li, res0, grouping=False)      # few-rows path, no grouping
    y2, _, t2 = _forward(moe, 0, wl, W, x, li, res0, grouping=False)      # grouped path, workspace grouping
    assert t1.expert_count is None
    assert np.array_equal(bits(y0), bits(y1)) and np.array_equal(bits(y0), bits(y2))
    assert torch.equal(t0.topk_ids, t1.topk_ids) and torch.equal(t0.topk_ids, t2.topk_ids)
    assert int(t0.expert_count.sum()) == 4 * wl.top_k


def test_expert_ffn_on_both_paths(moe, orc):
    from routed_fp8_expert_amd.workload import layer_weights
    wl = syn.WORKLOADS["a3b_multi"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    x = syn.make_x(wl, 0, 6, 0, "cuda")
    li = syn.make_logits_in(wl, 0, 6, "cuda")
    lw = layer_weights(wl, W)
    out = []
    for few in (8, 0):
        c = moe.Ctx(0)
        moe.moe_ctx_set_few_rows(c, few)
        rt = moe.Routing(6, wl.n_experts, wl.top_k, "cuda")
        ws = moe.workspace(lw, 6, "cuda")
        moe.moe_route(c, lw, x, rt, ws, logits_in=li)
        y = torch.full((6, wl.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_expert_ffn(c, lw, x, rt, y, None, ws)
        torch.cuda.synchronize()
        assert moe.moe_ctx_status(c) == 0
        c.close()
        out.append(bits(y))
    assert np.array_equal(out[0], out[1])


def test_few_rows_knob_rejects_below_auto(moe):
    c = moe.Ctx(0)
    with pytest.raises(moe.MoeError):
        moe.moe_ctx_set_few_rows(c, -2)
    moe.moe_ctx_set_few_rows(c, 0)
    moe.moe_ctx_set_few_rows(c, -1)
    c.close()


def test_mixed_grouping_arrays_rejected(moe):
    import ctypes as C
    from routed_fp8_expert_amd.workload import layer_weights
    from routed_fp8_expert_amd.binding import RoutingC, lib, _p, _stream
    wl = syn.WORKLOADS["tiny"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    lw = layer_weights(wl, W)
    x = syn.make_x(wl, 0, 3, 0, "cuda")
    rt = moe.Routing(3, wl.n_experts, wl.top_k, "cuda")
    ws = moe.workspace(lw, 3, "cuda")
    y = torch.full((3, wl.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    c = moe.Ctx(0)
    bad = RoutingC.from_buffer_copy(rt.c)
    bad.expert_offset = None
    rc = lib().moe_layer_forward(c.handle, lw.ref, _p(x), 3, wl.hidden, None, C.byref(bad), _p(y), None,
                                 wl.hidden, _p(ws), ws.numel(), _stream(None))
    torch.cuda.synchronize()
    assert rc == moe.binding.MOE_ERR_INVALID_ARG and bool(torch.all(y == 7.0))
    c.close()
