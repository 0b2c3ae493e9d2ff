"""GPU parity of the top-k tie rule at every site that selects experts.

The order is value descending with the lower expert index first among equal
values (GB10 blueprint, "Kernels": moe_topk_softmax, whose node output is
f32 weights and i32 ids; the tie rule itself is a reading, since the pages do
not state one).  Every other GPU parity test draws tie-free logits, so the
branch that resolves equal values is exercised here: rows of given logits
with exact duplicates (every logit equal, equal values straddling the k-th
place, +0 and -0 mixed, equal values on lanes of different 16-lane rows and
in one lane's several registers), and router-GEMV logits made exactly equal
by giving several experts the same router row.

Each case names the kernel that selects and asserts, from the ctx's launch
records, that this kernel ran:
  R = 1, single launch     every waiting workgroup of the one-launch layer
  R = 1, three launches    the last router workgroup of the lead kernel
  R <= 8 (4 above 256 experts), few rows
                           the gate/up workgroups of the few-rows path
  R up to E/2k, few rows   the top-k launch
  R > E/2k, grouped        the top-k + grouping launch (grouping checked too)
  moe_route                the top-k launch (R = 1) and top-k + grouping
Ids, their order and the grouping must equal the oracle's bit for bit; the
weights within 1e-5 and the layer output within the layer's tolerance.
"""
import numpy as np
import pytest
import torch

import moe_synth as syn
from gpu_helpers import W_TOL, check_layer, need_gpu, oracle_threads
from helpers import bits, router_only_layer, tie_free_x, tie_rows

pytestmark = pytest.mark.gpu

KIND = {"router": 0, "topk": 1, "group": 2, "gate_up": 3, "down": 4, "blend": 5, "layer": 8}


@pytest.fixture(scope="module")
def moe():
    need_gpu()
    import routed_fp8_expert_amd as m
    return m


@pytest.fixture(autouse=True)
def _threads(orc):
    orc.set_threads(oracle_threads())


def _ctx(moe, one_row_path=0, few_rows=-1):
    c = moe.Ctx(0)
    moe.moe_ctx_set_one_row_path(c, one_row_path)
    moe.moe_ctx_set_few_rows(c, few_rows)
    moe.moe_ctx_set_timing(c, True)
    return c


def _ran(moe, c, kind):
    _, n = moe.moe_ctx_kernel_stats(c, KIND[kind])
    return n


def _layer_case(moe, orc, wl, W, x, li, c, expect, what, grouping=True):
    from routed_fp8_expert_amd.workload import layer_weights
    R = x.shape[0]
    lw = layer_weights(wl, W)
    rt = moe.Routing(R, wl.n_experts, wl.top_k, "cuda", logits=True, grouping=grouping)
    ws = moe.workspace(lw, R, "cuda")
    y = torch.full((R, wl.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    res0 = syn.make_residual(wl, 0, R, "cuda")
    res = res0.clone()
    print(f"ties: {what}", flush=True)
    moe.moe_layer_forward(c, lw, x, y, res, ws, logits_in=li, routing=rt)
    torch.cuda.synchronize()
    assert moe.moe_ctx_status(c) == 0
    assert moe.moe_ctx_device_errors(c) == 0, f"{what}: device error word set"
    for kind, want in expect.items():
        got = _ran(moe, c, kind) > 0
        assert got == want, f"{what}: kernel '{kind}' {'did not run' if want else 'ran'}"
    check_layer(orc, wl, W, x, li, res0, y, res, rt, what=what)
    return rt


# R = 1: the single launch, and the three-launch path
ONE_ROW = [("tiny", 0, {"layer": True}), ("a3b", 0, {"layer": True}),
           ("tiny", 1, {"layer": False, "router": True}), ("a3b", 1, {"layer": False, "router": True}),
           ("a17b", 0, {"layer": False, "router": True})]


@pytest.mark.parametrize("name,path,expect", ONE_ROW)
@pytest.mark.parametrize("pattern", range(6))
def test_one_row_given_logits(moe, orc, name, path, expect, pattern):
    wl = syn.WORKLOADS[name]
    W = syn.make_layer_weights(wl, 0, "cuda")
    x = syn.make_x(wl, 0, 1, 0, "cuda")
    li = torch.from_numpy(tie_rows(wl.n_experts, wl.top_k, 6, 11)[pattern:pattern + 1].copy()).cuda()
    c = _ctx(moe, one_row_path=path)
    _layer_case(moe, orc, wl, W, x, li, c, expect, f"{name} path {path} pattern {pattern}")
    c.close()


def _dup_router_rows(orc, wl, W, x, where):
    """Give some experts the router row (and bias) of another, so that the
    router GEMV's logits tie exactly: 'top' copies the largest expert's row
    into two experts outside the top k+1 (one below its index if any, one
    above); 'straddle' copies the k-th largest's row likewise, making a group
    of three equal values at ranks k-1, k, k+1."""
    W = dict(W)
    rw = W["router_w"].clone()
    bias = W["router_bias"].clone() if W.get("router_bias") is not None else None
    lg = orc.router_logits(router_only_layer(orc, wl, W), bits(x))[0]
    order = np.argsort(-lg.astype(np.float64), kind="stable")
    k = wl.top_k
    src = int(order[0] if where == "top" else order[k - 1])
    outside = [int(e) for e in order[k + 1:]]
    lower = [e for e in outside if e < src]
    higher = [e for e in outside if e > src]
    dst = ([lower[len(lower) // 2]] if lower else []) + ([higher[len(higher) // 2]] if higher else [])
    while len(dst) < 2:
        dst.append([e for e in outside if e not in dst][0])
    for d in dst:
        rw[d] = rw[src]
        if bias is not None:
            bias[d] = bias[src]
    W["router_w"] = rw
    if bias is not None:
        W["router_bias"] = bias
    lg2 = orc.router_logits(router_only_layer(orc, wl, W), bits(x))[0]
    assert all(lg2[d] == lg2[src] for d in dst)
    return W, src, dst


@pytest.mark.parametrize("name,path,expect", ONE_ROW[:4])
@pytest.mark.parametrize("where", ["top", "straddle"])
def test_one_row_router_ties(moe, orc, name, path, expect, where):
    wl = syn.WORKLOADS[name]
    W0 = syn.make_layer_weights(wl, 0, "cuda")
    x, _ = tie_free_x(orc, wl, W0, 0, 1, device="cuda")
    W, src, dst = _dup_router_rows(orc, wl, W0, x, where)
    c = _ctx(moe, one_row_path=path)
    rt = _layer_case(moe, orc, wl, W, x, None, c, expect,
                     f"{name} path {path} router rows of {src} copied to {dst} ({where})")
    ids = rt.topk_ids.cpu().numpy()[0].tolist()
    if where == "top":
        n = min(3, wl.top_k)
        assert ids[:n] == sorted([src] + dst)[:n], ids
    c.close()


# R >= 2 (E / 2k = 16 here): the few-rows fused top-k (<= 8 rows), the
# top-k launch (9..16), the top-k + grouping launch (>= 17)
MULTI = [(3, {"topk": False, "gate_up": True}), (4, {"topk": False}), (6, {"topk": False}),
         (8, {"topk": False, "gate_up": True}), (12, {"topk": True}), (16, {"topk": True}),
         (24, {"topk": True}), (64, {"topk": True})]


@pytest.mark.parametrize("rows,expect", MULTI)
def test_multi_row_given_logits(moe, orc, rows, expect):
    wl = syn.WORKLOADS["a3b_multi"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    x = syn.make_x(wl, 0, rows, 0, "cuda")
    li = torch.from_numpy(tie_rows(wl.n_experts, wl.top_k, rows, 100 + rows)).cuda()
    c = _ctx(moe)
    _layer_case(moe, orc, wl, W, x, li, c, expect, f"a3b_multi {rows} rows")
    c.close()


@pytest.mark.parametrize("rows,expect", [(4, {"topk": False, "gate_up": True}), (8, {"topk": True}),
                                         (16, {"topk": True}), (32, {"topk": True})])
def test_multi_row_given_logits_nvfp4(moe, orc, rows, expect):
    """512 experts (eight logits a lane), top-10 (E / 2k = 25: few rows with
    the fused top-k up to 4 rows, with the top-k launch at 8 and 16, grouped
    at 32)."""
    wl = syn.WORKLOADS["a17b"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    x = syn.make_x(wl, 0, rows, 0, "cuda")
    li = torch.from_numpy(tie_rows(wl.n_experts, wl.top_k, rows, 200 + rows)).cuda()
    c = _ctx(moe)
    _layer_case(moe, orc, wl, W, x, li, c, expect, f"a17b {rows} rows")
    c.close()


@pytest.mark.parametrize("name,rows", [("a3b", 1), ("a3b", 6), ("a3b", 16), ("a17b", 1), ("a17b", 12),
                                       ("tiny", 1), ("tiny", 7)])
def test_route_given_logits(moe, orc, name, rows):
    """moe_route alone: ids, weights and (rows >= 2) the grouping."""
    from routed_fp8_expert_amd.workload import layer_weights
    wl = syn.WORKLOADS[name]
    W = syn.make_layer_weights(wl, 0, "cuda")
    lw = layer_weights(wl, W)
    x = syn.make_x(wl, 0, rows, 0, "cuda")
    li_np = tie_rows(wl.n_experts, wl.top_k, rows, 300 + rows)
    li = torch.from_numpy(li_np).cuda()
    rt = moe.Routing(rows, wl.n_experts, wl.top_k, "cuda")
    ws = moe.workspace(lw, rows, "cuda")
    c = _ctx(moe)
    print(f"ties: moe_route {name} {rows} rows", flush=True)
    moe.moe_route(c, lw, x, rt, ws, logits_in=li)
    torch.cuda.synchronize()
    assert moe.moe_ctx_status(c) == 0 and moe.moe_ctx_device_errors(c) == 0
    assert _ran(moe, c, "topk") == 1
    ids_o, w_o = orc.topk_softmax(li_np, wl.top_k)
    assert np.array_equal(rt.topk_ids.cpu().numpy(), ids_o)
    assert np.max(np.abs(rt.topk_w.cpu().numpy() - w_o)) <= W_TOL
    if rows >= 2:
        cnt, off, perm = orc.group(ids_o, wl.n_experts)
        assert np.array_equal(rt.expert_count.cpu().numpy(), cnt)
        assert np.array_equal(rt.expert_offset.cpu().numpy(), off)
        assert np.array_equal(rt.perm.cpu().numpy(), perm)
    c.close()
