"""moe_layer_forward_static (the entry point that allocates nothing: its
workspace is the library's static device scratch) against
moe_layer_forward with a caller's workspace, through the C ABI, on calls in a
row that shrink: 32 rows (grouped, matrix-core arm), 5 rows (few-rows path),
1 row (the one-launch layer), each compared bit for bit (ids, weights, shared
gate, grouping, y and the blended residual), which is within the layer's
tolerance a fortiori.  Also: a call whose workspace exceeds the scratch is
refused with nothing enqueued."""
import ctypes as C

import numpy as np
import pytest
import torch

import moe_synth as syn
from gpu_helpers import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    need_gpu()
    import routed_fp8_expert_amd as m
    return m


def _p(t):
    return None if t is None else t.data_ptr()


def _call(moe, ctx, lw, x, li, rt, y, res, ws=None):
    """One raw C-ABI call: moe_layer_forward_static when ws is None, else
    moe_layer_forward with the workspace."""
    L = moe.binding.lib()
    st = torch.cuda.current_stream().cuda_stream
    R = x.shape[0]
    if ws is None:
        rc = L.moe_layer_forward_static(ctx.handle, lw.ref, _p(x), R, x.stride(0), _p(li), rt.ref, _p(y),
                                        _p(res), y.stride(0), st)
    else:
        rc = L.moe_layer_forward(ctx.handle, lw.ref, _p(x), R, x.stride(0), _p(li), rt.ref, _p(y), _p(res),
                                 y.stride(0), _p(ws), ws.numel(), st)
    return rc


def _case(moe, ctx, wl, W, rows, layer):
    from routed_fp8_expert_amd.workload import layer_weights
    lw = layer_weights(wl, W)
    x = syn.make_x(wl, layer, rows, 0, "cuda")
    li = syn.make_logits_in(wl, layer, rows, "cuda")
    res0 = syn.make_residual(wl, layer, rows, "cuda")
    out = []
    for use_ws in (True, False):
        rt = moe.Routing(rows, wl.n_experts, wl.top_k, "cuda", logits=False, grouping=rows >= 2)
        y = torch.full((rows, wl.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
        res = res0.clone()
        ws = moe.workspace(lw, rows, "cuda") if use_ws else None
        rc = _call(moe, ctx, lw, x, li, rt, y, res, ws)
        assert rc == 0, moe.strerror(rc)
        torch.cuda.synchronize()
        out.append((rt, y, res))
    return out


@pytest.mark.parametrize("seq", [[("a3b_multi", 32), ("a3b_multi", 5), ("a3b", 1)],
                                 [("a3b_multi", 64), ("tiny", 1)]])
def test_static_scratch_equals_workspace_entry_point(moe, seq):
    ctx = moe.Ctx(0)
    for name, rows in seq:
        wl = syn.WORKLOADS[name]
        W = syn.make_layer_weights(wl, 0, "cuda")
        print(f"static scratch: {name} {rows} rows", flush=True)
        (ra, ya, sa), (rb, yb, sb) = _case(moe, ctx, wl, W, rows, 0)
        for f in ("topk_ids", "topk_w", "shared_gate", "expert_count", "expert_offset", "perm"):
            a, b = getattr(ra, f), getattr(rb, f)
            if a is not None:
                assert torch.equal(a, b), f"{name} {rows}: {f} differs"
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), f"{name} {rows}: y differs"
        assert torch.equal(sa.view(torch.int16), sb.view(torch.int16)), f"{name} {rows}: residual differs"
        assert not torch.isnan(yb.float()).any()
    assert moe.moe_ctx_device_errors(ctx) == 0
    ctx.close()


def test_static_scratch_too_small_is_refused(moe):
    """512 rows at the 35B-A3B shape need about 40 MB of workspace: refused
    with MOE_ERR_WORKSPACE_TOO_SMALL, nothing written."""
    from routed_fp8_expert_amd.workload import layer_weights
    wl = syn.WORKLOADS["a3b_zipf"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    lw = layer_weights(wl, W)
    rows = 512
    assert moe.moe_workspace_bytes(lw, rows) > 16 << 20
    ctx = moe.Ctx(0)
    x = syn.make_x(wl, 0, rows, 0, "cuda")
    rt = moe.Routing(rows, wl.n_experts, wl.top_k, "cuda")
    rt.topk_ids.fill_(-7)
    y = torch.full((rows, wl.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    rc = _call(moe, ctx, lw, x, syn.make_logits_in(wl, 0, rows, "cuda"), rt, y, None)
    assert rc == moe.binding.MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and torch.all(rt.topk_ids == -7)
    assert moe.moe_ctx_status(ctx) == 0
    ctx.close()
